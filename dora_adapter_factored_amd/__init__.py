"""MI355X (gfx950) DoRA hot path: factored row norm and fused compose.

The computation lives in the HIP library libdora_mi355x.so (C ABI declared in
include/dora.h); this package holds its sources (csrc/), the build step and a
thin ctypes binding.  Importing the package does not load the library; the
first call does, and raises ImportError if it has not been built.
"""
from .binding import (  # noqa: F401
    DoraError,
    DoRACompose,
    DoRAComposeInner,
    EXPORTED,
    compose,
    compose_backward,
    compose_backward_inner,
    compose_dual,
    compose_backward_workspace_size,
    default_eps,
    factored_norm,
    factored_norm_group,
    factored_norm_noalloc,
    library_path,
    load,
    merge,
    merge_workspace_size,
    norm_group_workspace_size,
    norm_workspace_size,
)
