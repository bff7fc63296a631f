"""The C-ABI library: it loads, exports every symbol include/dora.h declares, and
rejects bad arguments on the host before any launch (no GPU needed: every
call here returns from validation, so no device memory is touched)."""
import ctypes
import os
import re

import pytest
import torch

import dora_adapter_factored_amd as D
from dora_adapter_factored_amd import binding as Bn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dora.h")
FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
FAKE_WS = ctypes.c_void_p(0x100000)   # 256-byte aligned


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(dora_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    return D.load()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(D.EXPORTED)


def test_member_struct_layout_matches_the_header(tmp_path):
    # the binding's ctypes copy of DoraNormMember against the C compiler's
    # layout of the header's struct
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in Bn.NormMember._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "dora.h"\nint main(void) {\n'
                   '    printf("%zu", sizeof(DoraNormMember));\n'
                   + "".join(f'    printf(" %zu", offsetof(DoraNormMember, {f}));\n' for f in fields)
                   + "    return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(Bn.NormMember)] + [getattr(Bn.NormMember, f).offset for f in fields]
    assert got == want


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.dora_status_string(0) == b"ok"
    assert lib.dora_status_string(3).startswith(b"workspace")
    assert lib.dora_status_string(99) == b"unknown status"
    assert lib.dora_version() >= 100


def test_workspace_queries(lib):
    n = ctypes.c_size_t()
    assert lib.dora_factored_norm_workspace_size(8192, 8192, 384, 1, ctypes.byref(n)) == 0
    # O(d_out r + r^2)-sized: far below the dense [d_out, d_in] product (128 MiB in bf16)
    assert 0 < n.value < 16 << 20
    assert lib.dora_factored_norm_workspace_size(64, 48, 8, 0, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.dora_factored_norm_workspace_size(0, 48, 8, 0, ctypes.byref(n)) == Bn.DORA_ERR_INVALID_ARG
    assert lib.dora_factored_norm_workspace_size(64, 48, 8, 7, ctypes.byref(n)) == Bn.DORA_ERR_INVALID_ARG
    assert lib.dora_factored_norm_workspace_size(64, 48, 8, 2, ctypes.byref(n)) == Bn.DORA_ERR_UNSUPPORTED
    assert lib.dora_factored_norm_workspace_size(64, 48, 8, 1, None) == Bn.DORA_ERR_INVALID_ARG
    # d_m partial rows: one per token block (16 rows for d_out > 4096, else
    # 32), at most 1024 rows, fp32
    assert lib.dora_compose_backward_workspace_size(2048, 8192, ctypes.byref(n)) == 0
    assert n.value == 128 * 8192 * 4
    assert lib.dora_compose_backward_workspace_size(2048, 4096, ctypes.byref(n)) == 0
    assert n.value == 64 * 4096 * 4
    assert lib.dora_compose_backward_workspace_size(1 << 20, 8192, ctypes.byref(n)) == 0
    assert n.value == 1024 * 8192 * 4
    assert lib.dora_compose_backward_workspace_size(0, 8192, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.dora_compose_backward_workspace_size(-1, 8192, ctypes.byref(n)) == Bn.DORA_ERR_INVALID_ARG


def test_norm_transient_against_the_dense_product(lib):
    # The pages' accounting: the factored norm needs O(d r + r^2) scratch where
    # the dense route materialises d x d; at d = 8192, r = 512 the ratio of the
    # element counts is d^2 / (d r + r^2) = 15.06.
    d, r = 8192, 512
    assert round(d * d / (d * r + r * r), 2) == 15.06
    # this library's scratch (fp32 split partials included) stays an order of
    # magnitude below the bf16 dense product: 24x at r = 384, 13.8x at r = 512
    n = ctypes.c_size_t()
    for rr in (384, 512):
        assert lib.dora_factored_norm_workspace_size(d, d, rr, 1, ctypes.byref(n)) == 0
        dense_bytes = d * d * 2
        assert n.value * 10 < dense_bytes, (rr, n.value)


def _norm(lib, **kw):
    a = dict(W0=FAKE, A=FAKE, B=FAKE, m=FAKE, d_out=64, d_in=48, r=8, dtype=1, s=1.0, eps=1e-6,
             wnorm=FAKE, g=FAKE, ws=FAKE_WS, nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.dora_factored_norm(a["W0"], a["A"], a["B"], a["m"], a["d_out"], a["d_in"], a["r"], a["dtype"],
                                  a["s"], a["eps"], a["wnorm"], a["g"], a["ws"], a["nbytes"], a["stream"])


def test_norm_validation(lib):
    E = Bn
    assert _norm(lib, W0=None) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, A=None) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, B=None) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, wnorm=None) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, g=None) == E.DORA_ERR_INVALID_ARG          # m given without g
    assert _norm(lib, d_out=0) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, d_in=-3) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, r=1 << 31) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, dtype=5) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, dtype=2) == E.DORA_ERR_UNSUPPORTED
    assert _norm(lib, s=float("nan")) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, eps=-1.0) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, eps=float("inf")) == E.DORA_ERR_INVALID_ARG
    assert _norm(lib, ws=None) == E.DORA_ERR_WORKSPACE
    assert _norm(lib, nbytes=16) == E.DORA_ERR_WORKSPACE
    assert _norm(lib, ws=ctypes.c_void_p(0x100010)) == E.DORA_ERR_WORKSPACE   # misaligned
    assert b"256-byte" in lib.dora_last_error_detail()


def _norm_noalloc(lib, **kw):
    a = dict(W0=FAKE, A=FAKE, B=FAKE, m=FAKE, d_out=8, d_in=16, r=4, dtype=1, s=1.0, eps=1e-6,
             wnorm=FAKE, g=FAKE, stream=None)
    a.update(kw)
    return lib.dora_factored_norm_noalloc(a["W0"], a["A"], a["B"], a["m"], a["d_out"], a["d_in"], a["r"],
                                          a["dtype"], a["s"], a["eps"], a["wnorm"], a["g"], a["stream"])


def test_norm_noalloc_validation(lib):
    """Same argument checks as dora_factored_norm; sizes whose workspace is
    larger than the static scratch are refused before any device call."""
    E = Bn
    assert _norm_noalloc(lib, W0=None) == E.DORA_ERR_INVALID_ARG
    assert _norm_noalloc(lib, wnorm=None) == E.DORA_ERR_INVALID_ARG
    assert _norm_noalloc(lib, g=None) == E.DORA_ERR_INVALID_ARG
    assert _norm_noalloc(lib, d_out=0) == E.DORA_ERR_INVALID_ARG
    assert _norm_noalloc(lib, dtype=2) == E.DORA_ERR_UNSUPPORTED
    assert _norm_noalloc(lib, eps=-1.0) == E.DORA_ERR_INVALID_ARG
    limit = 16 << 20
    big = dict(d_out=8192, d_in=16384, r=1024)
    assert D.norm_workspace_size(big["d_out"], big["d_in"], big["r"], torch.bfloat16) > limit
    assert _norm_noalloc(lib, **big) == E.DORA_ERR_WORKSPACE
    assert b"static scratch" in lib.dora_last_error_detail()
    # every workload of the pages' shapes fits the scratch
    for d_out, d_in, r in ((8192, 8192, 384), (28672, 8192, 384), (27648, 5120, 384), (5120, 27648, 384),
                           (32768, 32768, 512)):
        for dt in (torch.bfloat16, torch.float32):
            assert D.norm_workspace_size(d_out, d_in, r, dt) <= limit


def test_noalloc_scratch_size_matches_the_header():
    src = open(HEADER).read()
    m = re.search(r"#define DORA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == 16 << 20


def _compose(lib, **kw):
    a = dict(base=FAKE, lora=ctypes.c_void_p(0x20000), g=FAKE, s=1.0, T=4, d_out=8, dtype=1, delta=0,
             y=ctypes.c_void_p(0x30000), stream=None)
    a.update(kw)
    return lib.dora_compose(a["base"], a["lora"], a["g"], a["s"], a["T"], a["d_out"], a["dtype"], a["delta"],
                            a["y"], a["stream"])


def test_compose_validation(lib):
    E = Bn
    assert _compose(lib, base=None) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, lora=None) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, g=None) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, y=None) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, T=-1) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, d_out=0) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, dtype=3) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, delta=2) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, s=float("inf")) == E.DORA_ERR_INVALID_ARG
    assert _compose(lib, y=ctypes.c_void_p(0x20000)) == E.DORA_ERR_INVALID_ARG   # y aliases lora_out
    # T == 0 is a no-op with NULL activations and launches nothing
    assert _compose(lib, T=0, base=None, lora=None, y=None) == E.DORA_OK


def _bwd(lib, **kw):
    a = dict(dy=FAKE, base=FAKE, lora=FAKE, g=FAKE, wnorm=FAKE, s=1.0, eps=1e-6, T=64, d_out=8, dtype=1,
             delta=0, db=ctypes.c_void_p(0x40000), dl=ctypes.c_void_p(0x50000), dm=FAKE, ws=FAKE_WS,
             nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.dora_compose_backward(a["dy"], a["base"], a["lora"], a["g"], a["wnorm"], a["s"], a["eps"], a["T"],
                                     a["d_out"], a["dtype"], a["delta"], a["db"], a["dl"], a["dm"], a["ws"],
                                     a["nbytes"], a["stream"])


def test_compose_backward_validation(lib):
    E = Bn
    assert _bwd(lib, dy=None) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, g=None) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, base=None) == E.DORA_ERR_INVALID_ARG        # d_m requested
    assert _bwd(lib, lora=None) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, wnorm=None) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, T=-5) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, d_out=1 << 31) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, dtype=-1) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, delta=7) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, eps=-0.5) == E.DORA_ERR_INVALID_ARG
    assert _bwd(lib, dl=ctypes.c_void_p(0x40000)) == E.DORA_ERR_INVALID_ARG   # d_base == d_lora
    assert _bwd(lib, ws=None) == E.DORA_ERR_WORKSPACE
    assert _bwd(lib, nbytes=4) == E.DORA_ERR_WORKSPACE
    assert _bwd(lib, ws=ctypes.c_void_p(0x100004)) == E.DORA_ERR_WORKSPACE


def _dual(lib, **kw):
    a = dict(base=FAKE, lora=ctypes.c_void_p(0x20000), g=FAKE, s=1.0, T=4, d_out=8, dtype=1, delta=0,
             y=ctypes.c_void_p(0x30000), inner=ctypes.c_void_p(0x60000), stream=None)
    a.update(kw)
    return lib.dora_compose_dual(a["base"], a["lora"], a["g"], a["s"], a["T"], a["d_out"], a["dtype"], a["delta"],
                                 a["y"], a["inner"], a["stream"])


def test_compose_dual_validation(lib):
    E = Bn
    assert _dual(lib, base=None) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, lora=None) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, g=None) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, y=None) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, inner=None) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, T=-1) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, d_out=0) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, dtype=3) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, delta=2) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, s=float("nan")) == E.DORA_ERR_INVALID_ARG
    assert _dual(lib, y=ctypes.c_void_p(0x20000)) == E.DORA_ERR_INVALID_ARG       # y aliases lora_out
    assert _dual(lib, inner=FAKE) == E.DORA_ERR_INVALID_ARG                       # inner aliases base_out
    assert _dual(lib, inner=ctypes.c_void_p(0x30000)) == E.DORA_ERR_INVALID_ARG   # y == inner
    assert _dual(lib, T=0, base=None, lora=None, y=None, inner=None) == E.DORA_OK


def _bwd_inner(lib, **kw):
    a = dict(dy=FAKE, inner=ctypes.c_void_p(0x70000), g=FAKE, wnorm=FAKE, s=1.0, eps=1e-6, T=64, d_out=8,
             dtype=1, delta=0, db=ctypes.c_void_p(0x40000), dl=ctypes.c_void_p(0x50000), dm=FAKE, ws=FAKE_WS,
             nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.dora_compose_backward_inner(a["dy"], a["inner"], a["g"], a["wnorm"], a["s"], a["eps"], a["T"],
                                           a["d_out"], a["dtype"], a["delta"], a["db"], a["dl"], a["dm"], a["ws"],
                                           a["nbytes"], a["stream"])


def test_compose_backward_inner_validation(lib):
    E = Bn
    assert _bwd_inner(lib, dy=None) == E.DORA_ERR_INVALID_ARG
    assert _bwd_inner(lib, g=None) == E.DORA_ERR_INVALID_ARG
    assert _bwd_inner(lib, inner=None) == E.DORA_ERR_INVALID_ARG       # d_m requested
    assert _bwd_inner(lib, wnorm=None) == E.DORA_ERR_INVALID_ARG
    assert _bwd_inner(lib, T=-5) == E.DORA_ERR_INVALID_ARG
    assert _bwd_inner(lib, dtype=9) == E.DORA_ERR_INVALID_ARG
    assert _bwd_inner(lib, delta=3) == E.DORA_ERR_INVALID_ARG
    assert _bwd_inner(lib, eps=float("nan")) == E.DORA_ERR_INVALID_ARG
    assert _bwd_inner(lib, dl=ctypes.c_void_p(0x40000)) == E.DORA_ERR_INVALID_ARG   # d_base == d_lora
    assert _bwd_inner(lib, db=ctypes.c_void_p(0x70000)) == E.DORA_ERR_INVALID_ARG   # d_base aliases inner
    assert _bwd_inner(lib, ws=None) == E.DORA_ERR_WORKSPACE
    assert _bwd_inner(lib, nbytes=8) == E.DORA_ERR_WORKSPACE
    assert _bwd_inner(lib, ws=ctypes.c_void_p(0x100008)) == E.DORA_ERR_WORKSPACE


def test_merge_workspace_size(lib):
    n = ctypes.c_size_t()
    # A transposed: d_in padded to whole 256-row tiles, r to whole 64-byte k-tiles
    assert lib.dora_merge_workspace_size(8192, 384, 1, ctypes.byref(n)) == 0 and n.value == 8192 * 384 * 2
    assert lib.dora_merge_workspace_size(1000, 40, 1, ctypes.byref(n)) == 0 and n.value == 1024 * 64 * 2
    assert lib.dora_merge_workspace_size(3, 5, 1, ctypes.byref(n)) == 0 and n.value == 256 * 32 * 2
    assert lib.dora_merge_workspace_size(100, 40, 0, ctypes.byref(n)) == 0 and n.value == 256 * 48 * 4
    assert lib.dora_merge_workspace_size(100, 40, 2, ctypes.byref(n)) == Bn.DORA_ERR_UNSUPPORTED
    assert lib.dora_merge_workspace_size(0, 40, 1, ctypes.byref(n)) == Bn.DORA_ERR_INVALID_ARG
    assert lib.dora_merge_workspace_size(10, 1 << 23, 1, ctypes.byref(n)) == Bn.DORA_ERR_INVALID_ARG
    assert lib.dora_merge_workspace_size(10, 4, 1, None) == Bn.DORA_ERR_INVALID_ARG


def _merge(lib, **kw):
    a = dict(W0=FAKE, A=ctypes.c_void_p(0x20000), B=ctypes.c_void_p(0x30000), g=ctypes.c_void_p(0x40000), s=1.0,
             d_out=64, d_in=48, r=8, dtype=1, W=ctypes.c_void_p(0x50000), ws=FAKE_WS, nbytes=1 << 30, stream=None)
    a.update(kw)
    return lib.dora_merge(a["W0"], a["A"], a["B"], a["g"], a["s"], a["d_out"], a["d_in"], a["r"], a["dtype"],
                          a["W"], a["ws"], a["nbytes"], a["stream"])


def test_merge_validation(lib):
    E = Bn
    for k in ("W0", "A", "B", "g", "W"):
        assert _merge(lib, **{k: None}) == E.DORA_ERR_INVALID_ARG, k
    assert _merge(lib, d_out=0) == E.DORA_ERR_INVALID_ARG
    assert _merge(lib, d_in=-1) == E.DORA_ERR_INVALID_ARG
    assert _merge(lib, r=0) == E.DORA_ERR_INVALID_ARG
    assert _merge(lib, r=1 << 23) == E.DORA_ERR_INVALID_ARG
    assert _merge(lib, d_out=1 << 30, d_in=1 << 30) == E.DORA_ERR_INVALID_ARG   # tile count
    assert _merge(lib, dtype=4) == E.DORA_ERR_INVALID_ARG
    assert _merge(lib, dtype=2) == E.DORA_ERR_UNSUPPORTED
    assert _merge(lib, s=float("nan")) == E.DORA_ERR_INVALID_ARG
    assert _merge(lib, W=ctypes.c_void_p(0x20000)) == E.DORA_ERR_INVALID_ARG    # W aliases A
    assert _merge(lib, W=ctypes.c_void_p(0x30000)) == E.DORA_ERR_INVALID_ARG    # W aliases B
    assert _merge(lib, W=ctypes.c_void_p(0x40000)) == E.DORA_ERR_INVALID_ARG    # W aliases g
    assert _merge(lib, W=FAKE_WS) == E.DORA_ERR_INVALID_ARG                     # W is the workspace
    assert _merge(lib, ws=None) == E.DORA_ERR_WORKSPACE
    assert _merge(lib, nbytes=100) == E.DORA_ERR_WORKSPACE
    assert _merge(lib, ws=ctypes.c_void_p(0x100040)) == E.DORA_ERR_WORKSPACE
    assert b"256-byte" in lib.dora_last_error_detail()


def test_norm_group_workspace_size(lib):
    n = ctypes.c_size_t()
    sizes = ((5120, 5120), (1024, 5120), (5120, 27648))   # members may differ in d_in
    d = (ctypes.c_int64 * 3)(*[o for o, _ in sizes])
    k = (ctypes.c_int64 * 3)(*[i for _, i in sizes])
    assert lib.dora_factored_norm_group_workspace_size(3, d, k, 384, 1, ctypes.byref(n)) == 0
    total = 0
    for d_out, d_in in sizes:   # each member's own region, 256-byte aligned
        one = ctypes.c_size_t()
        assert lib.dora_factored_norm_workspace_size(d_out, d_in, 384, 1, ctypes.byref(one)) == 0
        total += (one.value + 255) // 256 * 256
    assert n.value == total
    E = Bn
    assert lib.dora_factored_norm_group_workspace_size(0, d, k, 384, 1, ctypes.byref(n)) == E.DORA_ERR_INVALID_ARG
    assert lib.dora_factored_norm_group_workspace_size(9, d, k, 384, 1, ctypes.byref(n)) == E.DORA_ERR_INVALID_ARG
    assert lib.dora_factored_norm_group_workspace_size(3, None, k, 384, 1, ctypes.byref(n)) == E.DORA_ERR_INVALID_ARG
    assert lib.dora_factored_norm_group_workspace_size(3, d, None, 384, 1, ctypes.byref(n)) == E.DORA_ERR_INVALID_ARG
    assert lib.dora_factored_norm_group_workspace_size(3, d, k, 0, 1, ctypes.byref(n)) == E.DORA_ERR_INVALID_ARG
    assert lib.dora_factored_norm_group_workspace_size(3, d, k, 384, 2, ctypes.byref(n)) == E.DORA_ERR_UNSUPPORTED
    bad = (ctypes.c_int64 * 2)(64, 0)
    ok_in = (ctypes.c_int64 * 2)(48, 48)
    assert lib.dora_factored_norm_group_workspace_size(2, bad, ok_in, 8, 1, ctypes.byref(n)) == E.DORA_ERR_INVALID_ARG
    bad_in = (ctypes.c_int64 * 2)(48, 0)
    assert lib.dora_factored_norm_group_workspace_size(2, (ctypes.c_int64 * 2)(64, 64), bad_in, 8, 1,
                                                       ctypes.byref(n)) == E.DORA_ERR_INVALID_ARG


def _group(lib, members=None, **kw):
    if members is None:
        members = [dict()]
    arr = (Bn.NormMember * max(1, len(members)))()
    for j, over in enumerate(members):
        mb = dict(W0=0x10000, A=0x20000, B=0x30000, m=0x40000, wnorm=0x50000 + 0x1000 * j, g=0x60000 + 0x1000 * j,
                  d_out=64, d_in=48, s=1.0)
        mb.update(over)
        arr[j] = Bn.NormMember(mb["W0"], mb["A"], mb["B"], mb["m"], mb["wnorm"], mb["g"], mb["d_out"], mb["d_in"],
                               mb["s"])
    a = dict(n=len(members), arr=arr, r=8, dtype=1, eps=1e-6, ws=FAKE_WS, nbytes=1 << 30)
    a.update(kw)
    return lib.dora_factored_norm_group(a["n"], a["arr"], a["r"], a["dtype"], a["eps"], a["ws"], a["nbytes"], None)


def test_norm_group_validation(lib):
    E = Bn
    assert _group(lib, arr=None) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, n=0) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, [dict()] * 9) == E.DORA_ERR_INVALID_ARG
    for k in ("W0", "A", "B", "wnorm"):
        assert _group(lib, [dict(), {k: None}]) == E.DORA_ERR_INVALID_ARG, k
    assert _group(lib, [dict(g=None)]) == E.DORA_ERR_INVALID_ARG            # m given without g
    assert _group(lib, [dict(), dict(d_out=0)]) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, [dict(s=float("nan"))]) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, [dict(), dict(d_in=0)]) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, r=0) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, dtype=2) == E.DORA_ERR_UNSUPPORTED
    assert _group(lib, dtype=7) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, eps=-1.0) == E.DORA_ERR_INVALID_ARG
    assert _group(lib, ws=None) == E.DORA_ERR_WORKSPACE
    assert _group(lib, nbytes=8) == E.DORA_ERR_WORKSPACE
    assert _group(lib, ws=ctypes.c_void_p(0x100080)) == E.DORA_ERR_WORKSPACE


def test_binding_rejects_bad_tensors_before_the_library():
    # host tensors are refused by the shape/device checks of the binding
    cpu = torch.zeros(4, 8, dtype=torch.bfloat16)
    g = torch.ones(8)
    with pytest.raises(ValueError):
        D.compose(cpu, torch.zeros(4, 9, dtype=torch.bfloat16), g, 1.0)
    with pytest.raises(ValueError):
        D.compose(cpu, cpu.t(), g, 1.0)
    with pytest.raises(ValueError):
        D.factored_norm(cpu, torch.zeros(2, 8, dtype=torch.float32), torch.zeros(4, 2, dtype=torch.bfloat16), 1.0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(Bn, "_lib", None)
    monkeypatch.setattr(Bn, "_LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        Bn.load()
