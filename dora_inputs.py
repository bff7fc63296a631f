"""Seeded synthetic inputs for the DoRA hot path.

Shared by the tests, the benchmark and the smoke check.  This module holds no
part of the method's arithmetic (no norm, no compose): it draws random layers
with the shapes and distributions of the workloads studied in "Scaling DoRA:
High-Rank Adaptation via Factored Norms and Fused Kernels" (d_in = 8192 and
r = 384 at the headline shape, 32B-class layer dims, KV projections with small
d_out) and computes the two branch outputs with torch matmul.  The branch GEMMs
are not under test: the same tensors are handed to the GPU path and the oracle.

Distribution notation: "N(0, 1/d_in)" for W0 is a variance (row norms near 1);
the B and magnitude-noise widths are standard deviations.  A follows torch's
kaiming_uniform_(a=sqrt(5)) on an [r, d_in] tensor, whose closed form is
U(-1/sqrt(d_in), 1/sqrt(d_in)).  m starts from the DoRA initialisation
m0 = ||W0||_row and is perturbed by a factor (1 + noise) so that g = m / wnorm
sits near 1 with a spread of order 1e-3, the regime where the pages report
g mean ~1.0, std ~0.0015.

Random streams: one torch.Generator('cpu') per layer, seeded with the layer's
seed, draws W0, A, B, the m noise, x and dy in that order, in fp32; tensors
are then rounded (round-to-nearest-even) to the layer dtype.  The many-module
sweep draws on the device with seed 5000 + 7*layer + projection.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class LayerSpec:
    name: str
    d_out: int
    d_in: int
    r: int
    T: int
    dtype: str
    s: float
    b_std: float
    m_noise: float


# The five workloads.  Key 3 is the headline shape (d_in = 8192, r = 384).
CONFIGS = {
    1: LayerSpec("tiny-fp32-64x48-r8", 64, 48, 8, 32, "f32", 16.0 / 8.0, 0.02, 0.01),
    2: LayerSpec("square-bf16-4096-r16", 4096, 4096, 16, 2048, "bf16", 2.0, 0.01, 1e-3),
    3: LayerSpec("square-bf16-8192-r384", 8192, 8192, 384, 2048, "bf16", 384.0 / 384.0, 0.005, 1e-3),
    4: LayerSpec("mlp-up-bf16-28672x8192-r384", 28672, 8192, 384, 4096, "bf16", 1.0, 0.005, 1e-3),
}

# Many-module sweep: 64 layers x 7 adapted projections (d_out, d_in), r = 384.
SWEEP_LAYERS = 64
SWEEP_PROJECTIONS = (
    ("q", 5120, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 5120),
    ("gate", 27648, 5120), ("up", 27648, 5120), ("down", 5120, 27648),
)
SWEEP_R = 384
SWEEP_T = 2048


def config_seed(cfg_id: int) -> int:
    return 1000 * cfg_id


def sweep_seed(layer: int, proj: int) -> int:
    return 5000 + 7 * layer + proj


def sweep_spec(proj: int) -> LayerSpec:
    name, d_out, d_in = SWEEP_PROJECTIONS[proj]
    return LayerSpec(f"sweep-{name}-{d_out}x{d_in}-r384", d_out, d_in, SWEEP_R, SWEEP_T, "bf16",
                     1.0, 0.005, 1e-3)


@dataclass
class Layer:
    spec: LayerSpec
    W0: torch.Tensor
    A: torch.Tensor
    B: torch.Tensor
    m: torch.Tensor            # fp32 [d_out]
    x: torch.Tensor | None = None
    dy: torch.Tensor | None = None
    base_out: torch.Tensor | None = None
    lora_out: torch.Tensor | None = None
    extra: dict = field(default_factory=dict)


def _row_norm_init(W0: torch.Tensor) -> torch.Tensor:
    # m0 = ||W0||_row (DoRA initialisation), in fp64 then fp32.
    return torch.linalg.vector_norm(W0.to(torch.float64), dim=1)


def make_layer(spec: LayerSpec, seed: int, *, device="cpu", activations=True,
               gen_device="cpu", w_scale=1.0) -> Layer:
    """Draw one adapted layer (and its activations) for `spec`.

    gen_device='cpu' gives values independent of the GPU; 'cuda' draws on the
    device (used for the many-module sweep, where host generation would be slow).
    w_scale multiplies W0 (w_scale = 0 gives the W0 = 0 edge case).
    """
    dt = DTYPES[spec.dtype]
    g = torch.Generator(device=gen_device).manual_seed(seed)
    kw = dict(generator=g, device=gen_device, dtype=torch.float32)
    W0 = torch.randn(spec.d_out, spec.d_in, **kw).mul_(w_scale / math.sqrt(spec.d_in))
    bound = 1.0 / math.sqrt(spec.d_in)
    A = torch.rand(spec.r, spec.d_in, **kw).mul_(2.0 * bound).sub_(bound)
    B = torch.randn(spec.d_out, spec.r, **kw).mul_(spec.b_std)
    noise = torch.randn(spec.d_out, **kw).mul_(spec.m_noise)
    W0, A, B = W0.to(dt), A.to(dt), B.to(dt)
    m = (_row_norm_init(W0) * (1.0 + noise.to(torch.float64))).to(torch.float32)
    layer = Layer(spec, W0.to(device), A.to(device), B.to(device), m.to(device))
    if activations:
        x = torch.randn(spec.T, spec.d_in, **kw)
        dy = torch.randn(spec.T, spec.d_out, **kw)
        layer.x = x.to(dt).to(device)
        layer.dy = dy.to(dt).to(device)
        branch_outputs(layer)
    return layer


def branch_outputs(layer: Layer) -> None:
    """base_out = x W0^T and lora_out = (x A^T) B^T (no scale s; compose applies s).

    fp32 layers are computed in fp64 and rounded once; half-precision layers use
    torch matmul in the layer dtype on the layer's device.
    """
    x, W0, A, B = layer.x, layer.W0, layer.A, layer.B
    if x.dtype == torch.float32:
        x64, W64, A64, B64 = (t.to(torch.float64) for t in (x, W0, A, B))
        layer.base_out = (x64 @ W64.T).to(torch.float32)
        layer.lora_out = ((x64 @ A64.T) @ B64.T).to(torch.float32)
    else:
        layer.base_out = torch.matmul(x, W0.T.contiguous())
        layer.lora_out = torch.matmul(torch.matmul(x, A.T.contiguous()), B.T.contiguous())


def make_config(cfg_id: int, *, device="cpu", activations=True) -> Layer:
    spec = CONFIGS[cfg_id]
    return make_layer(spec, config_seed(cfg_id), device=device, activations=activations)


def custom_spec(d_out, d_in, r, T, dtype="bf16", s=1.0, b_std=0.005, m_noise=1e-3, name=None):
    return LayerSpec(name or f"custom-{dtype}-{d_out}x{d_in}-r{r}-T{T}", d_out, d_in, r, T, dtype,
                     s, b_std, m_noise)
