"""GPU parity of the merge for serving, W = diag(g)(W0 + sBA), through the C
ABI against the fp64 oracle (merge_with_scale) with the error bound of
parity_utils.check_merge.  Both sides take the same fp32 g: the GPU norm's.
"""
import sys

import numpy as np
import pytest
import torch

import dora_adapter_factored_amd as D
import dora_inputs as DI
import oracle
from parity_utils import check_merge, check_rel, host64, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_g(L):
    _, g = D.factored_norm(L.W0, L.A, L.B, L.spec.s, L.m)
    torch.cuda.synchronize()
    return g


def _check_layer(L, g, W, rows=None, tag=""):
    got = host64(W) if rows is None else host64(W)[rows]
    check_merge(got, L.W0.cpu(), L.A.cpu(), L.B.cpu(), g.cpu(), L.spec.s, L.W0.dtype, rows=rows, what=tag)


MERGE_SHAPES = [
    # d_out, d_in, r, dtype, b_std
    (128, 128, 32, "bf16", 0.3),      # one tile, one k-tile
    (300, 1000, 40, "bf16", 0.3),     # ragged rows, columns and k-tiles, aligned path
    (257, 1003, 37, "bf16", 0.3),     # d_in and r not multiples of 8: element-wise path
    (64, 48, 8, "f32", 0.3),
    (200, 520, 24, "f32", 0.3),       # fp32, r not a multiple of the 16-wide k-tile
    (130, 66, 5, "f32", 0.3),         # fp32 element-wise path
    (1, 1, 1, "bf16", 1.0),
    (129, 8, 1, "bf16", 1.0),
    (520, 8200, 200, "bf16", 0.05),
    (1024, 2048, 384, "bf16", 0.005),
]


@pytest.mark.parametrize("d_out,d_in,r,dt,b_std", MERGE_SHAPES)
def test_merge_shapes(d_out, d_in, r, dt, b_std):
    say(f"[merge] {d_out}x{d_in} r={r} {dt}")
    spec = DI.custom_spec(d_out, d_in, r, 1, dtype=dt, s=1.5, b_std=b_std)
    L = DI.make_layer(spec, 900 + d_out + r, device=DEV, activations=False)
    g = gpu_g(L)
    W = D.merge(L.W0, L.A, L.B, g, spec.s)
    torch.cuda.synchronize()
    _check_layer(L, g, W, tag=f"merge {d_out}x{d_in} r{r} {dt}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_merge_config(cfg):
    L = DI.make_config(cfg, device=DEV, activations=False)
    say(f"[merge] config {cfg} ({L.spec.name})")
    g = gpu_g(L)
    W = D.merge(L.W0, L.A, L.B, g, L.spec.s)
    torch.cuda.synchronize()
    rows = None if cfg in (1, 2) else sample_rows(L.spec.d_out, 96, seed=80 + cfg)
    _check_layer(L, g, W, rows=rows, tag=f"cfg{cfg}")
    # the merged rows carry the magnitudes: ||W_i|| = m_i up to the norm's
    # tolerance and the rounding of W
    rtol = 2e-3 + 2.0 ** -8 if L.W0.dtype == torch.bfloat16 else 1e-4
    nrm = torch.linalg.vector_norm(W.double(), dim=1).cpu().numpy()
    check_rel(nrm, host64(L.m), rtol, f"cfg{cfg} row norms")


def test_merge_in_place_and_deterministic():
    say("[merge] in place, determinism")
    L = DI.make_layer(DI.custom_spec(640, 1536, 64, 1, s=2.0, b_std=0.1), 77, device=DEV, activations=False)
    g = gpu_g(L)
    W1 = D.merge(L.W0, L.A, L.B, g, 2.0)
    W2 = D.merge(L.W0, L.A, L.B, g, 2.0)
    Wi = L.W0.clone()
    out = D.merge(Wi, L.A, L.B, g, 2.0, out=Wi)
    torch.cuda.synchronize()
    assert out.data_ptr() == Wi.data_ptr()
    assert torch.equal(W1, W2) and torch.equal(Wi, W1)


def _misaligned(t):
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def test_merge_unaligned_pointers_take_the_element_path():
    say("[merge] unaligned pointers")
    L = DI.make_layer(DI.custom_spec(384, 1024, 48, 1, b_std=0.2), 78, device=DEV, activations=False)
    g = gpu_g(L)
    W_a = D.merge(L.W0, L.A, L.B, g, 1.0)
    W_u = D.merge(_misaligned(L.W0), _misaligned(L.A), _misaligned(L.B), g, 1.0, out=_misaligned(L.W0))
    torch.cuda.synchronize()
    assert torch.equal(W_a, W_u)   # same products in the same order on either path


def test_merge_identity_cases():
    say("[merge] B = 0 with g = 1; s = 0")
    L = DI.make_layer(DI.custom_spec(256, 512, 16, 1), 79, device=DEV, activations=False)
    ones = torch.ones(256, device=DEV)
    L.B.zero_()
    W = D.merge(L.W0, L.A, L.B, ones, 3.0)
    torch.cuda.synchronize()
    assert torch.equal(W, L.W0)   # the un-adapted weight, bit for bit
    L2 = DI.make_layer(DI.custom_spec(256, 512, 16, 1, b_std=0.5), 80, device=DEV, activations=False)
    g = gpu_g(L2)
    W0g = D.merge(L2.W0, L2.A, L2.B, g, 0.0)
    torch.cuda.synchronize()
    ref = (g[:, None] * L2.W0.float()).to(torch.bfloat16)   # one fp32 product, one rounding
    assert torch.equal(W0g, ref)


def test_merged_weight_serves_the_adapted_layer():
    # x W^T with the merged weight against the oracle's compose of the two
    # branch outputs: the same layer in weight space and in activation space
    say("[merge] merged layer output vs the compose of the branches")
    L = DI.make_layer(DI.custom_spec(512, 768, 32, 64, s=1.0, b_std=0.05), 81, device=DEV)
    g = gpu_g(L)
    W = D.merge(L.W0, L.A, L.B, g, 1.0)
    torch.cuda.synchronize()
    x64 = host64(L.x)
    y_merged = x64 @ host64(W).T
    y_ref = oracle.compose_forward(x64 @ host64(L.W0).T, (x64 @ host64(L.A).T) @ host64(L.B).T, host64(g), 1.0)
    scale = np.abs(x64) @ np.abs(host64(W)).T
    assert np.all(np.abs(y_merged - y_ref) <= 2.0 ** -8 * scale + 1e-6)


@pytest.mark.parametrize("r", [8, 16, 32])
def test_merge_low_rank_stages_A_directly(r):
    # bf16 with r <= 32: the tile kernel builds its A^T stage from A itself.
    # An A that is not 16-byte aligned goes through the transpose instead;
    # the products and their order are the same, so W is bitwise equal.
    say(f"[merge] low rank r={r}: A staged directly vs transposed")
    L = DI.make_layer(DI.custom_spec(320, 1032, r, 1, s=1.5, b_std=0.1), 82 + r, device=DEV, activations=False)
    g = gpu_g(L)
    W_direct = D.merge(L.W0, L.A, L.B, g, 1.5)
    W_transposed = D.merge(L.W0, _misaligned(L.A), L.B, g, 1.5)
    torch.cuda.synchronize()
    assert torch.equal(W_direct, W_transposed)
    _check_layer(L, g, W_direct, tag=f"direct r{r}")


@pytest.mark.parametrize("d_out,d_in,r", [(4096, 4096, 384), (3900, 3952, 104), (2048, 8192, 200), (4096, 4096, 64)])
def test_merge_large_tiles(d_out, d_in, r):
    # bf16, aligned, r > 32 and 200-256 tiles of 256 x 256: the large-tile
    # kernel (8 waves of 128 x 64, four 64-row epilogue rounds); ragged rows,
    # columns and k-tiles in the second shape.  Sampled rows, then in place.
    say(f"[merge] large tiles {d_out}x{d_in} r={r}")
    spec = DI.custom_spec(d_out, d_in, r, 1, dtype="bf16", s=1.5, b_std=0.05)
    L = DI.make_layer(spec, 950 + r, device=DEV, activations=False, gen_device="cuda")
    g = gpu_g(L)
    W = D.merge(L.W0, L.A, L.B, g, spec.s)
    torch.cuda.synchronize()
    rows = sample_rows(d_out, 96, seed=r)
    rows = np.unique(np.concatenate([rows, np.arange(d_out - 40, d_out)]))   # the ragged last row tile
    _check_layer(L, g, W, rows=rows, tag=f"large tiles {d_out}x{d_in} r{r}")
    Wi = L.W0.clone()
    D.merge(Wi, L.A, L.B, g, spec.s, out=Wi)
    torch.cuda.synchronize()
    assert torch.equal(Wi, W)
