"""GPU: the allocation-free norm entry point (static per-GPU scratch) against
the workspace entry point, through the C ABI.

Two calls in a row on one GPU, the second smaller than the first, each
compared bitwise with dora_factored_norm on the same inputs and against the
oracle (sampled rows, the bf16 norm tolerance), so contents the first call
left in the shared scratch cannot leak into the second.
"""
import sys

import numpy as np
import pytest
import torch

import dora_adapter_factored_amd as D
import dora_inputs as DI
import oracle
from parity_utils import NORM_RTOL, check_rel, host64, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_layer(L, seed):
    spec = L.spec
    eps = D.default_eps(L.W0.dtype)
    wn_ref, g_ref = D.factored_norm(L.W0, L.A, L.B, spec.s, L.m, eps)
    wn, g = D.factored_norm_noalloc(L.W0, L.A, L.B, spec.s, L.m, eps)
    torch.cuda.synchronize()
    assert torch.equal(wn, wn_ref), f"{spec.name}: wnorm differs from dora_factored_norm"
    assert torch.equal(g, g_ref), f"{spec.name}: g differs from dora_factored_norm"
    rows = sample_rows(spec.d_out, 256, seed=seed) if spec.d_out > 2048 else None
    ref_wn = oracle.dense_row_norm(L.W0.cpu(), L.A.cpu(), L.B.cpu(), spec.s, rows=rows)
    m = host64(L.m)
    ref_g = oracle.magnitude_scale(m if rows is None else m[rows], ref_wn, eps)
    got_wn, got_g = host64(wn), host64(g)
    if rows is not None:
        got_wn, got_g = got_wn[rows], got_g[rows]
    check_rel(got_wn, ref_wn, NORM_RTOL[L.W0.dtype], f"{spec.name} wnorm")
    check_rel(got_g, ref_g, NORM_RTOL[L.W0.dtype], f"{spec.name} g")


def test_noalloc_norm_two_calls_second_smaller():
    big = DI.make_layer(DI.CONFIGS[3], DI.config_seed(3), device=DEV, activations=False)
    small = DI.make_layer(DI.custom_spec(1000, 1536, 256, 1, dtype="bf16", s=1.0), 17, device=DEV,
                          activations=False)
    torch.cuda.synchronize()
    say(f"[no-alloc] {big.spec.name}")
    _check_layer(big, 3)
    say(f"[no-alloc] {small.spec.name}")
    _check_layer(small, 17)


def test_noalloc_norm_fp32_and_low_rank():
    for spec, seed in ((DI.CONFIGS[1], 1000), (DI.custom_spec(700, 1200, 48, 1, dtype="f32", s=0.5), 5),
                       (DI.CONFIGS[2], DI.config_seed(2))):
        say(f"[no-alloc] {spec.name}")
        L = DI.make_layer(spec, seed, device=DEV, activations=False)
        _check_layer(L, seed)
