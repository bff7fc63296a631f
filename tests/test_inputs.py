"""The seeded input generator: determinism and the distributions it promises."""
import math

import numpy as np
import torch

import dora_inputs as DI
import oracle


def test_seeded_and_deterministic():
    spec = DI.custom_spec(48, 40, 6, 5, dtype="bf16")
    a = DI.make_layer(spec, 123)
    b = DI.make_layer(spec, 123)
    c = DI.make_layer(spec, 124)
    for name in ("W0", "A", "B", "m", "x", "dy", "base_out", "lora_out"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert not torch.equal(a.W0, c.W0)


def test_distributions_match_recipe():
    spec = DI.custom_spec(512, 1024, 32, 4, dtype="f32", b_std=0.005, m_noise=1e-3)
    L = DI.make_layer(spec, 7)
    rn = torch.linalg.vector_norm(L.W0.double(), dim=1)
    assert abs(rn.mean().item() - 1.0) < 0.01            # variance 1/d_in -> row norm ~ 1
    bound = 1.0 / math.sqrt(1024)
    assert L.A.abs().max().item() <= bound                # kaiming-uniform(a=sqrt(5)) bound
    assert abs(L.A.double().std().item() - bound / math.sqrt(3)) < 0.01 * bound
    assert abs(L.B.double().std().item() - 0.005) < 2e-4
    # g = m / wnorm concentrates near 1 with spread ~1e-3 (the near-unity regime)
    wn = oracle.dense_row_norm(L.W0, L.A, L.B, spec.s)
    g = oracle.as_f64(L.m) / wn
    assert abs(g.mean() - 1.0) < 5e-3 and 5e-4 < g.std() < 5e-3


def test_config_shapes():
    for k, spec in DI.CONFIGS.items():
        assert spec.dtype in DI.DTYPES
    assert DI.CONFIGS[3].d_in == 8192 and DI.CONFIGS[3].r == 384
    L = DI.make_config(1)
    assert L.W0.shape == (64, 48) and L.A.shape == (8, 48) and L.B.shape == (64, 8)
    assert L.base_out.shape == (32, 64) and L.lora_out.shape == (32, 64) and L.dy.shape == (32, 64)
    assert L.W0.dtype == torch.float32 and L.m.dtype == torch.float32
    assert len(DI.SWEEP_PROJECTIONS) == 7
