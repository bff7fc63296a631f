"""Helpers shared by the GPU parity tests: tolerance checks and oracle calls on
host copies of the very tensors the GPU path consumed."""
import numpy as np
import torch

import oracle

# Tolerances of the workloads' acceptance bar: norms relative 1e-4 with fp32 inputs, 2e-3 with
# bf16 inputs; bf16 compose outputs and grads |err| <= 2^-7 |ref| + 1e-3;
# fp32 compose max-abs 1e-4.
NORM_RTOL = {torch.float32: 1e-4, torch.bfloat16: 2e-3}
BF16_REL, BF16_ABS = 2.0 ** -7, 1e-3
F32_ABS = 1e-4


def host64(t):
    return oracle.as_f64(t.detach().cpu())


def check_rel(got, ref, rtol, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bad = err > rtol * np.abs(ref)
    if bad.any():
        i = int(np.argmax(err / np.maximum(np.abs(ref), 1e-300)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} exceed rel {rtol}; worst at {i}: "
                             f"got {got.flat[i]!r} ref {ref.flat[i]!r}")


def check_act(got, ref, dtype, what):
    """Activation-shaped outputs (compose y / grads, d_m)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    if dtype == torch.float32:
        bound = np.full_like(ref, F32_ABS)
    else:
        bound = BF16_REL * np.abs(ref) + BF16_ABS
    bad = ~(err <= bound)
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; worst at {i}: "
                             f"got {got.flat[i]!r} ref {ref.flat[i]!r} bound {bound.flat[i]!r}")


def sample_rows(n, k, seed=0):
    """Deterministic sample of k row indices of n, always including both ends
    and the first rows of each 128-row tile boundary region."""
    rng = np.random.default_rng(seed)
    fixed = {i for i in (0, 1, n - 1, n // 2) if i < n}
    fixed |= {min(n - 1, b) for b in range(127, n, 128 * 7)}
    extra = rng.choice(n, size=min(n, k), replace=False)
    return np.array(sorted(fixed | set(extra.tolist())), dtype=np.int64)


def check_merge(got, W0, A, B, g, s, dtype, rows=None, what="W"):
    """Merged weight against the oracle with an error bound derived from the
    kernel's arithmetic.  With u = 2^-24:
      - B A accumulated in fp32 over r products (in any order, rounding to
        nearest or toward zero): |err| <= 2 gamma_r sum_k |B_ik||A_kj|,
        gamma_r = r u / (1 - r u), times |g s|;
      - fmaf(s, acc, W0) and the product with g: |ref| 4u;
      - the final rounding to dtype: |ref| 2^-8 (bf16: 8-bit significand) or
        u (fp32).
    """
    if rows is not None:
        idx = torch.as_tensor(np.asarray(rows, dtype=np.int64))
        W0, B, g = W0[idx], B[idx], g[idx]
    W0, A, B, g = (oracle.as_f64(x) for x in (W0, A, B, g))
    got = np.asarray(got, np.float64)
    ref = oracle.merge_with_scale(W0, A, B, g, s)
    r = A.shape[0]
    u = 2.0 ** -24
    gamma = r * u / (1 - r * u)
    u_out = 2.0 ** -8 if dtype == torch.bfloat16 else u
    bound = (u_out + 4 * u) * np.abs(ref) + 2 * gamma * np.abs(g * s)[:, None] * (np.abs(B) @ np.abs(A))
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of bound; worst at {i}: "
                             f"got {got.flat[i]!r} ref {ref.flat[i]!r} bound {bound.flat[i]!r}")
