"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Inputs come from dora_inputs (seeded, synthetic); the oracle sees exact host
copies of the tensors the GPU consumed.  Small cases are compared element by
element; the full-size workloads (the bench's launch configuration) on
sampled rows / columns the oracle computes one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

import dora_adapter_factored_amd as D
import dora_inputs as DI
import oracle
from parity_utils import NORM_RTOL, check_act, check_rel, host64, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


_layers = {}


def config_layer(cfg):
    if cfg not in _layers:
        say(f"[parity] generating config {cfg} ({DI.CONFIGS[cfg].name})")
        _layers[cfg] = DI.make_config(cfg, device=DEV)
        torch.cuda.synchronize()
    return _layers[cfg]


def gpu_norm(L, s=None, m=True, eps=None):
    s = L.spec.s if s is None else s
    wn, g = D.factored_norm(L.W0, L.A, L.B, s, L.m if m else None, eps)
    torch.cuda.synchronize()
    return wn, g


def oracle_norm(L, rows=None, s=None, eps=None):
    s = L.spec.s if s is None else s
    eps = D.default_eps(L.W0.dtype) if eps is None else eps
    W0, A, B = L.W0.cpu(), L.A.cpu(), L.B.cpu()
    wn = oracle.dense_row_norm(W0, A, B, s, rows=rows)
    m = host64(L.m)
    g = oracle.magnitude_scale(m if rows is None else m[rows], wn, eps)
    return wn, g


# ------------------------------------------------------------------ norm
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_norm_config(cfg):
    L = config_layer(cfg)
    say(f"[parity] norm config {cfg}")
    wn, g = gpu_norm(L)
    rows = None if L.spec.d_out <= 4096 else sample_rows(L.spec.d_out, 384, seed=cfg)
    ref_wn, ref_g = oracle_norm(L, rows)
    got_wn, got_g = host64(wn), host64(g)
    if rows is not None:
        got_wn, got_g = got_wn[rows], got_g[rows]
        assert np.all(np.isfinite(host64(wn))) and np.all(host64(wn) > 0)
    rtol = NORM_RTOL[L.W0.dtype]
    check_rel(got_wn, ref_wn, rtol, f"cfg{cfg} wnorm")
    check_rel(got_g, ref_g, rtol, f"cfg{cfg} g")


EDGE_SHAPES = [
    # d_out, d_in, r, dtype
    (1000, 777, 13, "bf16"),     # nothing aligned: element-wise loads, ragged tiles
    (1000, 777, 13, "f32"),
    (1, 64, 1, "bf16"),          # single row, rank 1
    (130, 40, 100, "bf16"),      # r > d_in, d_in below one K tile
    (257, 512, 512, "bf16"),     # two slices of r
    (200, 264, 777, "bf16"),     # three slices, ragged last slice
    (96, 1032, 16, "bf16"),      # narrow-r tile
    (300, 136, 384, "f32"),      # fp32 with two slices of r
    (129, 256, 32, "bf16"), (129, 256, 64, "bf16"), (129, 256, 192, "bf16"), (129, 256, 384, "bf16"),
    (64, 48, 8, "f32"), (64, 48, 8, "bf16"),
    (300, 1000, 384, "bf16"),    # 256-row tiles: ragged rows, K tail inside a 32-wide tile
    (520, 8200, 200, "bf16"),    # 256-row tiles with r < 384 (ragged slice of r)
    (1000, 4104, 136, "bf16"),   # 256-row tiles from r = 129 (most of the 384 columns zero)
    (300, 2056, 128, "bf16"),    # the largest r of the 128-row tiles
    # r <= 32 bf16: the W0 pass forms each K-chunk's Gram term itself
    (520, 8200, 24, "bf16"),     # eight ragged K-chunks, r below the 32-wide tile
    (300, 4104, 8, "bf16"),      # rank 8 in a 16-wide tile, ragged rows
    # 32 < r <= 64 bf16: the wide 64-column tile, Gram blocks split over its waves
    (300, 4104, 48, "bf16"),     # ragged rows and K-chunks, three of four A blocks live
    (1000, 8200, 64, "bf16"),    # every A block live, many K-chunks
    (4096, 1000, 33, "bf16"),    # one live column in the last A block
    (77, 64, 40, "bf16"),        # a single k-tile
]


@pytest.mark.parametrize("d_out,d_in,r,dt", EDGE_SHAPES)
def test_norm_edge_shapes(d_out, d_in, r, dt):
    say(f"[parity] norm edge {d_out}x{d_in} r={r} {dt}")
    spec = DI.custom_spec(d_out, d_in, r, 1, dtype=dt, s=1.5, b_std=0.05)
    L = DI.make_layer(spec, 17 + d_out + r, device=DEV, activations=False)
    wn, g = gpu_norm(L)
    ref_wn, ref_g = oracle_norm(L)
    check_rel(host64(wn), ref_wn, NORM_RTOL[L.W0.dtype], "wnorm")
    check_rel(host64(g), ref_g, NORM_RTOL[L.W0.dtype], "g")


@pytest.mark.parametrize("d_out,d_in,r", [(4096, 8192, 16), (4090, 2056, 24), (4111, 2056, 24), (4100, 8200, 16),
                                          (8192, 4104, 24), (1024, 16384, 16)])
def test_norm_low_rank_forms_at_scale(d_out, d_in, r):
    # bf16 r <= 32: when the 16-row workgroups make one round (4081 to 4096
    # rows) and W0 has at most 2^25 elements (4096 x 8192; 4090 x 2056 with a
    # ragged last workgroup and a K tail) one whole-row kernel assembles wnorm
    # and g; otherwise (4111 rows, beyond 2^25, below 4081 rows) the K-split W0
    # pass (each K-chunk's Gram term formed in the pass) and the assembly
    # kernel run.  Sampled rows.
    say(f"[parity] low-rank norm {d_out}x{d_in} r={r}")
    spec = DI.custom_spec(d_out, d_in, r, 1, dtype="bf16", s=1.5, b_std=0.05)
    L = DI.make_layer(spec, 60 + r + d_out % 7, device=DEV, activations=False, gen_device="cuda")
    wn, g = gpu_norm(L)
    rows = sample_rows(d_out, 256, seed=r)
    ref_wn, ref_g = oracle_norm(L, rows)
    assert np.all(np.isfinite(host64(wn))) and np.all(host64(wn) > 0)
    check_rel(host64(wn)[rows], ref_wn, NORM_RTOL[L.W0.dtype], "wnorm")
    check_rel(host64(g)[rows], ref_g, NORM_RTOL[L.W0.dtype], "g")


@pytest.mark.parametrize("d_out,d_in,r", [(8000, 2056, 384), (7200, 4096, 136), (8192, 1792, 256),
                                          (7169, 3000, 200)])
def test_norm_eight_chunk_shapes(d_out, d_in, r):
    # bf16 r > 128 with 29 to 32 m-tiles of 256 rows: the large-tile pass in
    # eight K-chunks, chunk 7 ending in the B | Gs k-tiles.  Ragged last
    # m-tiles (8000, 7200, 7169 rows), K tails (2056, 3000) and the fewest
    # k-tiles per chunk (1792: 4 or 5 of 34); sampled rows against the
    # oracle, repeated calls bitwise equal, and a group of one member
    # bitwise equal too
    say(f"[parity] eight-chunk norm {d_out}x{d_in} r={r}")
    spec = DI.custom_spec(d_out, d_in, r, 1, dtype="bf16", s=1.5, b_std=0.05)
    L = DI.make_layer(spec, 90 + r + d_out % 11, device=DEV, activations=False, gen_device="cuda")
    wn, g = gpu_norm(L)
    rows = sample_rows(d_out, 256, seed=r + 1)
    ref_wn, ref_g = oracle_norm(L, rows)
    check_rel(host64(wn)[rows], ref_wn, NORM_RTOL[L.W0.dtype], "wnorm")
    check_rel(host64(g)[rows], ref_g, NORM_RTOL[L.W0.dtype], "g")
    wn2, g2 = gpu_norm(L)
    (wn3, g3), = D.factored_norm_group([(L.W0, L.A, L.B, L.spec.s, L.m)])
    torch.cuda.synchronize()
    assert torch.equal(wn, wn2) and torch.equal(g, g2)
    assert torch.equal(wn, wn3) and torch.equal(g, g3)


def test_norm_unaligned_operands_take_the_fallback_plan():
    # a W0 that is not 16-byte aligned cannot use the LDS-DMA tiles; the call
    # runs the register-staged plan inside the same workspace size
    say("[parity] norm unaligned W0, r=384 bf16")
    spec = DI.custom_spec(300, 520, 384, 1, dtype="bf16", s=1.5, b_std=0.05)
    L = DI.make_layer(spec, 23, device=DEV, activations=False)
    buf = torch.empty(L.W0.numel() + 1, dtype=L.W0.dtype, device=DEV)
    W0u = buf[1:].view_as(L.W0)
    W0u.copy_(L.W0)
    assert W0u.data_ptr() % 16 != 0
    wn, g = D.factored_norm(W0u, L.A, L.B, spec.s, L.m)
    torch.cuda.synchronize()
    ref_wn, ref_g = oracle_norm(L)
    check_rel(host64(wn), ref_wn, NORM_RTOL[L.W0.dtype], "wnorm")
    check_rel(host64(g), ref_g, NORM_RTOL[L.W0.dtype], "g")


@pytest.mark.parametrize("dt,r,d_in", [("bf16", 48, 520), ("f32", 48, 520), ("bf16", 16, 4096), ("bf16", 32, 2056)])
def test_norm_dominated_by_low_rank_term(dt, r, d_in):
    # W0 = 0: the whole norm comes from the cross-free s^2 B G B^T term (for
    # bf16 r <= 32 formed per K-chunk inside the W0 pass)
    say(f"[parity] norm W0=0 {dt} r={r} d_in={d_in}")
    spec = DI.custom_spec(300, d_in, r, 1, dtype=dt, s=2.0, b_std=0.3)
    L = DI.make_layer(spec, 5, device=DEV, activations=False, w_scale=0.0)
    wn, _ = gpu_norm(L, m=False)
    ref, _ = oracle_norm(L)
    check_rel(host64(wn), ref, NORM_RTOL[L.W0.dtype], "wnorm W0=0")


@pytest.mark.parametrize("d_out,d_in,r", [(96, 2048, 1536), (64, 512, 2048), (64, 512, 2056), (40, 9000, 448)])
def test_norm_wide_rank(d_out, d_in, r):
    # r from 1536 to 2048 takes the large-tile form with several slices of r,
    # Gram tiles of A over many 64-row blocks (several Gram units per W0-pass
    # workgroup) and an assembly kernel whose LDS holds B rows of more than
    # 64 KB; r = 2056 is past that form and runs the 128-row plan.
    say(f"[parity] norm wide rank {d_out}x{d_in} r={r}")
    spec = DI.custom_spec(d_out, d_in, r, 1, dtype="bf16", s=0.5, b_std=0.02)
    L = DI.make_layer(spec, 90 + r, device=DEV, activations=False)
    wn, g = gpu_norm(L)
    ref_wn, ref_g = oracle_norm(L)
    check_rel(host64(wn), ref_wn, NORM_RTOL[L.W0.dtype], "wnorm")
    check_rel(host64(g), ref_g, NORM_RTOL[L.W0.dtype], "g")


@pytest.mark.parametrize("r", [16, 36, 64, 384])
def test_norm_gram_term_dominant_with_cancellation(r):
    # A bf16 layer built so that s^2 B_i G B_i^T is about twice the base term
    # and the cross term cancels most of it: W0 = round(W1 - (s/2) B A) with
    # ||s (BA)_i|| about 2 ||W1_i||, so base ~ 2, 2s cross ~ -4, s^2 ba ~ 4 and
    # n^2 ~ 2.  An error of the Gram term relative to itself is multiplied by
    # about 2 in n^2 here, so this is where its rounding shows first.
    say(f"[parity] Gram-dominant bf16 layer r={r}")
    s = 1.0
    spec = DI.custom_spec(512, 2048, r, 1, dtype="bf16", s=s, b_std=math.sqrt(12.0 / r))
    L = DI.make_layer(spec, 40 + r, device=DEV, activations=False)
    W1, A, B = (t.cpu().to(torch.float64) for t in (L.W0, L.A, L.B))
    L.W0 = (W1 - 0.5 * s * (B @ A)).to(torch.bfloat16).to(DEV)
    wn, g = gpu_norm(L)
    ref_wn, ref_g = oracle_norm(L)
    # the construction did what it says: the Gram term is large against n^2
    W0d = L.W0.cpu().to(torch.float64)
    base = (W0d * W0d).sum(1)
    ba = ((B @ A) ** 2).sum(1) * s * s
    assert float((ba / torch.as_tensor(ref_wn ** 2)).median()) > 1.5
    assert float((base / torch.as_tensor(ref_wn ** 2)).median()) > 0.8
    check_rel(host64(wn), ref_wn, NORM_RTOL[L.W0.dtype], "wnorm")
    check_rel(host64(g), ref_g, NORM_RTOL[L.W0.dtype], "g")


def test_norm_zero_row_eps_clamp():
    say("[parity] zero row / eps clamp")
    spec = DI.custom_spec(64, 128, 8, 1, dtype="bf16")
    L = DI.make_layer(spec, 3, device=DEV, activations=False)
    L.W0[5].zero_()
    L.B[5].zero_()
    eps = 0.25
    wn, g = gpu_norm(L, eps=eps)
    assert wn[5].item() == 0.0
    assert g[5].item() == np.float32(L.m[5].item() / eps)
    ref_wn, ref_g = oracle_norm(L, eps=eps)
    check_rel(host64(wn)[np.arange(64) != 5], ref_wn[np.arange(64) != 5], 2e-3, "wnorm")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_norm_scale_zero(dt):
    say(f"[parity] s = 0 {dt}")
    spec = DI.custom_spec(333, 4104, 16, 1, dtype=dt)
    L = DI.make_layer(spec, 9, device=DEV, activations=False)
    wn, g = gpu_norm(L, s=0.0)
    ref = np.linalg.norm(host64(L.W0), axis=1)
    check_rel(host64(wn), ref, NORM_RTOL[L.W0.dtype], "wnorm s=0")


CANCEL_CASES = [(256, 512, 256, "bf16"), (256, 512, 32, "bf16"), (128, 256, 16, "f32")]


@pytest.mark.parametrize("d_out,d_in,r,dt", CANCEL_CASES)
def test_norm_near_cancellation(d_out, d_in, r, dt):
    # Rows with W0_i close to -s (BA)_i: n^2 is a small difference of large
    # terms, so relative error means nothing there.  Checked: wnorm finite and
    # >= 0 everywhere, and wnorm^2 within an absolute bound built from the
    # magnitudes the kernel sums (base, 2|s| sum_j |B_ij| (|W0||A|^T)_ij,
    # s^2 (|B||G||B|^T)_ii).  The bf16 rounding of (s/2) A A^T is at most 2^-8
    # relative and touches only the s^2 term; fp32 accumulation over d_in
    # terms adds at most d_in 2^-23 relative to the magnitudes (fp32 inputs:
    # the accumulation term alone).
    say(f"[parity] near cancellation {d_out}x{d_in} r={r} {dt}")
    dtype = DI.DTYPES[dt]
    g = torch.Generator().manual_seed(d_out + r)
    s = 1.25
    A = ((torch.rand(r, d_in, generator=g) * 2 - 1) / d_in ** 0.5).to(dtype)
    B = (torch.randn(d_out, r, generator=g) * 0.3).to(dtype)
    BA = B.double() @ A.double()
    W0 = torch.randn(d_out, d_in, generator=g, dtype=torch.float64) / d_in ** 0.5
    near = torch.arange(d_out) % 2 == 0
    W0[near] = -s * BA[near] + 1e-3 * W0[near]
    W0 = W0.to(dtype)
    wn, _ = D.factored_norm(W0.to(DEV), A.to(DEV), B.to(DEV), s)
    torch.cuda.synchronize()
    got = host64(wn)
    assert np.all(np.isfinite(got)) and np.all(got >= 0)
    W0d, Ad, Bd = (oracle.as_f64(t) for t in (W0, A, B))
    ref = oracle.dense_row_norm(W0, A, B, s)
    base = np.sum(W0d * W0d, axis=1)
    cross_abs = np.sum(np.abs(Bd) * (np.abs(W0d) @ np.abs(Ad).T), axis=1)
    G = Ad @ Ad.T
    gram_abs = np.sum((np.abs(Bd) @ np.abs(G)) * np.abs(Bd), axis=1)
    scale = base + 2 * abs(s) * cross_abs + s * s * gram_abs
    u = (2.0 ** -8 if dtype == torch.bfloat16 else 0.0) + d_in * 2.0 ** -23
    err = np.abs(got ** 2 - ref ** 2)
    assert np.all(err <= u * scale), (float(np.max(err / scale)), u)
    # the cancelling rows really are small against their terms
    assert np.max(ref[near.numpy()] ** 2 / scale[near.numpy()]) < 1e-2


def test_norm_deterministic():
    L = config_layer(3)
    say("[parity] norm determinism")
    a = gpu_norm(L)
    b = gpu_norm(L)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# --------------------------------------------------------------- compose
def oracle_g_f32(L):
    """g from the oracle, rounded to fp32: compose tests feed both sides this g."""
    _, g = oracle_norm(L)
    return torch.tensor(g, dtype=torch.float32)


def _compose_check(L, g32, rows=None, delta=False, tag=""):
    dt = L.base_out.dtype
    s = L.spec.s
    y = D.compose(L.base_out, L.lora_out, g32.to(DEV), s, delta_only=delta)
    torch.cuda.synchronize()
    base, lora, got = host64(L.base_out), host64(L.lora_out), host64(y)
    if rows is not None:
        base, lora, got = base[rows], lora[rows], got[rows]
    ref = oracle.compose_forward(base, lora, oracle.as_f64(g32), s, delta_only=delta)
    check_act(got, ref, dt, f"{tag} y(delta={delta})")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_compose_forward_config(cfg):
    L = config_layer(cfg)
    say(f"[parity] compose fwd config {cfg}")
    g32 = oracle_g_f32(L) if cfg != 4 else gpu_norm(L)[1].cpu()
    rows = None if cfg in (1, 2) else sample_rows(L.spec.T, 256, seed=cfg)
    _compose_check(L, g32, rows=rows, tag=f"cfg{cfg}")
    _compose_check(L, g32, rows=rows, delta=True, tag=f"cfg{cfg}")


def _peak_error(got, ref):
    """Largest |got - ref|, absolute and relative to the largest |ref|."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    return float(err.max()), float(err.max() / np.abs(ref).max())


def test_compose_error_near_unit_g():
    # [ScalingDoRA] §3 (compose stability) compares, in bf16 at [2048, 8192]
    # with g close to 1, the peak error of the composition evaluated as
    # g * (base + s lora) against the form base + (g - 1) base + g s lora,
    # both against fp64.  Here three evaluations share the bf16 branch
    # outputs and the fp32 g of the 8192^2 r=384 layer (g = 1 + O(1e-3)):
    #   naive   g * (base + s lora), each op a bf16 torch op (g rounded to bf16)
    #   stable  base + (g - 1) base + (g s) lora, each op a bf16 torch op
    #           ((g - 1) and g s formed in fp32, then rounded to bf16)
    #   fused   the compose kernel: the stable form in fp32, rounded once.
    # The kernel's error must be the smallest of the three, within bf16's
    # half-spacing at the result plus fp32 rounding, and the test prints the
    # three peaks so the ratio can be set beside the pages' figure.
    L = config_layer(3)
    g32 = oracle_g_f32(L)
    s = L.spec.s
    assert abs(float(g32.mean()) - 1.0) < 1e-2 and float(g32.std()) < 1e-2
    gd = g32.to(DEV)
    base, lora = L.base_out, L.lora_out
    y_fused = D.compose(base, lora, gd, s)
    bf = torch.bfloat16
    y_naive = gd.to(bf)[None, :] * (base + s * lora)
    y_stable = base + (gd - 1.0).to(bf)[None, :] * base + (gd * s).to(bf)[None, :] * lora
    torch.cuda.synchronize()
    ref = oracle.compose_forward(host64(base), host64(lora), oracle.as_f64(g32), s)
    peaks = {k: _peak_error(host64(v), ref) for k, v in
             (("fused", y_fused), ("stable", y_stable), ("naive", y_naive))}
    for k, (a, rel) in peaks.items():
        say(f"[compose error] {k:6s} peak |err| {a:.4e}  ({rel:.3e} of max |ref|)")
    say(f"[compose error] naive/fused {peaks['naive'][0] / peaks['fused'][0]:.2f}x  "
        f"naive/stable {peaks['naive'][0] / peaks['stable'][0]:.2f}x  |ref| max {np.abs(ref).max():.3f}")
    assert peaks["fused"][0] <= peaks["stable"][0] <= peaks["naive"][0]
    # one rounding to bf16 plus the fp32 evaluation of three terms
    err = np.abs(host64(y_fused) - ref)
    scale = np.abs(host64(base)) * (1 + np.abs(oracle.as_f64(g32) - 1)) + np.abs(oracle.as_f64(g32) * s * host64(lora))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(err <= 0.5 * ulp + 2.0 ** -21 * scale)


def _bwd_check(L, g32, wn32, delta=False, rows=None, cols=None, tag=""):
    dt = L.dy.dtype
    s = L.spec.s
    eps = D.default_eps(dt)
    g, wn = g32.to(DEV), wn32.to(DEV)
    db, dl, dm = D.compose_backward(L.dy, L.base_out, L.lora_out, g, wn, s, eps, delta_only=delta)
    torch.cuda.synchronize()
    csel = slice(None) if cols is None else cols
    dy, base, lora = (host64(t)[:, csel] for t in (L.dy, L.base_out, L.lora_out))
    r_db, r_dl, r_dm = oracle.compose_backward(dy, base, lora, oracle.as_f64(g32)[csel],
                                               oracle.as_f64(wn32)[csel], s, eps, delta_only=delta)
    got_db, got_dl = host64(db)[:, csel], host64(dl)[:, csel]
    if rows is not None:
        got_db, got_dl, r_db, r_dl = got_db[rows], got_dl[rows], r_db[rows], r_dl[rows]
    check_act(got_db, r_db, dt, f"{tag} d_base")
    check_act(got_dl, r_dl, dt, f"{tag} d_lora")
    check_act(host64(dm)[csel], r_dm, dt, f"{tag} d_m")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_compose_backward_config(cfg):
    L = config_layer(cfg)
    say(f"[parity] compose bwd config {cfg}")
    if cfg == 4:
        wn, g = gpu_norm(L)
        g32, wn32 = g.cpu(), wn.cpu()
        cols = sample_rows(L.spec.d_out, 256, seed=44)
    else:
        wn64, g64 = oracle_norm(L)
        g32, wn32 = torch.tensor(g64, dtype=torch.float32), torch.tensor(wn64, dtype=torch.float32)
        cols = None
    rows = None if cfg in (1, 2) else sample_rows(L.spec.T, 256, seed=cfg + 1)
    _bwd_check(L, g32, wn32, rows=rows, cols=cols, tag=f"cfg{cfg}")
    if cfg in (1, 3):
        _bwd_check(L, g32, wn32, delta=True, rows=rows, cols=cols, tag=f"cfg{cfg}")


COMPOSE_EDGE = [
    # T, d_out, dtype
    (1, 1000, "bf16"), (37, 1000, "bf16"), (37, 1003, "bf16"), (5, 7, "f32"), (70, 517, "f32"),
    (33, 520, "f16"), (65, 8, "bf16"), (2, 1, "bf16"), (300, 4104, "bf16"),
]


@pytest.mark.parametrize("T,d_out,dt", COMPOSE_EDGE)
def test_compose_edge_shapes(T, d_out, dt):
    say(f"[parity] compose edge T={T} d_out={d_out} {dt}")
    torch.manual_seed(T * 1000 + d_out)
    dtype = DI.DTYPES[dt]
    base = torch.randn(T, d_out).to(dtype).to(DEV)
    lora = torch.randn(T, d_out).to(dtype).to(DEV)
    dy = torch.randn(T, d_out).to(dtype).to(DEV)
    g32 = (1.0 + 1e-3 * torch.randn(d_out)).float()
    wn32 = (1.0 + 0.1 * torch.rand(d_out)).float()
    s = 0.75
    y = D.compose(base, lora, g32.to(DEV), s)
    db, dl, dm = D.compose_backward(dy, base, lora, g32.to(DEV), wn32.to(DEV), s, 1e-6)
    torch.cuda.synchronize()
    b64, l64, d64 = host64(base), host64(lora), host64(dy)
    g64, w64 = oracle.as_f64(g32), oracle.as_f64(wn32)
    check_act(host64(y), oracle.compose_forward(b64, l64, g64, s), dtype, "y")
    r_db, r_dl, r_dm = oracle.compose_backward(d64, b64, l64, g64, w64, s, 1e-6)
    tol_dtype = torch.bfloat16 if dtype == torch.float16 else dtype
    check_act(host64(db), r_db, tol_dtype, "d_base")
    check_act(host64(dl), r_dl, tol_dtype, "d_lora")
    check_act(host64(dm), r_dm, tol_dtype, "d_m")


def _misaligned(t):
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = buf[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


def test_unaligned_pointers_take_the_scalar_path():
    say("[parity] unaligned pointers")
    L = DI.make_layer(DI.custom_spec(256, 512, 16, 64, dtype="bf16"), 21, device=DEV)
    wn_a, g_a = gpu_norm(L)
    W0u, Au, Bu = _misaligned(L.W0), _misaligned(L.A), _misaligned(L.B)
    wn_u, g_u = D.factored_norm(W0u, Au, Bu, L.spec.s, L.m)
    ref, _ = oracle_norm(L)
    check_rel(host64(wn_u), ref, 2e-3, "wnorm unaligned")
    bu, lu = _misaligned(L.base_out), _misaligned(L.lora_out)
    y_a = D.compose(L.base_out, L.lora_out, g_a, L.spec.s)
    y_u = D.compose(bu, lu, g_a, L.spec.s)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_u)   # same arithmetic on either path


def test_t_zero():
    say("[parity] T = 0")
    g = torch.ones(64, device=DEV)
    empty = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    y = D.compose(empty, empty, g, 1.0)
    _, _, dm = D.compose_backward(empty, empty, empty, g, g, 1.0, 1e-6)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    assert torch.equal(dm, torch.zeros(64, device=DEV))


def test_init_exact_reproduces_base_output():
    # m0 = ||W0||_row from the same GPU routine and B = 0: g == 1 exactly and
    # y == base_out bitwise, delta == 0.
    say("[parity] init exactness")
    L = DI.make_layer(DI.custom_spec(1024, 2048, 64, 128, dtype="bf16", s=2.0), 31, device=DEV)
    L.B.zero_()
    DI.branch_outputs(L)
    m0, _ = D.factored_norm(L.W0, L.A, L.B, 2.0)
    _, g = D.factored_norm(L.W0, L.A, L.B, 2.0, m0.clone())
    y = D.compose(L.base_out, L.lora_out, g, 2.0)
    dlt = D.compose(L.base_out, L.lora_out, g, 2.0, delta_only=True)
    torch.cuda.synchronize()
    assert torch.equal(g, torch.ones_like(g))
    assert torch.equal(y, L.base_out)
    assert torch.count_nonzero(dlt).item() == 0


def test_inplace_alias_and_frozen_magnitude():
    say("[parity] aliasing and frozen m")
    L = DI.make_layer(DI.custom_spec(512, 256, 16, 96, dtype="bf16"), 41, device=DEV)
    _, g = gpu_norm(L)
    y_ref = D.compose(L.base_out, L.lora_out, g, L.spec.s)
    b = L.base_out.clone()
    y_in = D.compose(b, L.lora_out, g, L.spec.s, out=b)
    d_base, d_lora, _ = D.compose_backward(L.dy, None, None, g, None, L.spec.s, need_d_m=False)
    dyc = L.dy.clone()
    d_base2, _, _ = D.compose_backward(dyc, None, None, g, None, L.spec.s, need_d_m=False, need_d_lora=False,
                                       d_base=dyc)
    torch.cuda.synchronize()
    assert torch.equal(y_in, y_ref)
    assert torch.equal(d_base2, d_base)
    ref_db, ref_dl, _ = oracle.compose_backward(host64(L.dy), host64(L.base_out), host64(L.lora_out),
                                                host64(g), np.ones(512), L.spec.s, 1e-6)
    check_act(host64(d_base), ref_db, torch.bfloat16, "d_base frozen")
    check_act(host64(d_lora), ref_dl, torch.bfloat16, "d_lora frozen")


def test_backward_deterministic():
    L = config_layer(3)
    say("[parity] bwd determinism")
    wn, g = gpu_norm(L)
    a = D.compose_backward(L.dy, L.base_out, L.lora_out, g, wn, L.spec.s)
    a = tuple(t.clone() for t in a)
    b = D.compose_backward(L.dy, L.base_out, L.lora_out, g, wn, L.spec.s)
    torch.cuda.synchronize()
    for x, z in zip(a, b):
        assert torch.equal(x, z)


def test_end_to_end_chain_against_oracle():
    # GPU norm -> GPU g -> GPU compose, against the oracle's fp64 chain.
    for cfg in (1, 3):
        L = config_layer(cfg)
        say(f"[parity] end-to-end chain config {cfg}")
        wn, g = gpu_norm(L)
        y = D.compose(L.base_out, L.lora_out, g, L.spec.s)
        torch.cuda.synchronize()
        rows = None if cfg == 1 else sample_rows(L.spec.T, 128, seed=5)
        _, g_ref = oracle_norm(L)
        base, lora = host64(L.base_out), host64(L.lora_out)
        if rows is not None:
            base, lora = base[rows], lora[rows]
        ref = oracle.compose_forward(base, lora, g_ref, L.spec.s)
        got = host64(y) if rows is None else host64(y)[rows]
        check_act(got, ref, L.base_out.dtype, f"cfg{cfg} chain")


def test_autograd_function_matches_direct_calls():
    say("[parity] autograd wiring")
    L = DI.make_layer(DI.custom_spec(256, 128, 8, 40, dtype="bf16"), 51, device=DEV)
    wn, g = gpu_norm(L)
    base = L.base_out.clone().requires_grad_(True)
    lora = L.lora_out.clone().requires_grad_(True)
    m = L.m.clone().requires_grad_(True)
    eps = D.default_eps(torch.bfloat16)
    y = D.DoRACompose.apply(base, lora, m, g, wn, L.spec.s, eps, False)
    y.backward(L.dy)
    db, dl, dm = D.compose_backward(L.dy, L.base_out, L.lora_out, g, wn, L.spec.s, eps)
    torch.cuda.synchronize()
    assert torch.equal(base.grad, db) and torch.equal(lora.grad, dl) and torch.equal(m.grad, dm)


def test_sweep_layer_modules():
    # one layer of the many-module sweep (7 projections), sampled rows
    for proj in range(len(DI.SWEEP_PROJECTIONS)):
        spec = DI.sweep_spec(proj)
        say(f"[parity] sweep module {spec.name}")
        L = DI.make_layer(spec, DI.sweep_seed(0, proj), device=DEV, activations=False)
        wn, g = gpu_norm(L)
        rows = sample_rows(spec.d_out, 128, seed=proj)
        ref_wn, ref_g = oracle_norm(L, rows)
        check_rel(host64(wn)[rows], ref_wn, 2e-3, f"{spec.name} wnorm")
        check_rel(host64(g)[rows], ref_g, 2e-3, f"{spec.name} g")
        del L
        torch.cuda.empty_cache()


@pytest.mark.parametrize("proj", [1, 0, 4])
def test_sweep_shapes_compose(proj):
    # compose forward, backward and the (dy, inner) tier at the sweep's own
    # activation shapes, T = 2048 with d_out = 1024 (k), 5120 (q) and 27648
    # (gate): sampled tokens for the element-wise outputs, sampled columns
    # (over all tokens) for d_m
    spec = DI.sweep_spec(proj)
    say(f"[parity] sweep-shape compose {spec.name}")
    L = DI.make_layer(spec, DI.sweep_seed(0, proj), device=DEV, gen_device="cuda")
    wn, g = gpu_norm(L)
    g32, wn32 = g.cpu(), wn.cpu()
    rows = sample_rows(spec.T, 128, seed=100 + proj)
    cols = sample_rows(spec.d_out, 256, seed=110 + proj)
    _compose_check(L, g32, rows=rows, tag=spec.name)
    _bwd_check(L, g32, wn32, rows=rows, cols=cols, tag=spec.name)
    s, eps = spec.s, D.default_eps(L.dy.dtype)
    y, inner = D.compose_dual(L.base_out, L.lora_out, g, s)
    db, dl, dm = D.compose_backward_inner(L.dy, inner, g, wn, s, eps)
    torch.cuda.synchronize()
    b64, l64 = host64(L.base_out[rows]), host64(L.lora_out[rows])
    r_y, r_i = oracle.compose_forward_inner(b64, l64, host64(g), s)
    check_act(host64(y[rows]), r_y, L.dy.dtype, f"{spec.name} dual y")
    check_act(host64(inner[rows]), r_i, L.dy.dtype, f"{spec.name} inner")
    d64, i64 = host64(L.dy)[:, cols], host64(inner)[:, cols]
    r_db, r_dl, r_dm = oracle.compose_backward_inner(d64, i64, host64(g)[cols], host64(wn)[cols], s, eps)
    check_act(host64(db)[:, cols][rows], r_db[rows], L.dy.dtype, f"{spec.name} inner d_base")
    check_act(host64(dl)[:, cols][rows], r_dl[rows], L.dy.dtype, f"{spec.name} inner d_lora")
    check_act(host64(dm)[cols], r_dm, L.dy.dtype, f"{spec.name} inner d_m")
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d_out,d_in,r", [(1024, 2048, 384), (2048, 4096, 16), (8000, 2048, 384)])
def test_graph_capture_replays_match_eager(d_out, d_in, r):
    # norm, compose forward and backward captured in one HIP graph (the
    # library records no memsets): every replay, with eager work and a
    # synchronisation in between, gives bitwise the eager results
    say(f"[parity] graph capture {d_out}x{d_in} r={r}")
    L = DI.make_layer(DI.custom_spec(d_out, d_in, r, 256, s=1.0, b_std=0.02), 71 + r, device=DEV)
    s, eps = L.spec.s, D.default_eps(L.W0.dtype)
    ws_n = torch.empty(D.norm_workspace_size(d_out, d_in, r, L.W0.dtype), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(max(1, D.compose_backward_workspace_size(256, d_out)), dtype=torch.uint8, device=DEV)
    wn, g = torch.empty(d_out, device=DEV), torch.empty(d_out, device=DEV)
    y, db, dl = (torch.empty_like(L.base_out) for _ in range(3))
    dm = torch.empty(d_out, device=DEV)

    def run():
        D.factored_norm(L.W0, L.A, L.B, s, L.m, eps, wnorm=wn, g=g, ws=ws_n)
        D.compose(L.base_out, L.lora_out, g, s, out=y)
        D.compose_backward(L.dy, L.base_out, L.lora_out, g, wn, s, eps, d_base=db, d_lora=dl, d_m=dm, ws=ws_b)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (wn, g, y, db, dl, dm)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    other = DI.make_layer(DI.custom_spec(512, 1024, 64, 1), 72, device=DEV, activations=False)
    for rep in range(3):
        for t in (wn, g, y, db, dl, dm):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for got, ref, name in zip((wn, g, y, db, dl, dm), eager, ("wnorm", "g", "y", "d_base", "d_lora", "d_m")):
            assert torch.equal(got, ref), f"replay {rep}: {name}"
        D.factored_norm(other.W0, other.A, other.B, 1.0, other.m)   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("d_out,d_in", [(28000, 8200), (24000, 12288)])
def test_norm_balanced_k_split(d_out, d_in):
    # r = 384 with 110 or 94 m-tiles of 256 rows (the last one ragged) and
    # 134 or 198 k-tiles per workgroup under a uniform two-way K split, which
    # would leave CUs idle: 256 workgroups take equal ranges of the (m-tile,
    # k-tile) pairs instead, some running two segments (the tail of one
    # m-tile and the head of the next) and each m-tile summing its partial
    # slots.  Sampled rows plus every row at m-tile boundaries and the end.
    say(f"[parity] balanced K split {d_out}x{d_in} r=384")
    spec = DI.custom_spec(d_out, d_in, 384, 1, dtype="bf16", s=1.0, b_std=0.02)
    L = DI.make_layer(spec, 77 + d_in, device=DEV, activations=False, gen_device="cuda")
    wn, g = gpu_norm(L)
    edges = [b + o for b in range(0, d_out, 256 * 7) for o in (-1, 0, 255) if 0 <= b + o < d_out]
    rows = np.unique(np.concatenate([sample_rows(d_out, 160, seed=d_in), np.array(edges), np.arange(d_out - 40, d_out)]))
    ref_wn, ref_g = oracle_norm(L, rows)
    assert np.all(np.isfinite(host64(wn))) and np.all(host64(wn) > 0)
    check_rel(host64(wn)[rows], ref_wn, NORM_RTOL[L.W0.dtype], "wnorm")
    check_rel(host64(g)[rows], ref_g, NORM_RTOL[L.W0.dtype], "g")
    wn2, _ = gpu_norm(L)
    assert torch.equal(wn, wn2)
