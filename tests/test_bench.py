"""bench.py's host side (no GPU): the algorithmic work it divides by, the roof
it reports the norm against, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402

# (d_out, d_in, r, T): square 8192 at r = 384, the 28672-row MLP projection,
# and the square 4096 layer at r = 16
SQUARE, MLP_UP, LOW_RANK = (8192, 8192, 384, 2048), (28672, 8192, 384, 4096), (4096, 4096, 16, 2048)


@pytest.mark.parametrize("shape,gflop,mbytes", [
    (SQUARE, 55.31, 146.9),
    (MLP_UP, 190.6, 498.4),
    (LOW_RANK, 0.574, 33.87),
])
def test_norm_work(shape, gflop, mbytes):
    # the factored norm's FLOPs and its bytes (W0, A, B read once; m read;
    # wnorm and g written), against figures worked out by hand for these
    # layers to four significant digits
    d_out, d_in, r, _ = shape
    assert bench.norm_flops(d_out, d_in, r) / 1e9 == pytest.approx(gflop, rel=1e-3)
    assert bench.norm_bytes(d_out, d_in, r, 2) / 1e6 == pytest.approx(mbytes, rel=1e-3)


@pytest.mark.parametrize("shape,fwd_mb,bwd_mb", [
    (SQUARE, 100.7, 167.9),
    (MLP_UP, 704.8, 1174.7),
    (LOW_RANK, 50.35, 83.9),
])
def test_compose_bytes(shape, fwd_mb, bwd_mb):
    # forward: base and lora read, y written (6 B per bf16 element);
    # backward: dy, base, lora read, d_base and d_lora written (10 B)
    _, _, _, T = shape
    d_out = shape[0]
    assert bench.compose_fwd_bytes(T, d_out, 2) / 1e6 == pytest.approx(fwd_mb, rel=1e-3)
    assert bench.compose_bwd_bytes(T, d_out, 2) / 1e6 == pytest.approx(bwd_mb, rel=1e-3)
    # the training tier moves one activation less each way
    assert bench.compose_dual_bytes(T, d_out, 2) - bench.compose_fwd_bytes(T, d_out, 2) == T * d_out * 2
    assert bench.compose_bwd_bytes(T, d_out, 2) - bench.compose_bwd_inner_bytes(T, d_out, 2) == T * d_out * 2


def test_roofline_picks_the_bound_of_the_arithmetic_intensity():
    # 8192^2 r = 384 runs at ~376 FLOP/B, above the 2500 TFLOP/s / 8 TB/s
    # ridge (312.5 FLOP/B): judged against the MFMA peak
    d_out, d_in, r, _ = SQUARE
    f, b = bench.norm_flops(d_out, d_in, r), bench.norm_bytes(d_out, d_in, r, 2)
    roof = bench.norm_roofline(f, b, 80e-6, bench.PEAK_BF16_TFLOPS, 123)
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["traffic"] == 123
    assert roof["achieved"] == pytest.approx(f / 80e-6 / 1e12, rel=1e-4)
    assert roof["frac"] == pytest.approx(roof["achieved"] / bench.PEAK_BF16_TFLOPS, rel=1e-3)
    # 4096^2 r = 16 runs at ~17 FLOP/B: judged against HBM bandwidth
    d_out, d_in, r, _ = LOW_RANK
    f, b = bench.norm_flops(d_out, d_in, r), bench.norm_bytes(d_out, d_in, r, 2)
    roof = bench.norm_roofline(f, b, 13e-6, bench.PEAK_BF16_TFLOPS, None)
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == bench.PEAK_HBM_GBS
    assert roof["achieved"] == pytest.approx(b / 13e-6 / 1e9, rel=1e-4)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_traced_kernel_times_are_read_only_for_the_current_sources(tmp_path, monkeypatch):
    table = ["# Kernel durations, workload w, one MI355X", "", "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|", "| w0_pass | 48 | 60.4 | 58.0 | 66.6 | 16.9 |",
             "| gram_finalize<...> | 48 | 4.8 | 3.9 | 5.8 | 1.3 |", "| compose_fwd_vec (y) | 48 | 18.5 | 17.5 | 21.0 | 5.1 |",
             "", "| kernel | dispatches | p10 | median | p90 |", "|---|---|---|---|---|", "| w0_pass | 48 | 58.3 | 59.1 | 63.2 |",
             "", "captured: 2026-12-01 at abc1234", "source_sha256: abc"]
    (tmp_path / "kernels_w.txt").write_text("\n".join(table) + "\n")
    traffic = ["# HBM traffic per dispatch, workload w", "", "traffic_bytes_per_call: 223121169",
               "captured: 2026-12-01 at abc1234", "source_sha256: abc"]
    (tmp_path / "norm_traffic_w.txt").write_text("\n".join(traffic) + "\n")
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    monkeypatch.setattr(bench, "norm_source_digest", lambda: "abc")
    assert bench.stored_norm_kernels("w") == {"captured": "2026-12-01 at abc1234", "w0_pass": 60.4,
                                              "gram_finalize": 4.8}
    assert bench.stored_traffic("w") == (223121169, "2026-12-01 at abc1234")
    monkeypatch.setattr(bench, "norm_source_digest", lambda: "other")
    assert bench.stored_norm_kernels("w") is None
    assert bench.stored_traffic("w") is None
    assert bench.stored_norm_kernels("absent") is None
    # the W0 pass's own work at 8192^2 r = 384: the extended contraction and the base squares
    assert bench.w0_pass_flops(8192, 8192, 384) / 1e9 == pytest.approx(54.09, rel=1e-3)


def test_eager_comparator_computes_the_compose():
    # the bench's eager op sequence (the pages' comparator) computes what the
    # oracle does, here in fp32 on the CPU
    import numpy as np
    import torch

    import bench
    import oracle
    rng = np.random.default_rng(3)
    T, d = 7, 13
    base, lora, dy = (rng.standard_normal((T, d)) for _ in range(3))
    g, wn = 1 + 0.1 * rng.standard_normal(d), 1 + 0.1 * rng.standard_normal(d)
    s, eps = 0.75, 1e-6
    t = lambda a: torch.tensor(a, dtype=torch.float32)  # noqa: E731
    y = bench.eager_compose_fwd(t(base), t(lora), t(g), s).double().numpy()
    assert np.allclose(y, oracle.compose_forward(base, lora, g, s), rtol=1e-5, atol=1e-5)
    db, dl, dm = bench.eager_compose_bwd(t(dy), t(base), t(lora), t(g), t(wn), s, eps)
    r_db, r_dl, r_dm = oracle.compose_backward(dy, base, lora, g, wn, s, eps)
    for got, ref in ((db, r_db), (dl, r_dl), (dm, r_dm)):
        assert np.allclose(got.double().numpy(), ref, rtol=1e-5, atol=1e-5)
