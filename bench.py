"""Benchmark of the DoRA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

A step is one pass of the whole hot path over one synthetic layer: the
factored norm (Gram, W0 streaming pass, assembly -> wnorm, g), the fused
compose forward and the fused compose backward (d_base, d_lora, d_m).  The
default workload is the headline shape d_out = d_in = 8192, r = 384, bf16,
T = 2048 tokens.

Inputs are resident in HBM before timing starts.  Several copies of every
input are rotated so that one step's working set is not served from the 256 MB
Infinity Cache (MALL) by the previous step.  HIP events recorded on the stream
the library launches on time each call; the step loop is bracketed by
device synchronisations.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import dora_inputs as DI  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "factored-norm TFLOP/s & compose HBM GB/s (% roofline), d_in=8192 r=384 bf16"
MALL_BYTES = 256 << 20


def norm_flops(d_out, d_in, r):
    """Algorithmic FLOPs of the factored norm: U = W0 A^T (2 d_out d_in r),
    base squares (2 d_out d_in), Gram symmetric half (r (r+1) d_in),
    B G (2 d_out r^2), the two row dots (4 d_out r)."""
    return 2 * d_out * d_in * r + 2 * d_out * d_in + r * (r + 1) * d_in + 2 * d_out * r * r + 4 * d_out * r


def norm_bytes(d_out, d_in, r, esz):
    """Algorithmic bytes: W0, A, B read once; m read; wnorm and g written."""
    return (d_out * d_in + r * d_in + d_out * r) * esz + 3 * d_out * 4


def compose_fwd_bytes(T, d_out, esz):
    return 3 * T * d_out * esz + d_out * 4


def compose_bwd_bytes(T, d_out, esz):
    # dy, base, lora read; d_base, d_lora written; g, wnorm read; d_m written
    return 5 * T * d_out * esz + 3 * d_out * 4


def compose_dual_bytes(T, d_out, esz):
    # base, lora read; y and inner written; g read
    return 4 * T * d_out * esz + d_out * 4


def compose_bwd_inner_bytes(T, d_out, esz):
    # dy, inner read; d_base, d_lora written; g, wnorm read; d_m written
    return 4 * T * d_out * esz + 3 * d_out * 4


def merge_bytes(d_out, d_in, r, esz):
    # W0 read and W written once; A, B read once; g read
    return (2 * d_out * d_in + r * (d_in + d_out)) * esz + d_out * 4


COPY_CALIB_BYTES = 256 << 20
PROFILE_DIR = os.path.join(ROOT, "profiles")
NORM_SOURCES = ("dora_adapter_factored_amd/csrc/norm.hip", "dora_adapter_factored_amd/csrc/dora_launch.h",
                "dora_adapter_factored_amd/csrc/dora_balance.h",
                "dora_adapter_factored_amd/csrc/dora_device.h", "dora_adapter_factored_amd/csrc/dora_gfx950.h")


def norm_source_digest():
    """sha256 over what the norm kernels are built from (their sources, the
    hipcc flags and the ROCm version); a stored traffic or kernel-trace
    figure is only valid for the kernels it was taken on."""
    import hashlib
    from dora_adapter_factored_amd.build import HIPCC_FLAGS
    h = hashlib.sha256()
    for rel in NORM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(" ".join(HIPCC_FLAGS).encode())
    try:
        with open("/opt/rocm/.info/version") as f:
            h.update(f.read().strip().encode())
    except OSError:
        h.update(b"rocm-version-unknown")
    return h.hexdigest()


def norm_roofline(flop, nbytes, t, peak_mm, traffic):
    """The norm call against the roof its arithmetic intensity puts it under:
    MFMA when FLOP per algorithmic byte is above the ridge (peak FLOP/s over
    peak HBM bytes/s), HBM otherwise (low rank)."""
    kernel = "dora_factored_norm (every kernel of one call)"
    if flop / nbytes >= peak_mm * 1e12 / (PEAK_HBM_GBS * 1e9):
        ach = flop / t / 1e12
        return {"kernel": kernel, "bound": "mfma", "achieved": round(ach, 2), "peak": peak_mm, "unit": "TFLOP/s",
                "frac": round(ach / peak_mm, 4), "traffic": traffic}
    ach = nbytes / t / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}


def stored_traffic(workload):
    """Per-call HBM bytes of the norm, from the committed counter summary for
    this workload, or None when absent or counted on other kernel sources."""
    path = os.path.join(PROFILE_DIR, f"norm_traffic_{workload}.txt")
    try:
        with open(path) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith((" ", "#", "|")))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != norm_source_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_call"]), kv.get("captured", "unknown")
    except (KeyError, ValueError):
        return None


NORM_KERNELS = ("w0_pass", "w0_rows", "gram_split", "gram_partial", "gram_finalize", "norm_finalize", "row_sumsq")


def stored_norm_kernels(workload):
    """Average duration in us of each norm kernel in the committed rocprofv3
    kernel-trace summary of this workload's bench command, or None when
    absent or traced on other kernel sources.  The bench times the norm as
    one call (its kernels run back to back inside it), so a single kernel's
    time comes from the trace."""
    path = os.path.join(PROFILE_DIR, f"kernels_{workload}.txt")
    try:
        with open(path) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    digest = [l.split(":", 1)[1].strip() for l in lines if l.startswith("source_sha256:")]
    if not digest or digest[0] != norm_source_digest():
        return None
    captured = [l.split(":", 1)[1].strip() for l in lines if l.startswith("captured:")]
    out = {"captured": captured[0] if captured else "unknown"}
    for l in lines:
        if not l.startswith("| "):
            continue
        cells = [c.strip() for c in l.strip("|").split("|")]
        if len(cells) == 6 and cells[0] not in out:   # the averages table: kernel, calls, avg, min, max, %
            name = cells[0].split("<")[0]
            if name in NORM_KERNELS:
                try:
                    out[name] = float(cells[2])
                except ValueError:
                    pass
        elif l.startswith("| kernel | dispatches"):
            break
    return out if len(out) > 1 else None


def w0_pass_flops(d_out, d_in, r):
    """The W0 pass alone: U over the extended contraction [W0 | B] x [A | Gs]^T
    and the base squares."""
    return 2 * d_out * d_in * r + 2 * d_out * d_in + 2 * d_out * r * r


def copy_calibration(dev, reps=10):
    """A plain device-to-device copy of known size (int32, so its kernel is
    told apart from the bf16 copies that build the rotating input sets).
    Counter runs scale FETCH_SIZE / WRITE_SIZE by what this copy reads; its
    event-timed rate is the achievable-HBM context for the compose kernels."""
    n = COPY_CALIB_BYTES // 4
    src = torch.ones(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        dst.copy_(src)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]) * 1e-3
    del src, dst
    return {"bytes_read": COPY_CALIB_BYTES, "bytes_written": COPY_CALIB_BYTES,
            "GBps": round(2 * COPY_CALIB_BYTES / np.median(t) / 1e9, 1)}


def cpu_baseline(layer, budget_s=12.0):
    """The oracle as it stands, on a bounded row sample of the same layer."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    spec = layer.spec
    W0, A, B = layer.W0.cpu(), layer.A.cpu(), layer.B.cpu()
    m = oracle.as_f64(layer.m.cpu())
    chunk = 256
    rows_done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and rows_done < spec.d_out:
        rows = np.arange(rows_done, min(spec.d_out, rows_done + chunk))
        wn = oracle.dense_row_norm(W0, A, B, spec.s, rows=rows)
        oracle.magnitude_scale(m[rows], wn, 1e-7)
        rows_done += rows.size
    t_norm = time.perf_counter() - t0
    flops = norm_flops(spec.d_out, spec.d_in, spec.r) * rows_done / spec.d_out
    # compose forward + backward on a token sample
    tok = min(spec.T, 256)
    base, lora, dy = (oracle.as_f64(t[:tok].cpu()) for t in (layer.base_out, layer.lora_out, layer.dy))
    g = np.ones(spec.d_out)
    t1 = time.perf_counter()
    oracle.compose_forward(base, lora, g, spec.s)
    t_fwd = time.perf_counter() - t1
    t1 = time.perf_counter()
    oracle.compose_backward(dy, base, lora, g, g, spec.s, 1e-7)
    t_bwd = time.perf_counter() - t1
    esz = layer.W0.element_size()
    return {
        "value": flops / t_norm / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"dense fp64 norm of rows 0..{rows_done - 1} of {spec.d_out} ({t_norm:.1f} s); "
                  f"compose fwd+bwd on {tok} of {spec.T} tokens",
        "compose_fwd_GBps": compose_fwd_bytes(tok, spec.d_out, esz) / t_fwd / 1e9,
        "compose_bwd_GBps": compose_bwd_bytes(tok, spec.d_out, esz) / t_bwd / 1e9,
        "cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-serial", action="store_true",
                    help="config 5: report the one-stream schedule even where two streams are faster")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--crossover", action="store_true",
                    help="time the fused compose forward/backward against the eager op sequence (torch ops on "
                         "the GPU, the pages' comparator) over the workloads' activation shapes and a small-shape "
                         "grid, and print them as one JSON line")
    ap.add_argument("--library", action="store_true",
                    help="time the vendor library (hipBLASLt through torch) on the norm's dominant contraction "
                         "W0 A^T, on the Gram A A^T and on the eager merge, beside this library's norm and merge "
                         "at the r = 384 workloads, and print them as one JSON line")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the ceilings only (MFMA-only loops, streams, one CU's reads, the W0 pass's "
                         "access pattern) and print them as one JSON line")
    args = ap.parse_args()
    args.steps_given = any(a.startswith("--steps") for a in sys.argv[1:])
    args.warmup_given = any(a.startswith("--warmup") for a in sys.argv[1:])
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the DoRA norm and compose are "
              "per-layer kernels; sharding them across GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import dora_adapter_factored_amd as D

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.crossover:
        return crossover_main(args, D, dev)
    if args.library:
        return library_main(args, D, dev)
    if args.ceilings:
        from dora_adapter_factored_amd import ceilings as CL
        print(json.dumps({"metric": "measured ceilings (MI355X)", "ceilings": CL.measure(dev, full=True)}), flush=True)
        return
    if args.config == 5:
        return sweep_main(args, D, dev)
    spec = DI.CONFIGS[args.config]
    calib = copy_calibration(dev)
    print(f"[bench] copy calibration {calib}", file=sys.stderr, flush=True)
    print(f"[bench] generating {spec.name}", file=sys.stderr, flush=True)
    layer = DI.make_layer(spec, DI.config_seed(args.config), device=dev)
    dt = layer.W0.dtype
    esz = layer.W0.element_size()
    d_out, d_in, r, T, s = spec.d_out, spec.d_in, spec.r, spec.T, spec.s
    eps = D.default_eps(dt)

    # rotating copies: one step touches its own set of inputs and outputs.
    # Every timed loop (the step, and each entry point called on its own)
    # cycles through at least twice the 256 MB MALL, so no call finds its
    # inputs left in the last-level cache by an earlier one.
    step_bytes = (d_out * d_in + 2 * r * (d_in + d_out)) * esz + 7 * T * d_out * esz
    call_bytes = [step_bytes, norm_bytes(d_out, d_in, r, esz), compose_fwd_bytes(T, d_out, esz),
                  compose_bwd_bytes(T, d_out, esz), compose_dual_bytes(T, d_out, esz),
                  compose_bwd_inner_bytes(T, d_out, esz), merge_bytes(d_out, d_in, r, esz)]
    nsets = max(2, max(int(np.ceil(2 * MALL_BYTES / b)) + 1 for b in call_bytes))
    sets = []
    for i in range(nsets):
        c = (lambda t: t) if i == 0 else (lambda t: t.clone())
        sets.append(dict(W0=c(layer.W0), A=c(layer.A), B=c(layer.B), m=c(layer.m), base=c(layer.base_out),
                         lora=c(layer.lora_out), dy=c(layer.dy),
                         wn=torch.empty(d_out, device=dev), g=torch.empty(d_out, device=dev),
                         y=torch.empty_like(layer.base_out), inner=torch.empty_like(layer.base_out),
                         db=torch.empty_like(layer.base_out),
                         dl=torch.empty_like(layer.base_out), dm=torch.empty(d_out, device=dev)))
    ws_norm = torch.empty(D.norm_workspace_size(d_out, d_in, r, dt), dtype=torch.uint8, device=dev)
    ws_merge = torch.empty(D.merge_workspace_size(d_in, r, dt), dtype=torch.uint8, device=dev)
    w_merged = [torch.empty_like(layer.W0) for _ in range(min(nsets, 2))]
    ws_bwd = torch.empty(max(1, D.compose_backward_workspace_size(T, d_out)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run_norm(st):
        D.factored_norm(st["W0"], st["A"], st["B"], s, st["m"], eps, wnorm=st["wn"], g=st["g"], ws=ws_norm)

    def run_fwd(st):
        D.compose(st["base"], st["lora"], st["g"], s, out=st["y"])

    def run_bwd(st):
        D.compose_backward(st["dy"], st["base"], st["lora"], st["g"], st["wn"], s, eps,
                           d_base=st["db"], d_lora=st["dl"], d_m=st["dm"], ws=ws_bwd)

    def run_dual(st):
        D.compose_dual(st["base"], st["lora"], st["g"], s, out=st["y"], inner=st["inner"])

    def run_bwd_inner(st):
        D.compose_backward_inner(st["dy"], st["inner"], st["g"], st["wn"], s, eps,
                                 d_base=st["db"], d_lora=st["dl"], d_m=st["dm"], ws=ws_bwd)

    merge_i = [0]

    def run_merge(st):
        merge_i[0] += 1
        D.merge(st["W0"], st["A"], st["B"], st["g"], s, out=w_merged[merge_i[0] % len(w_merged)], ws=ws_merge)

    def step(st):
        run_norm(st)
        run_fwd(st)
        run_bwd(st)

    print(f"[bench] warmup {args.warmup} steps ({nsets} rotating input sets)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    # the timed region: K whole steps, device-synchronised on both sides
    ev_all = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_all[0].record(stream)
    for i in range(args.steps):
        step(sets[i % nsets])
    ev_all[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_step = ev_all[0].elapsed_time(ev_all[1]) * 1e-3 / args.steps
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    # per-call durations: each call K times back to back on the library's
    # stream (torch's current stream), HIP events around the K calls (an
    # event between every call costs a few microseconds of its own here).  A
    # spin kernel queued first, sized to outlast the host's issue of all K
    # calls, keeps the GPU from waiting on Python.
    cal = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    cal[0].record(stream)
    torch.cuda._sleep(1_000_000)
    cal[1].record(stream)
    torch.cuda.synchronize()
    ms_per_mcycle = max(cal[0].elapsed_time(cal[1]), 1e-3)
    spin = int(1_000_000 * (0.06 * args.steps + 2.0) / ms_per_mcycle)   # ~60 us of host time per call

    nbatch = 10 if args.steps >= 20 else 1   # batches: their means give p10 / p90

    def per_call(fn):
        """Mean seconds per call over K back-to-back calls, and p10 / p90 of
        the means of nbatch consecutive batches of those calls (events between
        batches only)."""
        for i in range(3):
            fn(sets[i % nsets])
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nbatch + 1)]
        torch.cuda._sleep(spin)
        ev[0].record(stream)
        for b in range(nbatch):
            for i in range(b * args.steps // nbatch, (b + 1) * args.steps // nbatch):
                fn(sets[i % nsets])
            ev[b + 1].record(stream)
        torch.cuda.synchronize()
        total = ev[0].elapsed_time(ev[nbatch]) * 1e-3 / args.steps
        per = [ev[b].elapsed_time(ev[b + 1]) * 1e-3 / ((b + 1) * args.steps // nbatch - b * args.steps // nbatch)
               for b in range(nbatch)]
        per_call.spread[fn.__name__] = (float(np.percentile(per, 10)), float(np.percentile(per, 90)),
                                        float(np.median(per)))
        return total

    per_call.spread = {}

    t_norm = per_call(run_norm)
    t_fwd = per_call(run_fwd)
    t_bwd = per_call(run_bwd)
    # the training tier (one saved activation): measured beside the step
    t_dual = per_call(run_dual)
    t_bwdi = per_call(run_bwd_inner)
    # the merge for serving: measured beside the step
    t_merge = per_call(run_merge)
    # measured ceilings (MFMA-only loops, streams, one CU's reads), same process
    from dora_adapter_factored_amd import ceilings as CL
    ceil = CL.measure(dev, full=False)
    # the same streams over arrays the size of one activation: the compose
    # kernels' fractions are taken against these (per-launch cost included)
    act = CL.streams(dev, nbytes=T * d_out * esz)
    print(f"[bench] ceilings {ceil}; at the activation size {act}", file=sys.stderr, flush=True)
    mb = merge_bytes(d_out, d_in, r, esz)
    db_, bib = compose_dual_bytes(T, d_out, esz), compose_bwd_inner_bytes(T, d_out, esz)
    F = norm_flops(d_out, d_in, r)
    nb = norm_bytes(d_out, d_in, r, esz)
    fb, bb = compose_fwd_bytes(T, d_out, esz), compose_bwd_bytes(T, d_out, esz)
    norm_tflops = F / t_norm / 1e12
    fwd_gbs, bwd_gbs = fb / t_fwd / 1e9, bb / t_bwd / 1e9
    peak_mm = PEAK_BF16_TFLOPS if dt != torch.float32 else PEAK_F32_MFMA_TFLOPS
    kern = stored_norm_kernels(spec.name)
    traced = None
    if kern:
        captured = kern.pop("captured")
        traced = {"stored": True, "source": f"profiles/kernels_{spec.name}.txt (rocprofv3 kernel trace)",
                  "captured": captured, "avg_us": kern}
        if "w0_pass" in kern:
            traced["w0_pass_TFLOPs"] = round(w0_pass_flops(d_out, d_in, r) / (kern["w0_pass"] * 1e-6) / 1e12, 1)
    traffic = stored_traffic(spec.name)

    hbm_read_ceiling = ceil["cu_read_hbm"]["chip_GBps"]
    spread = per_call.spread

    def ms_spread(name):
        lo, hi, _ = spread.get(name, (None, None, None))
        return None if lo is None else [round(lo * 1e3, 4), round(hi * 1e3, 4)]

    def ms_median(name):
        med = spread.get(name, (None, None, None))[2]
        return None if med is None else round(med * 1e3, 4)

    norm_ceiling = (ceil["mfma_32x32x16_bf16_TFLOPs"] if dt != torch.float32 else None)
    out = {
        "metric": METRIC,
        "value": round(norm_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "gpu_ms_per_step": round(gpu_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float32: "f32"}[dt],
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "config": {"workload": spec.name, "d_out": d_out, "d_in": d_in, "r": r, "tokens": T, "s": s,
                   "rotating_input_sets": nsets},
        "norm": {"ms": round(t_norm * 1e3, 4), "ms_p10_p90": ms_spread("run_norm"), "ms_median": ms_median("run_norm"), "TFLOPs": round(norm_tflops, 2),
                 "frac_mfma_peak": round(norm_tflops / peak_mm, 4),
                 "frac_measured_ceiling": (round(norm_tflops / norm_ceiling, 4) if norm_ceiling else None),
                 "frac_measured_hbm_read": round(nb / t_norm / 1e9 / hbm_read_ceiling, 4),
                 "algorithmic_flop": F,
                 "algorithmic_bytes": nb, "GBps": round(nb / t_norm / 1e9, 1),
                 "frac_hbm_peak": round(nb / t_norm / 1e9 / PEAK_HBM_GBS, 4),
                 "workspace_bytes": int(ws_norm.numel()), "kernels_traced": traced},
        "compose_fwd": {"ms": round(t_fwd * 1e3, 4), "ms_p10_p90": ms_spread("run_fwd"), "ms_median": ms_median("run_fwd"), "GBps": round(fwd_gbs, 1),
                        "frac_hbm_peak": round(fwd_gbs / PEAK_HBM_GBS, 4),
                        "frac_measured_ceiling": round(fwd_gbs / act["stream_2r1w"], 4),
                        "frac_measured_copy": round(fwd_gbs / calib["GBps"], 4), "algorithmic_bytes": fb},
        "compose_bwd": {"ms": round(t_bwd * 1e3, 4), "ms_p10_p90": ms_spread("run_bwd"), "ms_median": ms_median("run_bwd"), "GBps": round(bwd_gbs, 1),
                        "frac_hbm_peak": round(bwd_gbs / PEAK_HBM_GBS, 4),
                        "frac_measured_ceiling": round(bwd_gbs / act["stream_3r2w"], 4),
                        "frac_measured_copy": round(bwd_gbs / calib["GBps"], 4), "algorithmic_bytes": bb},
        "compose_dual": {"ms": round(t_dual * 1e3, 4), "ms_p10_p90": ms_spread("run_dual"), "ms_median": ms_median("run_dual"),
                         "GBps": round(db_ / t_dual / 1e9, 1),
                         "frac_hbm_peak": round(db_ / t_dual / 1e9 / PEAK_HBM_GBS, 4),
                         "frac_measured_ceiling": round(db_ / t_dual / 1e9 / act["stream_2r2w"], 4),
                         "algorithmic_bytes": db_},
        "compose_bwd_inner": {"ms": round(t_bwdi * 1e3, 4), "ms_p10_p90": ms_spread("run_bwd_inner"), "ms_median": ms_median("run_bwd_inner"),
                              "GBps": round(bib / t_bwdi / 1e9, 1),
                              "frac_hbm_peak": round(bib / t_bwdi / 1e9 / PEAK_HBM_GBS, 4),
                              "frac_measured_ceiling": round(bib / t_bwdi / 1e9 / act["stream_2r2w"], 4),
                              "algorithmic_bytes": bib},
        "merge": {"ms": round(t_merge * 1e3, 4), "ms_p10_p90": ms_spread("run_merge"), "ms_median": ms_median("run_merge"), "GBps": round(mb / t_merge / 1e9, 1),
                  "frac_hbm_peak": round(mb / t_merge / 1e9 / PEAK_HBM_GBS, 4),
                  "frac_measured_ceiling": round(mb / t_merge / 1e9 / ceil["stream_2r1w_GBps"], 4),
                  "algorithmic_bytes": mb, "TFLOPs": round(2 * d_out * d_in * r / t_merge / 1e12, 1)},
        "copy_calibration": calib,
        "measured_ceilings": dict({k: (round(v, 1) if isinstance(v, float) else {kk: round(vv, 1) for kk, vv in v.items()})
                                   for k, v in ceil.items()},
                                  streams_at_activation_size={"array_bytes": T * d_out * esz,
                                                              **{k + "_GBps": round(v, 1) for k, v in act.items()}}),
        "roofline": norm_roofline(F, nb, t_norm, peak_mm, traffic[0] if traffic else None),
    }
    if traffic:
        out["roofline"]["traffic_source"] = {"stored": True, "source": f"profiles/norm_traffic_{spec.name}.txt "
                                             "(rocprofv3 FETCH_SIZE + WRITE_SIZE)", "captured": traffic[1]}
    rf = out["roofline"]
    ceiling = norm_ceiling if rf["bound"] == "mfma" else hbm_read_ceiling
    rf["measured_ceiling"] = round(ceiling, 1) if ceiling else None
    rf["frac_measured_ceiling"] = round(rf["achieved"] / ceiling, 4) if ceiling else None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a row sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(layer, args.cpu_budget)
    print(json.dumps(out), flush=True)


def eager_compose_fwd(base, lora, g, s):
    """The compose as separate elementwise torch ops (the comparator the pages
    time their fused kernel against): y = base + (g - 1) * base + (g * s) * lora,
    each op a kernel over [T, d_out] in the activation dtype."""
    gb = g.to(base.dtype)
    return base + (gb - 1) * base + (gb * s) * lora


def eager_compose_bwd(dy, base, lora, g, wnorm, s, eps):
    """The backward as separate torch ops, norm detached: d_base = g dy,
    d_lora = (g s) dy, d_m = sum_t dy (base + s lora) / max(wnorm, eps)."""
    gb = g.to(dy.dtype)
    d_base = gb * dy
    d_lora = (gb * s) * dy
    d_m = (dy * (base + s * lora)).float().sum(0) / wnorm.clamp_min(eps)
    return d_base, d_lora, d_m


CROSSOVER_SHAPES = (
    # (tokens, d_out): the workloads' activation shapes ...
    (2048, 4096), (2048, 8192), (4096, 28672), (2048, 1024), (2048, 5120), (2048, 27648),
    # ... and a small-shape grid through 2048 x 6144, d_out down to 1024
    (128, 1024), (128, 4096), (512, 1024), (512, 2048), (512, 6144), (1024, 1024), (1024, 4096),
    (1024, 6144), (2048, 2048), (2048, 6144), (256, 8192), (8192, 8192),
)


def crossover_main(args, D, dev):
    """Fused compose forward / backward (this library) against the eager op
    sequence on the same GPU, per shape: time per call issued from the host,
    time per call replayed from a captured HIP graph (no host issue cost),
    and the ratios."""
    eps = D.default_eps(torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(5)
    stream = torch.cuda.current_stream(dev)
    rows = []
    for T, d_out in CROSSOVER_SHAPES:
        act = T * d_out * 2
        nsets = max(2, int(np.ceil(2 * MALL_BYTES / (5 * act))) + 1) if 5 * act < 2 * MALL_BYTES else 2
        nsets = min(nsets, 64)
        sets = []
        for _ in range(nsets):
            mk = lambda: torch.randn(T, d_out, device=dev, generator=gen).to(torch.bfloat16)  # noqa: E731
            sets.append(dict(base=mk(), lora=mk(), dy=mk(), y=torch.empty(T, d_out, dtype=torch.bfloat16, device=dev),
                             db=torch.empty(T, d_out, dtype=torch.bfloat16, device=dev),
                             dl=torch.empty(T, d_out, dtype=torch.bfloat16, device=dev),
                             dm=torch.empty(d_out, device=dev)))
        g = 1 + 1e-3 * torch.randn(d_out, device=dev, generator=gen)
        wn = 1 + 1e-3 * torch.randn(d_out, device=dev, generator=gen)
        ws = torch.empty(max(1, D.compose_backward_workspace_size(T, d_out)), dtype=torch.uint8, device=dev)
        s = 1.0
        fns = {
            "fused_fwd": lambda st: D.compose(st["base"], st["lora"], g, s, out=st["y"]),
            "eager_fwd": lambda st: eager_compose_fwd(st["base"], st["lora"], g, s),
            "fused_bwd": lambda st: D.compose_backward(st["dy"], st["base"], st["lora"], g, wn, s, eps,
                                                       d_base=st["db"], d_lora=st["dl"], d_m=st["dm"], ws=ws),
            "eager_bwd": lambda st: eager_compose_bwd(st["dy"], st["base"], st["lora"], g, wn, s, eps),
        }
        reps = max(20, min(400, int(2e9 / act)))
        res = {}
        for name, fn in fns.items():
            # issued from the host, call after call (what a framework sees)
            for i in range(3):
                fn(sets[i % nsets])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(1_000_000 * reps * 0.08))   # covers the host's issue of all reps calls
            e0.record(stream)
            for i in range(reps):
                fn(sets[i % nsets])
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / reps   # us per call
            # replayed from one captured HIP graph of 20 calls (the GPU's time alone)
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for i in range(3):
                    fn(sets[i % nsets])
            stream.wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(20):
                    fn(sets[i % nsets])
            graph.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(10):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            res[name + "_graph"] = e0.elapsed_time(e1) * 1e3 / 200
            del graph
        rows.append({"tokens": T, "d_out": d_out, **{k: round(v, 2) for k, v in res.items()},
                     "fwd_speedup": round(res["eager_fwd"] / res["fused_fwd"], 2),
                     "bwd_speedup": round(res["eager_bwd"] / res["fused_bwd"], 2),
                     "fwd_speedup_graph": round(res["eager_fwd_graph"] / res["fused_fwd_graph"], 2),
                     "bwd_speedup_graph": round(res["eager_bwd_graph"] / res["fused_bwd_graph"], 2)})
        print(f"[crossover] {rows[-1]}", file=sys.stderr, flush=True)
        del sets, ws
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "fused compose vs eager op sequence, us per call (bf16, one MI355X)",
                      "rows": rows}), flush=True)


def library_main(args, D, dev):
    """Context, not a target: the vendor GEMM library (hipBLASLt, reached
    through torch.mm / torch.addmm) on pieces of the same work, beside this
    library's whole calls.  The norm's dominant contraction W0 A^T alone
    (no base term, no Gram term, no row dots), the Gram A A^T alone, and the
    merge as the two-op eager sequence g * addmm(W0, B, A, alpha = s).
    Rotating input copies keep every timed loop past twice the MALL; the
    calls alternate between the two sides in four batches and the best
    batch's mean is reported."""
    stream = torch.cuda.current_stream(dev)
    rows = []
    for cfg in (3, 4):
        spec = DI.CONFIGS[cfg]
        d_out, d_in, r, s = spec.d_out, spec.d_in, spec.r, spec.s
        layer = DI.make_layer(spec, DI.config_seed(cfg), device=dev, activations=False)
        dt = layer.W0.dtype
        eps = D.default_eps(dt)
        nb = (d_out * d_in + r * (d_in + d_out)) * layer.W0.element_size()
        nsets = max(2, int(np.ceil(2 * MALL_BYTES / nb)) + 1)
        sets = [dict(W0=layer.W0, A=layer.A, B=layer.B, m=layer.m)]
        sets += [dict(W0=layer.W0.clone(), A=layer.A.clone(), B=layer.B.clone(), m=layer.m.clone())
                 for _ in range(nsets - 1)]
        for st in sets:
            st["wn"], st["g"] = torch.empty(d_out, device=dev), torch.empty(d_out, device=dev)
        ws_norm = torch.empty(D.norm_workspace_size(d_out, d_in, r, dt), dtype=torch.uint8, device=dev)
        ws_merge = torch.empty(D.merge_workspace_size(d_in, r, dt), dtype=torch.uint8, device=dev)
        w_out = torch.empty_like(layer.W0)
        fns = {
            "norm": lambda st: D.factored_norm(st["W0"], st["A"], st["B"], s, st["m"], eps, wnorm=st["wn"],
                                               g=st["g"], ws=ws_norm),
            "lib_mm_W0_At": lambda st: torch.mm(st["W0"], st["A"].t()),
            "lib_mm_A_At": lambda st: torch.mm(st["A"], st["A"].t()),
            "merge": lambda st: D.merge(st["W0"], st["A"], st["B"], st["g"], s, out=w_out, ws=ws_merge),
            "lib_eager_merge": lambda st: torch.addmm(st["W0"], st["B"], st["A"], alpha=s).mul_(
                st["g"].to(dt).unsqueeze(1)),
        }
        fns["norm"](sets[0])   # g for the merges
        for st in sets[1:]:
            st["g"].copy_(sets[0]["g"])
        reps = 40
        best = {k: float("inf") for k in fns}
        for trial in range(4):
            for name, fn in fns.items():
                for i in range(3):
                    fn(sets[i % nsets])
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(int(2e7))
                e0.record(stream)
                for i in range(reps):
                    fn(sets[i % nsets])
                e1.record(stream)
                torch.cuda.synchronize()
                best[name] = min(best[name], e0.elapsed_time(e1) * 1e3 / reps)
        mm = 2.0 * d_out * d_in * r
        row = {"workload": spec.name, **{k + "_us": round(v, 1) for k, v in best.items()},
               "norm_TFLOPs": round(norm_flops(d_out, d_in, r) / best["norm"] / 1e6, 1),
               "lib_mm_W0_At_TFLOPs": round(mm / best["lib_mm_W0_At"] / 1e6, 1),
               "lib_mm_A_At_TFLOPs": round(2.0 * r * r * d_in / best["lib_mm_A_At"] / 1e6, 1),
               "merge_TFLOPs": round(mm / best["merge"] / 1e6, 1),
               "lib_eager_merge_TFLOPs": round(mm / best["lib_eager_merge"] / 1e6, 1)}
        rows.append(row)
        print(f"[library] {row}", file=sys.stderr, flush=True)
        del sets, ws_norm, ws_merge, w_out, layer
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "this library's norm and merge beside the vendor GEMM library on pieces of the "
                                "same work, us per call (bf16, one MI355X)", "rows": rows}), flush=True)


SWEEP_METRIC = "many-module sweep: norm + compose fwd/bwd ms per step (64 layers x 7 projections, r=384 bf16)"


def sweep_main(args, D, dev):
    """The many-module sweep: 64 layers x 7 adapted projections, every
    module's weights resident; a step is every layer's norms (all seven
    projections in one grouped call) and compose forward and backward of
    every module, in model order.
    Activations are pooled per shape, two rotating copies."""
    nl, npj = DI.SWEEP_LAYERS, len(DI.SWEEP_PROJECTIONS)
    T, r = DI.SWEEP_T, DI.SWEEP_R
    print(f"[bench] generating {nl} x {npj} modules on the device", file=sys.stderr, flush=True)
    layers = []
    for li in range(nl):
        mods = []
        for pj in range(npj):
            L = DI.make_layer(DI.sweep_spec(pj), DI.sweep_seed(li, pj), device=dev, activations=False,
                              gen_device="cuda")
            L.wn = torch.empty(L.spec.d_out, device=dev)
            L.g = torch.empty(L.spec.d_out, device=dev)
            mods.append(L)
        layers.append(mods)
    torch.cuda.synchronize()
    weight_bytes = sum(L.W0.numel() * 2 + L.A.numel() * 2 + L.B.numel() * 2 for mods in layers for L in mods)
    gen = torch.Generator(device=dev).manual_seed(77)
    pool = {}
    for _, d_out, _ in DI.SWEEP_PROJECTIONS:
        if d_out in pool:
            continue
        sets = []
        for _ in range(2):
            mk = lambda: torch.randn(T, d_out, device=dev, generator=gen).to(torch.bfloat16)  # noqa: E731
            sets.append(dict(base=mk(), lora=mk(), dy=mk(), y=torch.empty(T, d_out, dtype=torch.bfloat16, device=dev),
                             db=torch.empty(T, d_out, dtype=torch.bfloat16, device=dev),
                             dl=torch.empty(T, d_out, dtype=torch.bfloat16, device=dev),
                             dm=torch.empty(d_out, device=dev)))
        pool[d_out] = sets
    grp = list(range(npj))      # every projection of a layer in one grouped call
    ws_group = torch.empty(D.norm_group_workspace_size([DI.SWEEP_PROJECTIONS[j][1] for j in grp],
                                                       [DI.SWEEP_PROJECTIONS[j][2] for j in grp], r,
                                                       torch.bfloat16), dtype=torch.uint8, device=dev)
    ws_single = torch.empty(max(D.norm_workspace_size(d_out, d_in, r, torch.bfloat16)
                                for _, d_out, d_in in DI.SWEEP_PROJECTIONS), dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(max(D.compose_backward_workspace_size(T, d_out) for _, d_out, _ in DI.SWEEP_PROJECTIONS),
                         dtype=torch.uint8, device=dev)
    eps = D.default_eps(torch.bfloat16)
    stream = torch.cuda.current_stream(dev)

    def norms(mods, grouped):
        if grouped:
            D.factored_norm_group([(mods[j].W0, mods[j].A, mods[j].B, mods[j].spec.s, mods[j].m) for j in grp],
                                  eps, outs=[(mods[j].wn, mods[j].g) for j in grp], ws=ws_group)
            rest = [j for j in range(npj) if j not in grp]
        else:
            rest = range(npj)
        for j in rest:
            L = mods[j]
            D.factored_norm(L.W0, L.A, L.B, L.spec.s, L.m, eps, wnorm=L.wn, g=L.g, ws=ws_single)

    def composes(mods, it):
        for L in mods:
            st = pool[L.spec.d_out][it % 2]
            D.compose(st["base"], st["lora"], L.g, L.spec.s, out=st["y"])
            D.compose_backward(st["dy"], st["base"], st["lora"], L.g, L.wn, L.spec.s, eps, d_base=st["db"],
                               d_lora=st["dl"], d_m=st["dm"], ws=ws_bwd)

    # Two-stream schedule: the norms depend on the weights alone, so every
    # layer's grouped norm is issued on a side stream and each layer's
    # compose (main stream) waits only for its own layer's norm.  The side
    # stream first waits for everything already on the main stream, so a
    # step's norms never overwrite g and wnorm that the previous step's
    # composes still read.  Both streams keep the default priority.
    side = torch.cuda.Stream(dev)
    norm_done = [torch.cuda.Event() for _ in range(nl)]

    def step(it, grouped=True, do_norm=True, do_compose=True, overlap=False):
        if overlap and do_norm and do_compose:
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for li, mods in enumerate(layers):
                    norms(mods, grouped)
                    norm_done[li].record(side)
            for li, mods in enumerate(layers):
                stream.wait_event(norm_done[li])
                composes(mods, it)
            return
        for mods in layers:
            if do_norm:
                norms(mods, grouped)
            if do_compose:
                composes(mods, it)

    def timed(k, **kw):
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(k):
            step(i, **kw)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / k, ev[0].elapsed_time(ev[1]) * 1e-3 / k

    steps = args.steps if args.steps_given else 10
    warm = args.warmup if args.warmup_given else 2
    print(f"[bench] sweep warmup {warm}, timing {steps} steps", file=sys.stderr, flush=True)
    for i in range(warm):
        step(i)
        step(i, overlap=True)
    wall_s, gpu_s = timed(steps)
    wall_o, gpu_o = timed(steps, overlap=True)
    overlap = not args.sweep_serial and gpu_o < gpu_s
    wall, gpu = (wall_o, gpu_o) if overlap else (wall_s, gpu_s)
    k2 = max(2, min(steps, 5))
    _, t_norm_g = timed(k2, do_compose=False)
    _, t_norm_s = timed(k2, grouped=False, do_compose=False)
    _, t_comp = timed(k2, do_norm=False)
    F = nl * sum(norm_flops(d_out, d_in, r) for _, d_out, d_in in DI.SWEEP_PROJECTIONS)
    cbytes = nl * sum(compose_fwd_bytes(T, d_out, 2) + compose_bwd_bytes(T, d_out, 2)
                      for _, d_out, _ in DI.SWEEP_PROJECTIONS)
    per_module_ws = {f"{n}-{d_out}x{d_in}": D.norm_workspace_size(d_out, d_in, r, torch.bfloat16)
                     for n, d_out, d_in in DI.SWEEP_PROJECTIONS}
    out = {
        "metric": SWEEP_METRIC,
        "value": round(gpu * 1e3, 3),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(wall * 1e3, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "config": {"workload": "sweep-64x7-r384-bf16", "layers": nl, "projections": [p[0] for p in
                   DI.SWEEP_PROJECTIONS], "tokens": T, "r": r, "weights_resident_bytes": weight_bytes},
        "sweep": {
            "schedule": "two streams (norms on a side stream, each layer's compose after its norm)" if overlap
                        else "one stream, layer by layer",
            "step_ms_one_stream": round(gpu_s * 1e3, 3),
            "step_ms_two_streams": round(gpu_o * 1e3, 3),
            "norm_ms_per_step_grouped": round(t_norm_g * 1e3, 3),
            "norm_ms_per_step_one_by_one": round(t_norm_s * 1e3, 3),
            "norm_TFLOPs_grouped": round(F / t_norm_g / 1e12, 1),
            "compose_ms_per_step": round(t_comp * 1e3, 3),
            "compose_GBps": round(cbytes / t_comp / 1e9, 1),
            "norm_workspace_bytes_per_module": per_module_ws,
            "norm_workspace_bytes_group": int(ws_group.numel()),
            "compose_bwd_workspace_bytes_max": int(ws_bwd.numel()),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a row sample of one layer", file=sys.stderr, flush=True)
        out["cpu_baseline"] = sweep_cpu_baseline(layers[0], args.cpu_budget)
    print(json.dumps(out), flush=True)


def sweep_cpu_baseline(mods, budget_s=12.0):
    """The oracle on a row and token sample of one layer of the sweep,
    extrapolated to a whole step (64 layers)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    per = budget_s / len(mods)
    total, parts = 0.0, []
    for L in mods:
        spec = L.spec
        W0, A, B = L.W0.cpu(), L.A.cpu(), L.B.cpu()
        rows_done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.8 * per and rows_done < spec.d_out:
            rows = np.arange(rows_done, min(spec.d_out, rows_done + 128))
            oracle.dense_row_norm(W0, A, B, spec.s, rows=rows)
            rows_done += rows.size
        t_norm = (time.perf_counter() - t0) * spec.d_out / rows_done
        tok = 64
        x = np.random.default_rng(0).standard_normal((tok, spec.d_out))
        g = np.ones(spec.d_out)
        t1 = time.perf_counter()
        oracle.compose_forward(x, x, g, spec.s)
        oracle.compose_backward(x, x, x, g, g, spec.s, 1e-7)
        t_comp = (time.perf_counter() - t1) * DI.SWEEP_T / tok
        total += t_norm + t_comp
        parts.append(f"{spec.name}: {rows_done} rows, {tok} tokens")
    return {"value": round(total * DI.SWEEP_LAYERS * 1e3, 1), "unit": "ms/step (extrapolated)",
            "cores": int(threads), "kind": "oracle",
            "sample": "one layer, row and token samples, scaled to 64 layers: " + "; ".join(parts),
            "cpu": _cpu_model()}


if __name__ == "__main__":
    main()
