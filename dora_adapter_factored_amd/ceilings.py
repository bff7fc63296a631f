"""Measured ceilings of the operations the DoRA kernels are built from.

Binding of libdora_ceilings.so (measurement-only kernels, not part of the
DoRA library's ABI).  Every figure is timed with HIP events on the current
stream, several launches back to back after a warm-up:

  mfma_32x32x16_bf16, mfma_16x16x32_bf16   TFLOP/s of MFMA-only loops (operands
                                           in registers, 8 waves x 192 accumulators
                                           per CU, one workgroup per CU)
  stream_2r1w, stream_2r2w, stream_3r2w    GB/s of 16-byte streams in the compose
                                           forward, dual forward / backward from
                                           (dy, inner), backward access patterns
                                           (the best of a blocked and a
                                           grid-stride form)
  cu_read_l2, cu_read_hbm                  GB/s one CU reads (all workgroups read
                                           one L2-resident region / each its own),
                                           and the whole chip's sum
  w0_stream, w0_stream_with_a              GB/s of the W0 pass's access pattern
  (w0_stream_with_a_tiled)                 (256 x 64-byte row pieces per k-tile
                                           through a 4-stage LDS-DMA ring, one
                                           barrier per tile) without MFMA, W0 alone
                                           and with the 384-row A tile per k-tile
                                           (A row-major, or k-tile-major so that
                                           each tile is one contiguous run)
  (w0_stream_with_a_7chunks)               the row-major pattern in seven K-chunks
                                           on 224 workgroups: 8/7 the k-tiles per
                                           CU, the same bytes per XCD
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdora_ceilings.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run `python -m dora_adapter_factored_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.dora_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
        lib.dora_ceiling_stream.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, ctypes.c_int, vp]
        lib.dora_ceiling_cu_read.argtypes = [vp, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
        lib.dora_ceiling_w0_stream.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, vp, vp]
        for f in (lib.dora_ceiling_mfma, lib.dora_ceiling_stream, lib.dora_ceiling_cu_read,
                  lib.dora_ceiling_w0_stream):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _time(fn, reps, warm=3):
    """Seconds per call of fn (HIP events around reps back-to-back calls)."""
    for _ in range(warm):
        fn()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def mfma(dev, kind: int, iters: int = 4000, workgroups: int = 256) -> float:
    """TFLOP/s of the MFMA-only loop (kind 0: 32x32x16, 1: 16x16x32 bf16)."""
    lib = load()
    out = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def run():
        _check(lib.dora_ceiling_mfma(kind, iters, workgroups, _p(out), st), "mfma")

    t = _time(run, 5)
    # a 128 x 96 wave tile per step: K = 16 (32x32x16) or K = 32 (16x16x32)
    flop = workgroups * 8 * iters * 2 * 128 * 96 * (16 if kind == 0 else 32)
    return flop / t / 1e12


def streams(dev, nbytes: int = 256 << 20, forms=(0, 4096)) -> dict:
    """GB/s of the 2-read/1-write, 2-read/2-write and 3-read/2-write streams
    over arrays of nbytes: the best of the blocked form (workgroups 0: one
    workgroup per 4 packets per thread, all loads issued before the stores)
    and a grid-stride form with 4096 workgroups.  Back-to-back launches cycle
    through enough sets of arrays to touch more than twice the 256 MB MALL,
    so small arrays are read from HBM, as the bench's rotating inputs are."""
    lib = load()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    nsets = max(1, -(-2 * (256 << 20) // (5 * nbytes)) + 1)
    sets = [[torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(5)] for _ in range(nsets)]
    out = {}
    for name, pattern, moved, has_c, has_z in (("stream_2r1w", 0, 3, False, False), ("stream_2r2w", 2, 4, False, True),
                                               ("stream_3r2w", 1, 5, True, True)):
        best = 0.0
        for wg in forms:
            i = [0]

            def run():
                a, b, c, y, z = sets[i[0] % nsets]
                i[0] += 1
                _check(lib.dora_ceiling_stream(pattern, _p(a), _p(b), _p(c) if has_c else None, _p(y),
                                               _p(z) if has_z else None, nbytes, wg, st), "stream")
            best = max(best, moved * nbytes / _time(run, max(10, 2 * nsets)) / 1e9)
        out[name] = best
    del sets
    return out


def cu_read(dev, bytes_per_wg: int = 256 << 10, workgroups: int = 256) -> dict:
    """GB/s per CU and for the chip: every workgroup reading one L2-resident
    region (stride 0), and each its own region (from HBM)."""
    lib = load()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    buf = torch.ones(workgroups * bytes_per_wg // 4, dtype=torch.int32, device=dev)
    out = torch.empty(workgroups * 512, dtype=torch.int32, device=dev)
    res = {}
    for name, stride, reps in (("cu_read_l2", 0, 8), ("cu_read_hbm", bytes_per_wg, 1)):
        def run():
            _check(lib.dora_ceiling_cu_read(_p(buf), bytes_per_wg, stride, reps, workgroups, 8, _p(out), st), "cu_read")
        t = _time(run, 10)
        per_cu = bytes_per_wg * reps / t / 1e9
        res[name] = {"per_cu_GBps": per_cu, "chip_GBps": per_cu * workgroups}
    del buf, out
    return res


def w0_stream(dev, d_out: int = 8192, d_in: int = 8192, r: int = 384) -> dict:
    """GB/s of the W0 pass's access pattern without MFMA: W0 bytes per second
    (and W0 + A bytes when the A tiles are moved too)."""
    lib = load()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    sets = [(torch.randn(d_out, d_in, device=dev).to(torch.bfloat16), torch.randn(r, d_in, device=dev).to(torch.bfloat16))
            for _ in range(3)]
    out = torch.empty(256 * 512, dtype=torch.int32, device=dev)
    res = {}
    modes = [("w0_stream", 0), ("w0_stream_with_a", 1), ("w0_stream_with_a_tiled", 2)]
    if d_out == 32 * 256:
        modes.append(("w0_stream_with_a_7chunks", 3))   # same bytes per XCD, 224 workgroups
    for name, with_a in modes:
        i = [0]

        def run():
            W0, A = sets[i[0] % len(sets)]
            i[0] += 1
            _check(lib.dora_ceiling_w0_stream(_p(W0), _p(A), d_out, d_in, r, with_a, _p(out), st), "w0_stream")
        t = _time(run, 12)
        w0b = d_out * d_in * 2
        # each of the 32 row tiles moves the 384-row A tile of every k-tile
        ab = 32 * 384 * d_in * 2 if with_a else 0
        res[name] = {"us": t * 1e6, "W0_GBps": w0b / t / 1e9, "moved_GBps": (w0b + ab) / t / 1e9}
    del sets, out
    return res


def measure(dev, full: bool = True) -> dict:
    """The ceilings the bench line's fractions are taken against (full: every probe)."""
    res = {"mfma_32x32x16_bf16_TFLOPs": mfma(dev, 0)}
    res.update({k + "_GBps": v for k, v in streams(dev).items()})
    res.update(cu_read(dev))
    if full:
        res["mfma_16x16x32_bf16_TFLOPs"] = mfma(dev, 1)
        res.update(w0_stream(dev))
    return res
