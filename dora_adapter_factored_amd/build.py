"""Build the HIP library libdora_mi355x.so in-tree for gfx950.

    python -m dora_adapter_factored_amd.build

Each .hip source is compiled to an object under _build/ (in parallel), then
linked into dora_adapter_factored_amd/libdora_mi355x.so.  hipcc cross-compiles,
so this works on a host without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libdora_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ("dora_capi.hip", "compose.hip", "norm.hip", "merge.hip")
# measurement-only kernels (bench.py --ceilings), a library of their own
CEILINGS_LIB_PATH = os.path.join(PKG, "libdora_ceilings.so")
CEILINGS_SOURCES = ("ceilings.hip",)
ARCH = "gfx950"

# Packed-fp32 VALU ops are kept out of the device code.  MFMA results are
# kept in VGPR form: with the large accumulator tiles of the W0 pass the
# default heuristics otherwise shuttle accumulators between AGPRs and VGPRs
# every k-tile and spill to scratch; in VGPR form AGPRs only serve as spill
# space and nothing reaches scratch memory.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the DoRA library needs ROCm's hipcc to build")
    return exe


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source and link the shared libraries (the DoRA library
    and the measurement-only ceilings library); returns the DoRA library's
    path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags)
    objs, cmds = {}, []
    for src in SOURCES + CEILINGS_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs[src] = obj
        cmds.append([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    for path, srcs in ((LIB_PATH, SOURCES), (CEILINGS_LIB_PATH, CEILINGS_SOURCES)):
        tmp = path + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *(objs[s] for s in srcs)])
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
