"""Host checks of the large-tile W0 pass's balanced K split (csrc/dora_balance.h).

The header is compiled by the host C++ compiler with __host__ / __device__
defined empty.  For each plan shape, every workgroup's segments are listed and
checked: each (m-tile, k-tile) unit is walked by exactly one segment, the
slots of each m-tile are exactly 0 .. slots(mt) - 1 (each written once, so the
assembly reads no stale partial), and segments are non-empty.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dora_adapter_factored_amd", "csrc")

CHECKER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "dora_balance.h"
using namespace dora;
int main(int argc, char** argv) {
    const int n_mt = atoi(argv[1]), nkt = atoi(argv[2]), nwg = atoi(argv[3]);
    const Balance b{(int64_t)n_mt * nkt, nwg, nkt};
    std::vector<int> walked((size_t)n_mt * nkt, 0);
    std::vector<std::vector<int>> slot_hits(n_mt);
    int most = 0, max_segs = 0, bad = 0;
    for (int mt = 0; mt < n_mt; ++mt) {
        slot_hits[mt].assign(b.slots(mt), 0);
        if (b.slots(mt) > most) most = b.slots(mt);
    }
    for (int id = 0; id < nwg; ++id) {
        int segs = 0;
        balance_segments(b, id, [&](const BalanceSeg& s) {
            ++segs;
            if (s.mt < 0 || s.mt >= n_mt || s.kt_begin < 0 || s.kt_end > nkt || s.kt_begin >= s.kt_end) { ++bad; return; }
            for (int k = s.kt_begin; k < s.kt_end; ++k) walked[(size_t)s.mt * nkt + k] += 1;
            if (s.slot < 0 || s.slot >= (int)slot_hits[s.mt].size()) { ++bad; return; }
            slot_hits[s.mt][s.slot] += 1;
        });
        if (segs > max_segs) max_segs = segs;
    }
    for (int v : walked) bad += v != 1;
    for (auto& h : slot_hits) for (int v : h) bad += v != 1;
    printf("%d %d %d\n", bad, most, max_segs);
    return 0;
}
"""


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("balance")
    src, exe = d / "check.cpp", d / "check"
    src.write_text(CHECKER)
    subprocess.run([cxx, "-std=c++17", "-O1", "-D__host__=", "-D__device__=", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True)

    def run(n_mt, nkt, nwg):
        out = subprocess.run([str(exe), str(n_mt), str(nkt), str(nwg)], check=True, capture_output=True,
                             text=True).stdout.split()
        return tuple(int(x) for x in out)

    return run


# (m-tiles, k-tiles per m-tile): the 28672 x 8192, 36864 x 8192 and
# 28672 x 16384 r = 384 plans, and ragged shapes, all with at least one unit
# per workgroup (the plan's condition for this split)
SHAPES = [(112, 134), (144, 134), (112, 262), (113, 135), (9, 61), (8, 64), (127, 257), (64, 70), (1, 256)]


@pytest.mark.parametrize("n_mt,nkt", SHAPES)
def test_balance_covers_every_unit_once(checker, n_mt, nkt):
    bad, most, max_segs = checker(n_mt, nkt, 256)
    assert bad == 0
    assert most >= 1 and max_segs >= 1


def test_balance_two_segments_per_workgroup(checker):
    # 28672 x 8192: each range is shorter than one m-tile's K, so it meets
    # two m-tiles at most, and an m-tile has at most four partial slots
    bad, most, max_segs = checker(112, 134, 256)
    assert bad == 0 and max_segs <= 2 and most <= 4
