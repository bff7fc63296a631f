// Balanced K split of the large-tile W0 pass: which (m-tile, k-tile) units
// a workgroup walks, and which partial slot each of its segments writes.
//
// Host and device code (plan, kernel, assembly) share these functions; the
// header needs no HIP declarations beyond __host__ / __device__, so a host
// compiler can build it with those defined empty.
#pragma once

#include <stdint.h>

namespace dora {

// Workgroup w of nwg owns units [w U / nwg, (w + 1) U / nwg) of the
// m-tile-major sequence of all (m-tile, k-tile) pairs, U = units =
// n_mtiles * nkt.  The plan takes this split only where every workgroup
// owns at least one unit (U >= nwg), so the workgroups meeting one m-tile
// are consecutive and each holds some of its units: its partials go to slot
// w - (first workgroup of the m-tile), and the slots of an m-tile are dense.
// nwg = 0: the uniform split.
struct Balance {
    int64_t units;   // all units
    int nwg, nkt;    // workgroups; k-tiles per m-tile

    // the workgroup whose range holds unit u
    __host__ __device__ int wg_of(int64_t u) const { return (int)(((u + 1) * nwg + units - 1) / units) - 1; }
    // partial slots of m-tile mt (workgroups whose ranges meet it)
    __host__ __device__ int slots(int mt) const {
        return wg_of((int64_t)(mt + 1) * nkt - 1) - wg_of((int64_t)mt * nkt) + 1;
    }
};

// One segment of a workgroup's walk: k-tiles [kt_begin, kt_end) of m-tile
// mt, partials to slot.
struct BalanceSeg {
    int mt, kt_begin, kt_end, slot;
};

// Calls f(seg) for each segment of workgroup id, in walk order: one, or two
// where the range crosses an m-tile boundary (a range is shorter than one
// m-tile's K when the plan takes this split).
template <typename F>
__host__ __device__ inline void balance_segments(const Balance& b, int id, F&& f) {
    const int64_t u0 = (int64_t)id * b.units / b.nwg, u1 = (int64_t)(id + 1) * b.units / b.nwg;
    for (int64_t u = u0; u < u1;) {
        const int mt = (int)(u / b.nkt);
        const int64_t t0 = (int64_t)mt * b.nkt, e = u1 < t0 + b.nkt ? u1 : t0 + b.nkt;
        f(BalanceSeg{mt, (int)(u - t0), (int)(e - t0), id - b.wg_of(t0)});
        u = e;
    }
}

}  // namespace dora
