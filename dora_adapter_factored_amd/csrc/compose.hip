// Fused DoRA compose, forward and backward, for gfx950.
//
// Forward ("Scaling DoRA", §3 compose kernel and Data Availability contract):
//   y = base + ((g - 1) * base + (g * s) * lora)      (delta_only drops base)
// in fp32 with one rounding to the activation dtype; 2 reads + 1 write per
// element.  Backward (§3 backward kernel, norm detached):
//   d_base = g * dy (delta_only: (g - 1) * dy),  d_lora = (g * s) * dy,
//   d_m_j  = sum_t dy_tj * (base_tj + s * lora_tj) / max(wnorm_j, eps)
// with d_m reduced in a fixed order: per-token-block partial sums written to
// the workspace, then one finalize pass.  No atomics, so d_m is bitwise
// reproducible.
//
// Training tier (§4, Tier 1): the dual-output forward also writes
// inner = base + s * lora (2 reads + 2 writes), and the backward can take
// (dy, inner) instead of (dy, base, lora): d_m_j = sum_t dy_tj * inner_tj /
// max(wnorm_j, eps), 2 reads + 2 writes.
//
// Both kernels are HBM-bound streams over [T, d_out].  A workgroup owns a
// strip of 64 sixteen-byte packets along d_out (one wave reads 1 KiB of a
// row) and 4 row lanes; each thread keeps g for its packet in registers for
// the whole strip and walks rows, with several rows' loads in flight before
// the first store.
#include "dora_device.h"
#include "dora_gfx950.h"
#include "dora_launch.h"

namespace dora {
namespace {

constexpr int kThreads = 256;
constexpr int kTC = 64;          // packets along d_out per workgroup
constexpr int kTR = 4;           // row lanes per workgroup
constexpr int kMaxParts = 1024;  // cap on d_m partial rows (grid-strides beyond)
// Rows per thread per step (loads in flight) and rows per d_m partial are
// template parameters chosen per shape from measurements on MI355X: wide
// activations run fastest with more, smaller workgroups (RPT 2 forward,
// 16-row token blocks backward), narrow ones with more rows in flight.
constexpr int kMaxGridY = 65535;

template <typename T, bool DELTA, int kRPT, bool DUAL>
__global__ __launch_bounds__(kThreads) void compose_fwd_vec(const T* base, const T* lora,
                                                            const float* __restrict__ g, float s,
                                                            int64_t nrows, int64_t d_out, T* y, T* inner) {
    constexpr int N = Pack<T>::N;
    constexpr int kFwdRowsPerBlock = kTR * kRPT;
    const int tc = threadIdx.x % kTC, tr = threadIdx.x / kTC;
    const int64_t col = ((int64_t)blockIdx.x * kTC + tc) * N;
    if (col >= d_out) return;
    float gm1[N], gs[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float gv = g[col + e];
        gm1[e] = gv - 1.0f;
        gs[e] = gv * s;
    }
    for (int64_t rb = blockIdx.y; rb * kFwdRowsPerBlock < nrows; rb += gridDim.y) {
        const int64_t r0 = rb * kFwdRowsPerBlock + tr;
        Pack<T> b[kRPT], l[kRPT];
#pragma unroll
        for (int i = 0; i < kRPT; ++i) {
            const int64_t row = r0 + (int64_t)i * kTR;
            if (row < nrows) {
                b[i] = load_pack_stream(base + row * d_out + col);
                l[i] = load_pack_stream(lora + row * d_out + col);
            }
        }
#pragma unroll
        for (int i = 0; i < kRPT; ++i) {
            const int64_t row = r0 + (int64_t)i * kTR;
            if (row < nrows) {
                Pack<T> o, in;
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float bf = Cvt<T>::to_f(b[i].e[e]);
                    const float lf = Cvt<T>::to_f(l[i].e[e]);
                    const float d = fmaf(gm1[e], bf, gs[e] * lf);
                    o.e[e] = Cvt<T>::from_f(DELTA ? d : bf + d);
                    if (DUAL) in.e[e] = Cvt<T>::from_f(fmaf(s, lf, bf));
                }
                store_pack_stream(y + row * d_out + col, o);
                if (DUAL) store_pack_stream(inner + row * d_out + col, in);
            }
        }
    }
}

template <typename T, bool DELTA, bool DUAL>
__global__ __launch_bounds__(kThreads) void compose_fwd_scalar(const T* base, const T* lora,
                                                               const float* __restrict__ g, float s,
                                                               int64_t n, int64_t d_out, T* y, T* inner) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kThreads) {
        const float gv = g[i % d_out];
        const float bf = Cvt<T>::to_f(base[i]);
        const float lf = Cvt<T>::to_f(lora[i]);
        const float d = fmaf(gv - 1.0f, bf, (gv * s) * lf);
        y[i] = Cvt<T>::from_f(DELTA ? d : bf + d);
        if (DUAL) inner[i] = Cvt<T>::from_f(fmaf(s, lf, bf));
    }
}

// With INNER, `base` points at inner = base + s * lora and lora is unused.
template <typename T, bool DELTA, bool DM, bool DB, bool DL, int kRPT, int kBwdTokenBlock, bool INNER>
__global__ __launch_bounds__(kThreads) void compose_bwd_vec(const T* dy, const T* __restrict__ base,
                                                            const T* __restrict__ lora,
                                                            const float* __restrict__ g, float s,
                                                            int64_t nrows, int64_t d_out, T* d_base,
                                                            T* d_lora, float* __restrict__ dm_part) {
    constexpr int N = Pack<T>::N;
    static_assert(kBwdTokenBlock % (kTR * kRPT) == 0, "token block is whole steps");
    constexpr int kSteps = kBwdTokenBlock / (kTR * kRPT);
    // d_m partials of row lanes 1 .. kTR - 1, element-major: lane tc of a
    // wave writes and reads consecutive words (no bank conflicts)
    __shared__ float red[kTR - 1][N][kTC];
    const int tc = threadIdx.x % kTC, tr = threadIdx.x / kTC;
    const int64_t col = ((int64_t)blockIdx.x * kTC + tc) * N;
    const bool active = col < d_out;
    float gb[N], gl[N], acc[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float gv = active ? g[col + e] : 0.0f;
        gb[e] = DELTA ? gv - 1.0f : gv;
        gl[e] = gv * s;
        acc[e] = 0.0f;
    }
    if (active) {
        for (int64_t rb = blockIdx.y; rb * kBwdTokenBlock < nrows; rb += gridDim.y) {
#pragma unroll
            for (int st = 0; st < kSteps; ++st) {
                const int64_t r0 = rb * kBwdTokenBlock + st * (kTR * kRPT) + tr;
                Pack<T> dv[kRPT], bv[kRPT], lv[kRPT];
#pragma unroll
                for (int i = 0; i < kRPT; ++i) {
                    const int64_t row = r0 + (int64_t)i * kTR;
                    if (row < nrows) {
                        const int64_t off = row * d_out + col;
                        dv[i] = load_pack_stream(dy + off);
                        if (DM) {
                            bv[i] = load_pack_stream(base + off);
                            if (!INNER) lv[i] = load_pack_stream(lora + off);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < kRPT; ++i) {
                    const int64_t row = r0 + (int64_t)i * kTR;
                    if (row < nrows) {
                        const int64_t off = row * d_out + col;
                        Pack<T> ob, ol;
#pragma unroll
                        for (int e = 0; e < N; ++e) {
                            const float df = Cvt<T>::to_f(dv[i].e[e]);
                            if (DB) ob.e[e] = Cvt<T>::from_f(gb[e] * df);
                            if (DL) ol.e[e] = Cvt<T>::from_f(gl[e] * df);
                            if (DM) {
                                const float inner = INNER ? Cvt<T>::to_f(bv[i].e[e])
                                                          : fmaf(s, Cvt<T>::to_f(lv[i].e[e]),
                                                                 Cvt<T>::to_f(bv[i].e[e]));
                                acc[e] = fmaf(df, inner, acc[e]);
                            }
                        }
                        if (DB) store_pack_stream(d_base + off, ob);
                        if (DL) store_pack_stream(d_lora + off, ol);
                    }
                }
            }
        }
    }
    if (DM) {
        if (tr > 0) {
#pragma unroll
            for (int e = 0; e < N; ++e) red[tr - 1][e][tc] = acc[e];
        }
        lds_barrier();   // the d_base / d_lora stores stay in flight
        if (tr == 0 && active) {
#pragma unroll
            for (int e = 0; e < N; ++e) {
                float v = acc[e];
#pragma unroll
                for (int q = 0; q < kTR - 1; ++q) v += red[q][e][tc];
                dm_part[(int64_t)blockIdx.y * d_out + col + e] = v;
            }
        }
    }
}

template <typename T, bool DELTA, bool DM, bool DB, bool DL, int kBwdTokenBlock, bool INNER>
__global__ __launch_bounds__(kThreads) void compose_bwd_scalar(const T* dy, const T* __restrict__ base,
                                                               const T* __restrict__ lora,
                                                               const float* __restrict__ g, float s,
                                                               int64_t nrows, int64_t d_out, T* d_base,
                                                               T* d_lora, float* __restrict__ dm_part) {
    const int64_t col = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (col >= d_out) return;
    const float gv = g[col];
    const float gb = DELTA ? gv - 1.0f : gv, gl = gv * s;
    float acc = 0.0f;
    for (int64_t rb = blockIdx.y; rb * kBwdTokenBlock < nrows; rb += gridDim.y) {
        const int64_t rend = (rb + 1) * kBwdTokenBlock < nrows ? (rb + 1) * kBwdTokenBlock : nrows;
        for (int64_t row = rb * kBwdTokenBlock; row < rend; ++row) {
            const int64_t off = row * d_out + col;
            const float df = Cvt<T>::to_f(dy[off]);
            if (DM)
                acc = fmaf(df, INNER ? Cvt<T>::to_f(base[off]) : fmaf(s, Cvt<T>::to_f(lora[off]), Cvt<T>::to_f(base[off])),
                           acc);
            if (DB) d_base[off] = Cvt<T>::from_f(gb * df);
            if (DL) d_lora[off] = Cvt<T>::from_f(gl * df);
        }
    }
    if (DM) dm_part[(int64_t)blockIdx.y * d_out + col] = acc;
}

// d_m_j = (sum over partial rows p of part[p][j]) / max(wnorm_j, eps).
// A workgroup owns 64 columns; its 4 waves sum interleaved partial rows
// (p = w, w + 4, ...) with independent loads in flight, then wave 0 adds the
// four sums in wave order.  The order is fixed, so d_m is reproducible.
constexpr int kFinCols = 32;                       // d_m columns per workgroup
constexpr int kFinLanes = kThreads / kFinCols;      // partial rows per column, summed side by side
constexpr int kFinBatch = 16;                       // loads a lane issues before summing

// d_m_j = (sum over partial rows p of part[p][j]) / max(wnorm_j, eps).  Lane
// w of column j sums rows w, w + kFinLanes, ... in order, loading a batch of
// them at once; the kFinLanes sums are then added in lane order.  The order
// is fixed, so the result is bitwise reproducible.
__global__ __launch_bounds__(kThreads) void dm_finalize(const float* __restrict__ part, int nparts,
                                                        const float* __restrict__ wnorm, float eps,
                                                        int64_t d_out, float* __restrict__ d_m) {
    __shared__ float red[kFinLanes][kFinCols];
    const int c = threadIdx.x % kFinCols, w = threadIdx.x / kFinCols;
    const int64_t j = (int64_t)blockIdx.x * kFinCols + c;
    // wnorm is requested with the partials, not after them
    const float wn = (w == 0 && j < d_out) ? wnorm[j] : 1.0f;
    float acc = 0.0f;
    if (j < d_out) {
        for (int p0 = w; p0 < nparts; p0 += kFinLanes * kFinBatch) {
            float x[kFinBatch];
#pragma unroll
            for (int t = 0; t < kFinBatch; ++t) {
                const int p = p0 + t * kFinLanes;
                x[t] = p < nparts ? part[(int64_t)p * d_out + j] : 0.0f;
            }
#pragma unroll
            for (int t = 0; t < kFinBatch; ++t) acc += x[t];
        }
    }
    red[w][c] = acc;
    __syncthreads();
    if (w == 0 && j < d_out) {
        float v = red[0][c];
#pragma unroll
        for (int q = 1; q < kFinLanes; ++q) v += red[q][c];
        d_m[j] = nparts > 0 ? v / fmaxf(wn, eps) : 0.0f;
    }
}

inline bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Backward tiling for a shape: narrow activations keep 8 rows per thread in
// flight over 32-row token blocks, wide ones 4 rows over 16-row blocks.
bool bwd_narrow(int64_t d_out) { return d_out <= 4096; }
int bwd_token_block(int64_t d_out) { return bwd_narrow(d_out) ? 32 : 16; }

int bwd_parts(int64_t T, int64_t d_out) {
    const int tb = bwd_token_block(d_out);
    int64_t p = (T + tb - 1) / tb;
    return (int)(p < kMaxParts ? p : kMaxParts);
}

template <typename T, bool DELTA, bool DUAL>
void fwd_launch(bool vec, bool wide, dim3 grid, unsigned sgrid, const T* b, const T* l, const float* g, float s,
                int64_t nrows, int64_t d_out, T* o, T* in, hipStream_t st) {
    if (!vec)
        compose_fwd_scalar<T, DELTA, DUAL><<<sgrid, kThreads, 0, st>>>(b, l, g, s, nrows * d_out, d_out, o, in);
    else if (wide)
        compose_fwd_vec<T, DELTA, 2, DUAL><<<grid, kThreads, 0, st>>>(b, l, g, s, nrows, d_out, o, in);
    else
        compose_fwd_vec<T, DELTA, 4, DUAL><<<grid, kThreads, 0, st>>>(b, l, g, s, nrows, d_out, o, in);
}

template <typename T>
hipError_t fwd_typed(const void* base, const void* lora, const float* g, float s, int64_t nrows,
                     int64_t d_out, bool delta, void* y, void* inner, hipStream_t st) {
    constexpr int N = Pack<T>::N;
    const T* b = static_cast<const T*>(base);
    const T* l = static_cast<const T*>(lora);
    T* o = static_cast<T*>(y);
    T* in = static_cast<T*>(inner);
    const bool dual = inner != nullptr;
    const bool vec = d_out % N == 0 && aligned16(base) && aligned16(lora) && aligned16(y) && aligned16(inner);
    const bool wide = d_out >= 8192;
    dim3 grid(1, 1);
    unsigned sgrid = 1;
    if (vec) {
        const int64_t gx = (d_out / N + kTC - 1) / kTC;
        const int rpb = kTR * (wide ? 2 : 4);
        int64_t gy = (nrows + rpb - 1) / rpb;
        if (gy > kMaxGridY) gy = kMaxGridY;
        grid = dim3((unsigned)gx, (unsigned)gy);
    } else {
        int64_t gx = (nrows * d_out + kThreads - 1) / kThreads;
        if (gx > 65536) gx = 65536;
        sgrid = (unsigned)gx;
    }
    if (delta) {
        if (dual) fwd_launch<T, true, true>(vec, wide, grid, sgrid, b, l, g, s, nrows, d_out, o, in, st);
        else fwd_launch<T, true, false>(vec, wide, grid, sgrid, b, l, g, s, nrows, d_out, o, in, st);
    } else {
        if (dual) fwd_launch<T, false, true>(vec, wide, grid, sgrid, b, l, g, s, nrows, d_out, o, in, st);
        else fwd_launch<T, false, false>(vec, wide, grid, sgrid, b, l, g, s, nrows, d_out, o, in, st);
    }
    return hipGetLastError();
}

template <typename T, bool DELTA, bool DM, bool DB, bool DL, bool INNER>
void bwd_launch(bool vec, const T* dy, const T* b, const T* l, const float* g, float s, int64_t nrows,
                int64_t d_out, T* db, T* dl, float* part, int nparts, hipStream_t st) {
    const bool narrow = bwd_narrow(d_out);
    if (vec) {
        constexpr int N = Pack<T>::N;
        const int64_t gx = (d_out / N + kTC - 1) / kTC;
        dim3 grid((unsigned)gx, (unsigned)nparts);
        if (narrow)
            compose_bwd_vec<T, DELTA, DM, DB, DL, 8, 32, INNER><<<grid, kThreads, 0, st>>>(dy, b, l, g, s, nrows,
                                                                                          d_out, db, dl, part);
        else
            compose_bwd_vec<T, DELTA, DM, DB, DL, 4, 16, INNER><<<grid, kThreads, 0, st>>>(dy, b, l, g, s, nrows,
                                                                                          d_out, db, dl, part);
    } else {
        dim3 grid((unsigned)((d_out + kThreads - 1) / kThreads), (unsigned)nparts);
        if (narrow)
            compose_bwd_scalar<T, DELTA, DM, DB, DL, 32, INNER><<<grid, kThreads, 0, st>>>(dy, b, l, g, s, nrows,
                                                                                          d_out, db, dl, part);
        else
            compose_bwd_scalar<T, DELTA, DM, DB, DL, 16, INNER><<<grid, kThreads, 0, st>>>(dy, b, l, g, s, nrows,
                                                                                          d_out, db, dl, part);
    }
}

template <typename T, bool DELTA, bool DM, bool INNER>
void bwd_dispatch_outputs(bool vec, const T* dy, const T* b, const T* l, const float* g, float s,
                          int64_t nrows, int64_t d_out, T* db, T* dl, float* part, int nparts,
                          hipStream_t st) {
    if (db && dl)
        bwd_launch<T, DELTA, DM, true, true, INNER>(vec, dy, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
    else if (db)
        bwd_launch<T, DELTA, DM, true, false, INNER>(vec, dy, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
    else if (dl)
        bwd_launch<T, DELTA, DM, false, true, INNER>(vec, dy, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
    else
        bwd_launch<T, DELTA, DM, false, false, INNER>(vec, dy, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
}

// inner_mode: `base` holds inner = base + s * lora and `lora` is unused.
template <typename T>
hipError_t bwd_typed(const void* dy, const void* base, const void* lora, const float* g,
                     const float* wnorm, float s, float eps, int64_t nrows, int64_t d_out, bool delta,
                     bool inner_mode, void* d_base, void* d_lora, float* d_m, void* ws, hipStream_t st) {
    constexpr int N = Pack<T>::N;
    const T* dyp = static_cast<const T*>(dy);
    const T* b = static_cast<const T*>(base);
    const T* l = static_cast<const T*>(lora);
    T* db = static_cast<T*>(d_base);
    T* dl = static_cast<T*>(d_lora);
    const bool want_dm = d_m != nullptr;
    if (nrows > 0 && (db || dl || want_dm)) {
        const bool vec = d_out % N == 0 && aligned16(dy) && aligned16(db) && aligned16(dl) &&
                         (!want_dm || (aligned16(base) && (inner_mode || aligned16(lora))));
        float* part = static_cast<float*>(ws);
        if (want_dm) {
            const int nparts = bwd_parts(nrows, d_out);
            if (inner_mode) {
                if (delta)
                    bwd_dispatch_outputs<T, true, true, true>(vec, dyp, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
                else
                    bwd_dispatch_outputs<T, false, true, true>(vec, dyp, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
            } else {
                if (delta)
                    bwd_dispatch_outputs<T, true, true, false>(vec, dyp, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
                else
                    bwd_dispatch_outputs<T, false, true, false>(vec, dyp, b, l, g, s, nrows, d_out, db, dl, part, nparts, st);
            }
        } else {
            // frozen magnitude: only dy is read; the token grid needs no partials
            const int tb = bwd_token_block(d_out);
            int64_t gy = (nrows + tb - 1) / tb;
            const int nblk = (int)(gy < kMaxGridY ? gy : kMaxGridY);
            if (delta)
                bwd_dispatch_outputs<T, true, false, false>(vec, dyp, b, l, g, s, nrows, d_out, db, dl, nullptr, nblk, st);
            else
                bwd_dispatch_outputs<T, false, false, false>(vec, dyp, b, l, g, s, nrows, d_out, db, dl, nullptr, nblk, st);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (want_dm) {
        const int nparts = nrows > 0 ? bwd_parts(nrows, d_out) : 0;
        dm_finalize<<<(unsigned)((d_out + kFinCols - 1) / kFinCols), kThreads, 0, st>>>(
            static_cast<const float*>(ws), nparts, wnorm, eps, d_out, d_m);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

size_t compose_bwd_workspace_bytes(int64_t T, int64_t d_out) {
    if (T <= 0) return 0;
    return align_up((size_t)bwd_parts(T, d_out) * (size_t)d_out * sizeof(float), 256);
}

hipError_t launch_compose_fwd(const void* base, const void* lora, const float* g, float s, int64_t T,
                              int64_t d_out, int dtype, bool delta_only, void* y, void* inner, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    switch (dtype) {
        case kF32: return fwd_typed<float>(base, lora, g, s, T, d_out, delta_only, y, inner, stream);
        case kBF16: return fwd_typed<bf16_t>(base, lora, g, s, T, d_out, delta_only, y, inner, stream);
        default: return fwd_typed<f16_t>(base, lora, g, s, T, d_out, delta_only, y, inner, stream);
    }
}

hipError_t launch_compose_bwd(const void* dy, const void* base, const void* lora, const float* g,
                              const float* wnorm, float s, float eps, int64_t T, int64_t d_out,
                              int dtype, bool delta_only, bool inner_mode, void* d_base, void* d_lora,
                              float* d_m, void* workspace, hipStream_t stream) {
    switch (dtype) {
        case kF32:
            return bwd_typed<float>(dy, base, lora, g, wnorm, s, eps, T, d_out, delta_only, inner_mode, d_base,
                                    d_lora, d_m, workspace, stream);
        case kBF16:
            return bwd_typed<bf16_t>(dy, base, lora, g, wnorm, s, eps, T, d_out, delta_only, inner_mode, d_base,
                                     d_lora, d_m, workspace, stream);
        default:
            return bwd_typed<f16_t>(dy, base, lora, g, wnorm, s, eps, T, d_out, delta_only, inner_mode, d_base,
                                    d_lora, d_m, workspace, stream);
    }
}

}  // namespace dora
