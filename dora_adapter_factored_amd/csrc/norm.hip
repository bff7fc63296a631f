// Factored DoRA row norm on gfx950 MFMA.
//
// "Scaling DoRA" §2 writes the squared row norm of W0 + sBA as three terms,
//   n2_i = ||W0_i||^2 + 2s B_i.(W0 A^T)_i + s^2 B_i (A A^T) B_i^T,
// computed through O(d_out r + r^2) intermediates, accumulated in fp32, and
// assembled as sqrt(max(n2, 0)) (App. B); g = m / max(wnorm, eps) (§4).
//
// Mapping onto the chip.  With Gs = (s/2) * A A^T, the last two terms are
// 2s * B_i . (U_i + B_i Gs) where U = W0 A^T.  U_i + B_i Gs is one GEMM row
// over the extended contraction [W0_i | B_i] x [A | Gs]^T (K = d_in + r), and
// its dot with B_i is linear in every K-chunk and every slice of r.  So:
//   1. gram_partial / gram_finalize: Gs = (s/2) A A^T (MFMA, split-K partial
//      tiles summed in a fixed order, rounded once to the operand dtype).
//   2. w0_pass: one streaming pass over W0.  Each workgroup owns BM rows of
//      W0, BN columns of r and a K-chunk of the extended contraction; W0 and A
//      (then B and Gs) tiles are staged through LDS and fed to MFMA with fp32
//      accumulation.  The W0 tile loader also accumulates ||W0_i||^2 from the
//      registers it already holds.  The epilogue dots each accumulator row
//      with B_i in registers, so U never reaches HBM: a workgroup writes BM
//      partial scalars (and BM partial base sums).
//   3. norm_finalize: sums the partials in a fixed order, forms n2, clamps,
//      takes the square root and divides m.
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "dora_device.h"
#include "dora_launch.h"

namespace dora {
namespace {

constexpr int kNumCU = 256;
constexpr int kNumXCD = 8;

// ------------------------------------------------------------- MFMA traits
// One "k-step" contracts 32 elements of K.  In a k-step each lane supplies 8
// consecutive K values of its row (lane/16 picks which 8); the same
// assignment is used for both operands, so every product pairs matching K.
template <typename E> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int VEC = 8;   // elements per 16-byte chunk
    static constexpr int BK = 64;   // K per LDS tile: 8 chunks per row
    typedef bf16x8_t frag_t;
    __device__ __forceinline__ static frag_t load_frag(const bf16_t* p) {
        return *reinterpret_cast<const bf16x8_t*>(p);
    }
    __device__ __forceinline__ static void mma(f32x4_t& c, const frag_t& a, const frag_t& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int VEC = 4;
    static constexpr int BK = 32;
    struct frag_t {
        f32x4_t lo, hi;
    };
    __device__ __forceinline__ static frag_t load_frag(const float* p) {
        frag_t f;
        f.lo = *reinterpret_cast<const f32x4_t*>(p);
        f.hi = *reinterpret_cast<const f32x4_t*>(p + 4);
        return f;
    }
    __device__ __forceinline__ static void mma(f32x4_t& c, const frag_t& a, const frag_t& b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[i], b.lo[i], c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[i], b.hi[i], c, 0, 0, 0);
    }
};

// A row-major operand [rows][ld] whose valid K range is [0, kmax).
struct Operand {
    const void* p;
    int64_t ld, rows, kmax;
};

// The contraction of one workgroup: k-tiles [0, nkt0) read phase 0, k-tiles
// [nkt0, nkt0 + nkt1) read phase 1.  "left" rows index the output rows (M),
// "right" rows index the output columns (N).
struct Contraction {
    Operand left0, right0, left1, right1;
    int nkt0, nkt1;
};

template <typename E, bool ALIGNED>
__device__ __forceinline__ u32x4_t load_chunk(const Operand& o, int64_t row, int64_t k) {
    constexpr int VEC = Mma<E>::VEC;
    const E* p = static_cast<const E*>(o.p);
    if (ALIGNED) {
        if (row < o.rows && k < o.kmax) return *reinterpret_cast<const u32x4_t*>(p + row * o.ld + k);
        return u32x4_t{0u, 0u, 0u, 0u};
    } else {
        Pack<E> v;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v.e[e] = (row < o.rows && k + e < o.kmax) ? p[row * o.ld + k + e] : Cvt<E>::from_f(0.0f);
        return v.u;
    }
}

template <typename E>
__device__ __forceinline__ float chunk_sumsq(u32x4_t u) {
    Pack<E> v;
    v.u = u;
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < Pack<E>::N; ++e) {
        const float x = Cvt<E>::to_f(v.e[e]);
        s = fmaf(x, x, s);
    }
    return s;
}

// Tile geometry of a workgroup: WM x WN waves, each wave MT x NT blocks of
// 16 x 16 outputs.
template <typename E, int WM, int WN, int MT, int NT>
struct Tile {
    static constexpr int NTH = WM * WN * 64;
    static constexpr int BM = WM * MT * 16;
    static constexpr int BN = WN * NT * 16;
    static constexpr int BK = Mma<E>::BK;
    static constexpr int VEC = Mma<E>::VEC;
    static constexpr int CPR = BK / VEC;   // 16-byte chunks per tile row (8)
    static constexpr int LD = BK + VEC;    // LDS row pitch: +16 bytes keeps 16 rows on distinct banks
    static constexpr int LCH = (BM * CPR + NTH - 1) / NTH;
    static constexpr int RCH = (BN * CPR + NTH - 1) / NTH;
    static constexpr int BUF = (BM + BN) * LD;   // elements per LDS stage
    static constexpr int LDS_BYTES = 2 * BUF * (int)sizeof(E);
    static_assert(CPR == 8, "tile rows are 8 chunks");
    static_assert(NTH % CPR == 0, "a thread keeps the same chunk column across tiles");
};

// Streams k-tiles [kt_begin, kt_end) of `c` through double-buffered LDS into
// the MFMA accumulators.  When `base_rows` is set, the squares of every phase-0
// left element are summed per thread (bsum[j] covers chunk j of the thread).
template <typename E, int WM, int WN, int MT, int NT, bool ALIGNED>
__device__ __forceinline__ void mainloop(const Contraction& c, int64_t m0, int64_t n0, int kt_begin,
                                         int kt_end, bool base_rows, f32x4_t (&acc)[MT][NT],
                                         float (&bsum)[Tile<E, WM, WN, MT, NT>::LCH], E* lds) {
    typedef Tile<E, WM, WN, MT, NT> TL;
    typedef Mma<E> M;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int cc = tid % TL::CPR;   // chunk column, fixed for this thread

    u32x4_t lreg[TL::LCH], rreg[TL::RCH];

    auto load_tile = [&](int kt) {
        const bool ph0 = kt < c.nkt0;
        const Operand& L = ph0 ? c.left0 : c.left1;
        const Operand& R = ph0 ? c.right0 : c.right1;
        const int64_t k = (int64_t)(ph0 ? kt : kt - c.nkt0) * TL::BK + cc * TL::VEC;
#pragma unroll
        for (int j = 0; j < TL::LCH; ++j) {
            const int ch = tid + j * TL::NTH;
            if (TL::BM * TL::CPR % TL::NTH == 0 || ch < TL::BM * TL::CPR)
                lreg[j] = load_chunk<E, ALIGNED>(L, m0 + ch / TL::CPR, k);
        }
#pragma unroll
        for (int j = 0; j < TL::RCH; ++j) {
            const int ch = tid + j * TL::NTH;
            if (TL::BN * TL::CPR % TL::NTH == 0 || ch < TL::BN * TL::CPR)
                rreg[j] = load_chunk<E, ALIGNED>(R, n0 + ch / TL::CPR, k);
        }
    };
    auto store_tile = [&](int buf, bool ph0) {
        E* Ls = lds + buf * TL::BUF;
        E* Rs = Ls + TL::BM * TL::LD;
#pragma unroll
        for (int j = 0; j < TL::LCH; ++j) {
            const int ch = tid + j * TL::NTH;
            if (TL::BM * TL::CPR % TL::NTH == 0 || ch < TL::BM * TL::CPR) {
                *reinterpret_cast<u32x4_t*>(Ls + (ch / TL::CPR) * TL::LD + cc * TL::VEC) = lreg[j];
                if (base_rows && ph0) bsum[j] += chunk_sumsq<E>(lreg[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < TL::RCH; ++j) {
            const int ch = tid + j * TL::NTH;
            if (TL::BN * TL::CPR % TL::NTH == 0 || ch < TL::BN * TL::CPR)
                *reinterpret_cast<u32x4_t*>(Rs + (ch / TL::CPR) * TL::LD + cc * TL::VEC) = rreg[j];
        }
    };
    auto compute = [&](int buf) {
        const E* Ls = lds + buf * TL::BUF + (wm * MT * 16 + (lane & 15)) * TL::LD + (lane >> 4) * 8;
        const E* Rs = lds + buf * TL::BUF + (TL::BM + wn * NT * 16 + (lane & 15)) * TL::LD + (lane >> 4) * 8;
#pragma unroll
        for (int ks = 0; ks < TL::BK / 32; ++ks) {
            typename M::frag_t a[MT], b[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt] = M::load_frag(Ls + mt * 16 * TL::LD + ks * 32);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b[nt] = M::load_frag(Rs + nt * 16 * TL::LD + ks * 32);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) M::mma(acc[mt][nt], a[mt], b[nt]);
        }
    };

    if (kt_begin >= kt_end) return;
    load_tile(kt_begin);
    store_tile(0, kt_begin < c.nkt0);
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int buf = (kt - kt_begin) & 1;
        const bool more = kt + 1 < kt_end;
        if (more) load_tile(kt + 1);
        compute(buf);
        if (more) store_tile(buf ^ 1, kt + 1 < c.nkt0);
        __syncthreads();
    }
}

// ------------------------------------------------------------- W0 pass
struct W0PassArgs {
    Contraction c;
    const void* B;          // [d_out, r], for the row-dot epilogue
    int64_t d_out, r;
    int ksplit, n_mtiles, n_ntiles;
    int xcd_map;            // workgroups on one XCD share (n-tile, k-chunk)
    float* part_base;       // [ksplit][d_out]
    float* part_cross;      // [n_ntiles * ksplit][d_out]
};

template <typename E, int WM, int WN, int MT, int NT, bool ALIGNED>
__global__ __launch_bounds__(WM * WN * 64) void w0_pass(W0PassArgs a) {
    typedef Tile<E, WM, WN, MT, NT> TL;
    __shared__ __attribute__((aligned(16))) char smem[TL::LDS_BYTES];
    E* lds = reinterpret_cast<E*>(smem);

    // Workgroup -> (m-tile, n-tile, k-chunk).  Workgroups are handed to the 8
    // XCDs round-robin; when possible all workgroups of one XCD share the same
    // (n-tile, k-chunk), i.e. the same slice of A, which then stays in that
    // XCD's L2 while W0 streams past.
    const int Q = a.n_ntiles * a.ksplit;
    const int id = blockIdx.x;
    int q, mtile;
    if (a.xcd_map) {
        const int xcd = id % kNumXCD, slot = id / kNumXCD;
        q = xcd % Q;
        mtile = slot * (kNumXCD / Q) + xcd / Q;
    } else {
        q = id % Q;
        mtile = id / Q;
    }
    if (mtile >= a.n_mtiles) return;
    const int ntile = q / a.ksplit, kc = q % a.ksplit;
    const int64_t m0 = (int64_t)mtile * TL::BM, n0 = (int64_t)ntile * TL::BN;
    const int nkt = a.c.nkt0 + a.c.nkt1;
    const int kt_begin = (int)((int64_t)kc * nkt / a.ksplit);
    const int kt_end = (int)((int64_t)(kc + 1) * nkt / a.ksplit);
    const bool base_rows = ntile == 0;

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float bsum[TL::LCH];
#pragma unroll
    for (int j = 0; j < TL::LCH; ++j) bsum[j] = 0.0f;

    mainloop<E, WM, WN, MT, NT, ALIGNED>(a.c, m0, n0, kt_begin, kt_end, base_rows, acc, bsum, lds);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // base partial: the 8 threads of a row hold the 8 chunk columns
    if (base_rows) {
#pragma unroll
        for (int j = 0; j < TL::LCH; ++j) {
            float v = bsum[j];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            const int ch = tid + j * TL::NTH;
            const int64_t m = m0 + ch / TL::CPR;
            if ((tid % TL::CPR) == 0 && ch < TL::BM * TL::CPR && m < a.d_out)
                a.part_base[(int64_t)kc * a.d_out + m] = v;
        }
    }

    // cross partial: sum_n B[m][n] * acc[m][n] over this workgroup's columns.
    // acc[mt][nt][j] is row wm*MT*16 + mt*16 + 4*(lane/16) + j, column
    // wn*NT*16 + nt*16 + lane%16 of the tile.
    const E* Bp = static_cast<const E*>(a.B);
    float* red = reinterpret_cast<float*>(smem);   // [WN][BM], LDS is free after the main loop
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = wm * MT * 16 + mt * 16 + 4 * (lane >> 4) + j;
            const int64_t m = m0 + row;
            float v = 0.0f;
            if (m < a.d_out) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int64_t n = n0 + wn * NT * 16 + nt * 16 + (lane & 15);
                    if (n < a.r) v = fmaf(Cvt<E>::to_f(Bp[m * a.r + n]), acc[mt][nt][j], v);
                }
            }
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            if ((lane & 15) == 0) red[wn * TL::BM + row] = v;
        }
    }
    __syncthreads();
    for (int row = tid; row < TL::BM; row += TL::NTH) {
        const int64_t m = m0 + row;
        if (m < a.d_out) {
            float v = red[row];
#pragma unroll
            for (int w = 1; w < WN; ++w) v += red[w * TL::BM + row];
            a.part_cross[((int64_t)ntile * a.ksplit + kc) * a.d_out + m] = v;
        }
    }
}

// ------------------------------------------------------------- Gram
constexpr int kGramTile = 64;   // WM = WN = 2, MT = NT = 2

struct GramArgs {
    Contraction c;     // left0 = right0 = A
    int ntiles, nsplit, nupper;
    int64_t rnp;       // ntiles * 64
    float* part;       // [nsplit][rnp][rnp], upper tiles only
};

template <typename E, bool ALIGNED>
__global__ __launch_bounds__(256) void gram_partial(GramArgs a) {
    typedef Tile<E, 2, 2, 2, 2> TL;
    __shared__ __attribute__((aligned(16))) char smem[TL::LDS_BYTES];
    const int id = blockIdx.x;
    const int split = id / a.nupper;
    int u = id % a.nupper, ti = 0;
    while (u >= a.ntiles - ti) {
        u -= a.ntiles - ti;
        ++ti;
    }
    const int tj = ti + u;
    const int nkt = a.c.nkt0;
    const int kt_begin = (int)((int64_t)split * nkt / a.nsplit);
    const int kt_end = (int)((int64_t)(split + 1) * nkt / a.nsplit);
    f32x4_t acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float bsum[TL::LCH];
    mainloop<E, 2, 2, 2, 2, ALIGNED>(a.c, (int64_t)ti * kGramTile, (int64_t)tj * kGramTile, kt_begin, kt_end,
                                     false, acc, bsum, reinterpret_cast<E*>(smem));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / 2, wn = wave % 2;
    float* out = a.part + (int64_t)split * a.rnp * a.rnp;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = (int64_t)ti * kGramTile + wm * 32 + mt * 16 + 4 * (lane >> 4) + j;
                const int64_t k = (int64_t)tj * kGramTile + wn * 32 + nt * 16 + (lane & 15);
                out[i * a.rnp + k] = acc[mt][nt][j];
            }
}

// Gs[i][j] = (s/2) * sum_split G[i][j] for i < r, j < r; zero for r <= j < ldg.
// Only upper tiles were computed; the lower ones are read transposed.
template <typename E>
__global__ __launch_bounds__(256) void gram_finalize(const float* __restrict__ part, int nsplit, int64_t rnp,
                                                     int64_t r, int64_t ldg, float half_s, E* __restrict__ gs) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= r * ldg) return;
    const int64_t i = idx / ldg, j = idx % ldg;
    float v = 0.0f;
    if (j < r) {
        const bool upper = (i / kGramTile) <= (j / kGramTile);
        const int64_t off = upper ? i * rnp + j : j * rnp + i;
        float sum = 0.0f;
        for (int sp = 0; sp < nsplit; ++sp) sum += part[(int64_t)sp * rnp * rnp + off];
        v = half_s * sum;
    }
    gs[idx] = Cvt<E>::from_f(v);
}

// ------------------------------------------------------------- base only
// s == 0: wnorm_i = ||W0_i||.  One wave per row.
template <typename E, bool ALIGNED>
__global__ __launch_bounds__(256) void row_sumsq(const E* __restrict__ W0, int64_t d_out, int64_t d_in,
                                                 float* __restrict__ part_base) {
    constexpr int VEC = Pack<E>::N;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= d_out) return;
    const E* p = W0 + row * d_in;
    float s = 0.0f;
    if (ALIGNED) {
        for (int64_t k = (int64_t)lane * VEC; k < d_in; k += 64 * VEC) s += chunk_sumsq<E>(load_pack_stream(p + k).u);
    } else {
        for (int64_t k = lane; k < d_in; k += 64) {
            const float x = Cvt<E>::to_f(p[k]);
            s = fmaf(x, x, s);
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
    if (lane == 0) part_base[row] = s;
}

// ------------------------------------------------------------- finalize
__global__ __launch_bounds__(256) void norm_finalize(const float* __restrict__ pbase, int nbase,
                                                     const float* __restrict__ pcross, int ncross, int64_t d_out,
                                                     float two_s, const float* __restrict__ m, float eps,
                                                     float* __restrict__ wnorm, float* __restrict__ g) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= d_out) return;
    float base = 0.0f, cd = 0.0f;
    for (int c = 0; c < nbase; ++c) base += pbase[(int64_t)c * d_out + i];
    for (int c = 0; c < ncross; ++c) cd += pcross[(int64_t)c * d_out + i];
    const float n2 = fmaxf(fmaf(two_s, cd, base), 0.0f);
    const float wn = sqrtf(n2);
    wnorm[i] = wn;
    if (m) g[i] = m[i] / fmaxf(wn, eps);
}

// ------------------------------------------------------------- configs
struct TileCfg {
    int wm, wn, mt, nt;
};
// Ordered by the width BN of the slice of r a workgroup covers.
constexpr TileCfg kCfgs[] = {
    {4, 1, 2, 1},    // BM 128, BN 16
    {2, 2, 4, 1},    // BM 128, BN 32
    {2, 2, 4, 2},    // BM 128, BN 64
    {2, 2, 4, 4},    // BM 128, BN 128
    {2, 2, 4, 6},    // BM 128, BN 192
    {2, 2, 4, 12},   // BM 128, BN 384
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

template <typename E, int CFG, bool AL>
hipError_t launch_w0_cfg(const W0PassArgs& a, int grid, hipStream_t st) {
    constexpr TileCfg t = kCfgs[CFG];
    w0_pass<E, t.wm, t.wn, t.mt, t.nt, AL><<<grid, t.wm * t.wn * 64, 0, st>>>(a);
    return hipGetLastError();
}

template <typename E, bool AL>
hipError_t launch_w0(int cfg, const W0PassArgs& a, int grid, hipStream_t st) {
    switch (cfg) {
        case 0: return launch_w0_cfg<E, 0, AL>(a, grid, st);
        case 1: return launch_w0_cfg<E, 1, AL>(a, grid, st);
        case 2: return launch_w0_cfg<E, 2, AL>(a, grid, st);
        case 3: return launch_w0_cfg<E, 3, AL>(a, grid, st);
        case 4: return launch_w0_cfg<E, 4, AL>(a, grid, st);
        default:
            if constexpr (sizeof(E) == 2) return launch_w0_cfg<E, 5, AL>(a, grid, st);
            return hipErrorInvalidValue;
    }
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename E>
hipError_t norm_typed(const NormPlan& p, const void* W0, const void* A, const void* B, const float* m, float s,
                      float eps, float* wnorm, float* g, void* ws, hipStream_t st) {
    constexpr int VEC = Mma<E>::VEC;
    char* w = static_cast<char*>(ws);
    float* pbase = reinterpret_cast<float*>(w + p.off_pbase);
    const int64_t d_out = p.d_out, d_in = p.d_in, r = p.r;
    hipError_t e;
    if (p.base_only) {
        const bool al = d_in % VEC == 0 && al16(W0);
        const unsigned grid = (unsigned)((d_out + 3) / 4);
        if (al)
            row_sumsq<E, true><<<grid, 256, 0, st>>>(static_cast<const E*>(W0), d_out, d_in, pbase);
        else
            row_sumsq<E, false><<<grid, 256, 0, st>>>(static_cast<const E*>(W0), d_out, d_in, pbase);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        norm_finalize<<<(unsigned)((d_out + 255) / 256), 256, 0, st>>>(pbase, 1, nullptr, 0, d_out, 0.0f, m, eps,
                                                                        wnorm, g);
        return hipGetLastError();
    }
    E* gs = reinterpret_cast<E*>(w + p.off_gs);
    float* gpart = reinterpret_cast<float*>(w + p.off_gpart);
    float* pcross = reinterpret_cast<float*>(w + p.off_pcross);
    const bool al = d_in % VEC == 0 && r % VEC == 0 && al16(W0) && al16(A) && al16(B);

    // 1. Gs = (s/2) A A^T
    GramArgs ga;
    ga.c.left0 = Operand{A, d_in, r, d_in};
    ga.c.right0 = ga.c.left0;
    ga.c.left1 = ga.c.right1 = Operand{nullptr, 0, 0, 0};
    ga.c.nkt0 = (int)((d_in + p.bk - 1) / p.bk);
    ga.c.nkt1 = 0;
    ga.ntiles = p.gram_tiles;
    ga.nsplit = p.gram_split;
    ga.nupper = p.gram_tiles * (p.gram_tiles + 1) / 2;
    ga.rnp = (int64_t)p.gram_tiles * kGramTile;
    ga.part = gpart;
    const unsigned ggrid = (unsigned)(ga.nupper * ga.nsplit);
    if (al)
        gram_partial<E, true><<<ggrid, 256, 0, st>>>(ga);
    else
        gram_partial<E, false><<<ggrid, 256, 0, st>>>(ga);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gram_finalize<E><<<(unsigned)((r * p.ldg + 255) / 256), 256, 0, st>>>(gpart, ga.nsplit, ga.rnp, r, p.ldg,
                                                                          0.5f * s, gs);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // 2. streaming pass over [W0 | B] x [A | Gs]^T with the row-dot epilogue
    W0PassArgs wa;
    wa.c.left0 = Operand{W0, d_in, d_out, d_in};
    wa.c.right0 = Operand{A, d_in, r, d_in};
    wa.c.left1 = Operand{B, r, d_out, r};
    wa.c.right1 = Operand{gs, p.ldg, r, r};
    wa.c.nkt0 = p.nkt_w0;
    wa.c.nkt1 = p.nkt_g;
    wa.B = B;
    wa.d_out = d_out;
    wa.r = r;
    wa.ksplit = p.ksplit;
    wa.n_mtiles = p.n_mtiles;
    wa.n_ntiles = p.n_ntiles;
    const int Q = p.n_ntiles * p.ksplit;
    wa.xcd_map = (Q <= kNumXCD && kNumXCD % Q == 0) ? 1 : 0;
    wa.part_base = pbase;
    wa.part_cross = pcross;
    int grid;
    if (wa.xcd_map) {
        const int per = kNumXCD / Q;   // m-tiles per XCD slot
        grid = kNumXCD * ((p.n_mtiles + per - 1) / per);
    } else {
        grid = Q * p.n_mtiles;
    }
    e = al ? launch_w0<E, true>(p.cfg, wa, grid, st) : launch_w0<E, false>(p.cfg, wa, grid, st);
    if (e != hipSuccess) return e;

    // 3. assemble
    norm_finalize<<<(unsigned)((d_out + 255) / 256), 256, 0, st>>>(pbase, p.ksplit, pcross, Q, d_out, 2.0f * s, m,
                                                                    eps, wnorm, g);
    return hipGetLastError();
}

}  // namespace

NormPlan plan_norm(int64_t d_out, int64_t d_in, int64_t r, int dtype, bool base_only) {
    NormPlan p{};
    p.dtype = dtype;
    p.d_out = d_out;
    p.d_in = d_in;
    p.r = r;
    p.base_only = base_only;
    const int esz = (int)dtype_size(dtype);
    const int vec = 16 / esz;
    p.bk = dtype == kF32 ? Mma<float>::BK : Mma<bf16_t>::BK;
    if (base_only) {
        p.off_pbase = 0;
        p.bytes = align_up((size_t)d_out * 4, 256);
        return p;
    }
    // widest configuration this dtype instantiates (fp32 fragments double the
    // register footprint, so fp32 stops at BN = 192)
    const int max_cfg = dtype == kF32 ? 4 : kNumCfgs - 1;
    int cfg = 0;
    while (cfg < max_cfg && kCfgs[cfg].wn * kCfgs[cfg].nt * 16 < r) ++cfg;
    p.cfg = cfg;
    p.bm = kCfgs[cfg].wm * kCfgs[cfg].mt * 16;
    p.bn = kCfgs[cfg].wn * kCfgs[cfg].nt * 16;
    p.n_mtiles = (int)((d_out + p.bm - 1) / p.bm);
    p.n_ntiles = (int)((r + p.bn - 1) / p.bn);
    p.nkt_w0 = (int)((d_in + p.bk - 1) / p.bk);
    p.nkt_g = (int)((r + p.bk - 1) / p.bk);
    const int nkt = p.nkt_w0 + p.nkt_g;
    // k-split: smallest power of two that fills the CUs, keeping >= 4 k-tiles per chunk
    int ks = 1;
    while (ks < kNumXCD && (int64_t)p.n_mtiles * p.n_ntiles * ks < kNumCU && nkt / (2 * ks) >= 4) ks *= 2;
    p.ksplit = ks;
    // Gram
    p.gram_tiles = (int)((r + kGramTile - 1) / kGramTile);
    const int nupper = p.gram_tiles * (p.gram_tiles + 1) / 2;
    int gs = (kNumCU + nupper - 1) / nupper;
    const int max_split = p.nkt_w0 / 4 > 1 ? p.nkt_w0 / 4 : 1;
    if (gs > max_split) gs = max_split;
    if (gs < 1) gs = 1;
    p.gram_split = gs;
    p.ldg = (int64_t)align_up((size_t)r, (size_t)vec);
    const size_t rnp = (size_t)p.gram_tiles * kGramTile;
    size_t off = 0;
    p.off_gs = off;
    off = align_up(off + (size_t)r * p.ldg * esz, 256);
    p.off_gpart = off;
    off = align_up(off + (size_t)gs * rnp * rnp * 4, 256);
    p.off_pbase = off;
    off = align_up(off + (size_t)p.ksplit * d_out * 4, 256);
    p.off_pcross = off;
    off = align_up(off + (size_t)p.ksplit * p.n_ntiles * d_out * 4, 256);
    p.bytes = off;
    return p;
}

hipError_t launch_norm(const NormPlan& p, const void* W0, const void* A, const void* B, const float* m, float s,
                       float eps, float* wnorm, float* g, void* workspace, hipStream_t stream) {
    if (p.dtype == kF32) return norm_typed<float>(p, W0, A, B, m, s, eps, wnorm, g, workspace, stream);
    return norm_typed<bf16_t>(p, W0, A, B, m, s, eps, wnorm, g, workspace, stream);
}

}  // namespace dora
