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
//   1. gram_partial / gram_finalize: Gs = (s/2) A A^T (MFMA, split-K partials
//      of the upper 64 x 64 tiles summed in a fixed order, rounded once to
//      the operand dtype).
//   2. w0_pass: one streaming pass over W0.  Each workgroup owns BM rows of
//      W0, BN columns of r and a K-chunk of the extended contraction; W0 and A
//      (then B and Gs) tiles are staged through LDS and fed to MFMA with fp32
//      accumulation.  The W0 tile loader also accumulates ||W0_i||^2 from the
//      registers it already holds.  The epilogue dots each accumulator row
//      with B_i in registers, so U never reaches HBM: a workgroup writes BM
//      partial scalars (and BM partial base sums).
//   3. norm_finalize: sums the partials in a fixed order, forms n2, clamps,
//      takes the square root and divides m.
// At low rank (bf16, r <= 32) the Gram term is a sum over K-chunks of
// B_i A_c A_c^T B_i^T, so the W0 pass forms each chunk's term from the A
// fragments it already holds and no Gram kernel runs; where 16-row
// workgroups make exactly one round (and W0 has at most 2^25 elements) a
// single kernel (w0_rows_narrow) owns whole rows and also does step 3.
// Every reduction has a fixed order, so results are bitwise reproducible.
#include "dora_balance.h"
#include "dora_device.h"
#include "dora_gfx950.h"
#include "dora_launch.h"

namespace dora {
namespace {

constexpr int kNumCU = 256;
constexpr int kNumXCD = 8;

// a compile-time int carried by value (selects template paths from lambdas)
template <int V>
struct IntC {
    static constexpr int value = V;
};

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
    // DMA layout: k-step ks, lane group q reads logical chunk 4 ks + q of a
    // 128-byte row whose swizzle is sw.
    __device__ __forceinline__ static frag_t load_frag_swz(const char* row, int ks, int q, int sw) {
        return *reinterpret_cast<const bf16x8_t*>(row + (((ks * 4 + q) ^ sw) << 4));
    }
    __device__ __forceinline__ static float frag_sumsq(const frag_t& a) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = static_cast<float>(a[e]);
            s = fmaf(x, x, s);
        }
        return s;
    }
    // A fragment held as FL = 1 sixteen-byte register packet.
    static constexpr int FL = 1;
    __device__ __forceinline__ static frag_t frag_from_regs(const u32x4_t* r) {
        return __builtin_bit_cast(bf16x8_t, r[0]);
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
    // DMA layout: one k-step per tile; lane group q reads logical chunks 2q
    // and 2q + 1 (8 floats) of a 128-byte row whose swizzle is sw.
    __device__ __forceinline__ static frag_t load_frag_swz(const char* row, int ks, int q, int sw) {
        frag_t f;
        f.lo = *reinterpret_cast<const f32x4_t*>(row + (((ks * 8 + 2 * q) ^ sw) << 4));
        f.hi = *reinterpret_cast<const f32x4_t*>(row + (((ks * 8 + 2 * q + 1) ^ sw) << 4));
        return f;
    }
    __device__ __forceinline__ static float frag_sumsq(const frag_t& a) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(a.lo[e], a.lo[e], s);
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(a.hi[e], a.hi[e], s);
        return s;
    }
    // A fragment held as FL = 2 sixteen-byte register packets.
    static constexpr int FL = 2;
    __device__ __forceinline__ static frag_t frag_from_regs(const u32x4_t* r) {
        frag_t f;
        f.lo = __builtin_bit_cast(f32x4_t, r[0]);
        f.hi = __builtin_bit_cast(f32x4_t, r[1]);
        return f;
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
// 16 x 16 outputs.  A tile row holds BK elements = 128 bytes = 8 chunks.
template <typename E, int WM, int WN, int MT, int NT>
struct Tile {
    static constexpr int NW = WM * WN;
    static constexpr int NTH = NW * 64;
    static constexpr int BM = WM * MT * 16;
    static constexpr int BN = WN * NT * 16;
    static constexpr int BK = Mma<E>::BK;
    static constexpr int VEC = Mma<E>::VEC;
    static constexpr int CPR = BK / VEC;   // 16-byte chunks per tile row (8)
    static_assert(CPR == 8, "tile rows are 8 chunks");
    static_assert(NTH % CPR == 0, "a thread keeps the same chunk column across tiles");

    // Register-staged path (unaligned operands): rows padded by 16 bytes so
    // that the 16 rows one MFMA fragment read touches fall on distinct banks.
    static constexpr int LD = BK + VEC;
    static constexpr int LCH = (BM * CPR + NTH - 1) / NTH;
    static constexpr int RCH = (BN * CPR + NTH - 1) / NTH;
    static constexpr int BUF = (BM + BN) * LD;
    static constexpr int STAGED_BYTES = 2 * BUF * (int)sizeof(E);

    // LDS-DMA path (aligned operands): unpadded 128-byte rows, chunk-swizzled;
    // a ring of LS stages for the left operand (the HBM stream) and RS stages
    // for the right operand (L2-resident).
    static constexpr int LS = 3, RS = 2;
    static constexpr int LBYTES = BM * 128, RBYTES = BN * 128;
    static constexpr int DMA_BYTES = LS * LBYTES + RS * RBYTES;
    static constexpr int LPW = BM / 8 / NW;   // left DMA instructions per wave per tile
    static_assert(BM / 8 % NW == 0, "left tile splits evenly across waves");

};

// Register-staged main loop, used when operands are not 16-byte aligned.
// Streams k-tiles [kt_begin, kt_end) of `c` through double-buffered LDS into
// the MFMA accumulators.  When base_dst is set, the squares of every phase-0
// left element are summed and row partials written to base_dst[m].
template <typename E, int WM, int WN, int MT, int NT>
__device__ __forceinline__ void mainloop_staged(const Contraction& c, int64_t m0, int64_t n0, int kt_begin,
                                                int kt_end, float* base_dst, int64_t d_out,
                                                f32x4_t (&acc)[MT][NT], char* smem) {
    typedef Tile<E, WM, WN, MT, NT> TL;
    typedef Mma<E> M;
    E* lds = reinterpret_cast<E*>(smem);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int cc = tid % TL::CPR;   // chunk column, fixed for this thread

    u32x4_t lreg[TL::LCH], rreg[TL::RCH];
    float bsum[TL::LCH];
#pragma unroll
    for (int j = 0; j < TL::LCH; ++j) bsum[j] = 0.0f;

    auto load_tile = [&](int kt) {
        const bool ph0 = kt < c.nkt0;
        const Operand& L = ph0 ? c.left0 : c.left1;
        const Operand& R = ph0 ? c.right0 : c.right1;
        const int64_t k = (int64_t)(ph0 ? kt : kt - c.nkt0) * TL::BK + cc * TL::VEC;
#pragma unroll
        for (int j = 0; j < TL::LCH; ++j) {
            const int ch = tid + j * TL::NTH;
            if (TL::BM * TL::CPR % TL::NTH == 0 || ch < TL::BM * TL::CPR)
                lreg[j] = load_chunk<E, false>(L, m0 + ch / TL::CPR, k);
        }
#pragma unroll
        for (int j = 0; j < TL::RCH; ++j) {
            const int ch = tid + j * TL::NTH;
            if (TL::BN * TL::CPR % TL::NTH == 0 || ch < TL::BN * TL::CPR)
                rreg[j] = load_chunk<E, false>(R, n0 + ch / TL::CPR, k);
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
                if (base_dst && ph0) bsum[j] += chunk_sumsq<E>(lreg[j]);
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

    if (kt_begin < kt_end) {
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
    if (base_dst) {
        // the 8 threads of a row hold its 8 chunk columns
#pragma unroll
        for (int j = 0; j < TL::LCH; ++j) {
            float v = bsum[j];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            const int ch = tid + j * TL::NTH;
            const int64_t m = m0 + ch / TL::CPR;
            if (cc == 0 && ch < TL::BM * TL::CPR && m < d_out) base_dst[m] = v;
        }
    }
}


// Chunk swizzle of the DMA layout: logical chunk c of tile row i sits in
// physical slot c ^ swz(i).  Any 8 consecutive rows, and the even (odd) rows
// of any aligned 16 rows, map one logical chunk to 8 distinct slots, so a
// 16-row fragment read is free of bank conflicts with 32 or 64 banks.  Within
// a DMA group of 8 rows the swizzle depends only on the group's parity.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }


// One operand of one phase as the DMA sees it: a buffer starting at the
// workgroup's first tile row, sized to the rows that exist, so rows past the
// operand read zeros.  A lane's chunk depends on the parity of its 8-row
// group (the swizzle flips with row bit 3), so offsets come in two flavours.
struct DmaSrc {
    i32x4_t rsrc;
    int ld_bytes, kmax_bytes;
    int off_even, off_odd;       // lane byte offset inside an even / odd group
    int chunk_even, chunk_odd;   // byte offset of the lane's chunk within its row
};

template <typename E>
__device__ __forceinline__ DmaSrc make_dma_src(const Operand& o, int64_t row0, int lane) {
    DmaSrc d;
    const int64_t ldb = o.ld * (int64_t)sizeof(E);
    const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<const char*>(o.p) + row0 * ldb);
    int64_t bytes = (o.rows - row0) * ldb;
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7ffffff0) bytes = 0x7ffffff0;
    d.rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    d.rsrc[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
    d.rsrc[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    d.rsrc[3] = 0x00020000;
    d.ld_bytes = (int)ldb;
    d.kmax_bytes = (int)(o.kmax * (int64_t)sizeof(E));
    const int r_in = lane >> 3;
    d.chunk_even = ((lane & 7) ^ r_in) * 16;
    d.chunk_odd = ((lane & 7) ^ r_in ^ 1) * 16;
    d.off_even = r_in * (int)ldb + d.chunk_even;
    d.off_odd = r_in * (int)ldb + d.chunk_odd;
    return d;
}

// Enqueue the DMA of tile rows [0, ROWS) at K byte offset k0b into LDS at
// dst.  One instruction moves a group of 8 rows (1 KiB): lane l fills slot
// l % 8 of row l / 8 with the logical chunk the swizzle puts there.  The
// groups are dealt to waves [W_FIRST, W_FIRST + W_COUNT); other waves issue
// nothing.  Chunks past the K extent of the operand read zeros.  AUX is the
// loads' cache policy (non-temporal for W0 and B, read once).
template <int ROWS, int W_FIRST, int W_COUNT, int AUX = 0>
__device__ __forceinline__ void dma_tile(const DmaSrc& d, int k0b, char* dst, int wave, int tile_kbytes) {
    constexpr int GROUPS = ROWS / 8;
    if (wave < W_FIRST || wave >= W_FIRST + W_COUNT) return;
    const int w = wave - W_FIRST;
    const bool full = k0b + tile_kbytes <= d.kmax_bytes;
    const int kleft = d.kmax_bytes - k0b;
#pragma unroll
    for (int q = 0; q < (GROUPS + W_COUNT - 1) / W_COUNT; ++q) {
        const int grp = w + q * W_COUNT;
        if (GROUPS % W_COUNT == 0 || grp < GROUPS) {
            const bool odd = grp & 1;
            int voff = (odd ? d.off_odd : d.off_even) + grp * 8 * d.ld_bytes + k0b;
            if (!full) voff = (odd ? d.chunk_odd : d.chunk_even) < kleft ? voff : kOutOfRange;
            raw_buffer_load_lds(d.rsrc, (lds_void_t*)(dst + grp * 1024), 16, voff, 0, 0, AUX);
        }
    }
}

// LDS-DMA main loop for 16-byte aligned operands.  Tiles go global -> LDS
// without passing through registers (global -> VGPR loads interleaved with
// MFMA measure ~40% slower): the left operand (W0, streamed from HBM) runs
// LS = 3 stages deep, i.e. is requested two k-tiles ahead, the right operand
// (A or Gs, L2-resident) RS = 2 stages, one tile ahead.  Per k-tile j:
//   wait for this thread's DMA of tiles <= j (only left(j+1) may be pending),
//   barrier (all threads' DMA landed; stage of tile j-1 free),
//   enqueue right(j+1) and left(j+2), then MFMA over tile j.
// The walk over the k-tiles starts at tile `rot`: with a power-of-two row
// pitch, workgroups that walk K in lockstep read the same column offset of
// every row and pile onto a few memory channels; rotating the start spreads
// them.  The base term is summed from the left fragments the MFMAs consume;
// the WN waves sharing a row block split its 16-row blocks between them.
// With GRAM (bf16, one n-tile covering r), the right fragments also feed this
// K range's Gram blocks G_c = A_c A_c^T: wave wn accumulates block (b1, b2)
// of 16-row blocks of the tile's A rows, b1 its own blocks wn NT + j, b2 >=
// b1 any block, in gacc[j * WN * NT + b2]; the waves together cover the
// upper half once.
template <typename E, int WM, int WN, int MT, int NT, bool ROLES, bool GRAM = false, int NG = 1>
__device__ __forceinline__ void mainloop_dma(const Contraction& c, int64_t m0, int64_t n0, int kt_begin,
                                             int kt_end, int rot, float* base_dst, int64_t d_out,
                                             f32x4_t (&acc)[MT][NT], char* smem, f32x4_t (&gacc)[NG]) {
    constexpr int NBLK = WN * NT;   // 16-row blocks of the right tile
    static_assert(!GRAM || NG == NT * NBLK, "one Gram accumulator per (own block, any block)");
    typedef Tile<E, WM, WN, MT, NT> TL;
    typedef Mma<E> M;
    static_assert(TL::NW % 2 == 0, "DMA lane offsets assume an even wave count");
    constexpr int TKB = TL::BK * (int)sizeof(E);   // bytes of K per tile row (128)
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int q = lane >> 4;
    char* lring = smem;
    char* rring = smem + TL::LS * TL::LBYTES;

    const DmaSrc L0 = make_dma_src<E>(c.left0, m0, lane);
    const DmaSrc R0 = make_dma_src<E>(c.right0, n0, lane);
    const DmaSrc L1 = make_dma_src<E>(c.left1, m0, lane);
    const DmaSrc R1 = make_dma_src<E>(c.right1, n0, lane);
    // Load roles.  Vector-memory loads complete in issue order per wave, so a
    // wave that issues both streams makes every L2-resident right tile wait
    // behind the HBM-latency left tile issued before it.  With ROLES, wave 0
    // issues all left (W0) DMA and waves 1.. all right (A / Gs) DMA, and each
    // waits only on its own queue.
    constexpr int LW0 = 0, LWN = ROLES ? 1 : TL::NW;
    constexpr int RW0 = ROLES ? 1 : 0, RWN = ROLES ? TL::NW - 1 : TL::NW;
    constexpr int LPI = (TL::BM / 8 + LWN - 1) / LWN;   // left DMA instructions per issuing wave per tile

    int lrow[MT], lsw[MT], rrow[NT], rsw[NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        lrow[mt] = wm * MT * 16 + mt * 16 + (lane & 15);
        lsw[mt] = swz(lrow[mt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        rrow[nt] = wn * NT * 16 + nt * 16 + (lane & 15);
        rsw[nt] = swz(rrow[nt]);
    }
    float bs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bs[mt] = 0.0f;

    const int n = kt_end - kt_begin;
    bool base_tile = false;   // the tile being computed is a W0 | A one
    // k-tile visited at step i (the walk starts at a rotated tile)
    auto tile = [&](int i) __attribute__((always_inline)) {
        int t = i + rot;
        if (t >= n) t -= n;
        return kt_begin + t;
    };
    auto issue_left = [&](int i, int stage) __attribute__((always_inline)) {
        const int kt = tile(i);
        char* dst = lring + stage * TL::LBYTES;
        if (kt < c.nkt0)
            dma_tile<TL::BM, LW0, LWN, kCachePolicyNT>(L0, kt * TKB, dst, wave, TKB);
        else
            dma_tile<TL::BM, LW0, LWN, kCachePolicyNT>(L1, (kt - c.nkt0) * TKB, dst, wave, TKB);
    };
    auto issue_right = [&](int i, int stage) __attribute__((always_inline)) {
        const int kt = tile(i);
        char* dst = rring + stage * TL::RBYTES;
        if (kt < c.nkt0)
            dma_tile<TL::BN, RW0, RWN>(R0, kt * TKB, dst, wave, TKB);
        else
            dma_tile<TL::BN, RW0, RWN>(R1, (kt - c.nkt0) * TKB, dst, wave, TKB);
    };
    auto compute = [&](const char* Lt, const char* Rt, bool base) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < TL::BK / 32; ++ks) {
            typename M::frag_t a[MT], b[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt] = M::load_frag_swz(Lt + lrow[mt] * 128, ks, q, lsw[mt]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b[nt] = M::load_frag_swz(Rt + rrow[nt] * 128, ks, q, rsw[nt]);
            if (base) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    if (mt % WN == wn) bs[mt] += M::frag_sumsq(a[mt]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) M::mma(acc[mt][nt], a[mt], b[nt]);
            if constexpr (GRAM) {
                // base is set on the W0 | A k-tiles only, the ones G_c sums over
                if (base_tile) {
#pragma unroll
                    for (int b2 = 0; b2 < NBLK; ++b2) {
                        const int row = b2 * 16 + (lane & 15);
                        const typename M::frag_t f = M::load_frag_swz(Rt + row * 128, ks, q, swz(row));
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            if (b2 >= wn * NT + j) M::mma(gacc[j * NBLK + b2], b[j], f);
                    }
                }
            }
        }
    };

    // Per k-tile j: wait for this thread's DMA of tiles <= j (only left(j+1)
    // may still be in flight), barrier (every thread's DMA landed, and the
    // stages of tile j-1 are free), enqueue right(j+1) and left(j+2), then
    // MFMA over tile j.  Left runs 3 stages deep, right 2.
    if (n > 0) {
        issue_left(0, 0);
        issue_right(0, 0);
        if (n > 1) issue_left(1, 1);
        int ls = 0, rs = 0;   // stages holding the tile of step j
        for (int j = 0; j < n; ++j) {
            // this wave's DMA of tile j is done; only its left(j+1) may be pending
            const bool left_issuer = wave >= LW0 && wave < LW0 + LWN;
            if (j + 1 < n && left_issuer)
                wait_vmcnt<ROLES ? LPI : TL::LPW>();
            else
                wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            const int rs_next = rs ^ 1;
            const int ls_next2 = ls == 0 ? 2 : ls - 1;   // (ls + 2) % 3
            if (j + 1 < n) issue_right(j + 1, rs_next);
            if (j + 2 < n) issue_left(j + 2, ls_next2);
            base_tile = tile(j) < c.nkt0;
            compute(lring + ls * TL::LBYTES, rring + rs * TL::RBYTES, base_dst != nullptr && base_tile);
            ls = ls == 2 ? 0 : ls + 1;
            rs = rs_next;
        }
    }
    __builtin_amdgcn_s_barrier();   // LDS is free for the caller's epilogue
    if (base_dst) {
        // lanes l, l+16, l+32, l+48 hold the four chunk columns of one row
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (mt % WN != wn) continue;
            float v = bs[mt];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            const int64_t m = m0 + wm * MT * 16 + mt * 16 + lane;
            if (lane < 16 && m < d_out) base_dst[m] = v;
        }
    }
}

// Buffer load of 16 bytes per lane into registers; offsets at or beyond the
// buffer's size read zeros.
__device__ i32x4_t raw_buffer_load_b128(i32x4_t rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4i32");


// One operand of one phase as seen by direct-to-register fragment loads: a
// buffer starting at the first of the 16-row blocks this wave reads.  Lane l
// reads row l % 16 of a block, K elements 8 (l / 16) .. 8 (l / 16) + 7 of a
// 32-element k-step (FL packets of 16 bytes).
struct FragSrc {
    i32x4_t rsrc;
    int ld_bytes, kmax_bytes, lane_off, kq_bytes;
};

template <typename E>
__device__ __forceinline__ FragSrc make_frag_src(const Operand& o, int64_t row0, int lane) {
    FragSrc f;
    const int64_t ldb = o.ld * (int64_t)sizeof(E);
    const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<const char*>(o.p) + row0 * ldb);
    int64_t bytes = (o.rows - row0) * ldb;
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7ffffff0) bytes = 0x7ffffff0;
    f.rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    f.rsrc[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
    f.rsrc[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    f.rsrc[3] = 0x00020000;
    f.ld_bytes = (int)ldb;
    f.kmax_bytes = (int)(o.kmax * (int64_t)sizeof(E));
    f.kq_bytes = (lane >> 4) * 8 * (int)sizeof(E);
    f.lane_off = (lane & 15) * (int)ldb + f.kq_bytes;
    return f;
}

// f if p else g, field by field (p uniform: scalar selects, no branch).
__device__ __forceinline__ FragSrc select_src(bool p, const FragSrc& f, const FragSrc& g) {
    FragSrc o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o.rsrc[q] = p ? f.rsrc[q] : g.rsrc[q];
    o.ld_bytes = p ? f.ld_bytes : g.ld_bytes;
    o.kmax_bytes = p ? f.kmax_bytes : g.kmax_bytes;
    o.lane_off = p ? f.lane_off : g.lane_off;
    o.kq_bytes = f.kq_bytes;
    return o;
}

// Load the fragments of NB consecutive 16-row blocks for every k-step of the
// k-tile starting at element k0: regs[(ks * NB + b) * FL + h].  With live
// false every offset is out of range: the loads read zeros and move no data.
// AUX is the loads' cache policy.
template <typename E, int NB, int AUX = 0>
__device__ __forceinline__ void load_frags(const FragSrc& f, int64_t k0, u32x4_t* regs, bool live = true) {
    typedef Mma<E> M;
    constexpr int FR = M::BK / 32, FL = M::FL;
#pragma unroll
    for (int ks = 0; ks < FR; ++ks) {
        const int kb = (int)((k0 + ks * 32) * (int64_t)sizeof(E));
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int h = 0; h < FL; ++h) {
                const bool ok = live && kb + f.kq_bytes + h * 16 < f.kmax_bytes;
                const int voff = ok ? f.lane_off + b * 16 * f.ld_bytes + kb + h * 16 : kOutOfRange;
                regs[(ks * NB + b) * FL + h] =
                    __builtin_bit_cast(u32x4_t, raw_buffer_load_b128(f.rsrc, voff, 0, AUX));
            }
        }
    }
}

// W0 pass main loop, narrow form (small r: 4 waves stacked along d_out, MT
// blocks each, all NT blocks of r per wave).  Nothing is shared between
// waves, so both operands are loaded straight into registers, D register
// sets deep (D - 1 tiles in flight), with no LDS and no barrier.  K-walk
// rotated as in the wide form.
// Every step issues its loads unconditionally: the phase picks the operand
// buffers by scalar selects, and the walk is padded to a multiple of D with
// empty tiles whose loads are out of range (zeros, no data moved; they add
// nothing to U, the base or the Gram blocks).  The load stream is then the
// same every step, so the compiler's own waits on each register set stay at
// (D - 2) tiles in flight; loads under a branch made it wait for every
// outstanding load before each MFMA, i.e. one memory latency per k-tile.
// One wave's rows [mrow0, mrow0 + 16 MT) over k-tiles [kt_begin, kt_end).
// With GIP, the right fragments (rows of A) also feed this K range's Gram
// blocks G_c = A_c A_c^T: gacc holds the upper blocks (b1 <= b2) in order.
// bsum[mt] receives the base partial of row mrow0 + mt * 16 + lane % 16 in
// every lane (zero without want_base or for an empty range).
template <typename E, int MT, int NT, bool GIP, int NG, int D>
__device__ __forceinline__ void mainloop_w0_narrow(const Contraction& c, int64_t mrow0, int64_t n0, int kt_begin,
                                                   int kt_end, int rot, bool want_base, f32x4_t (&acc)[MT][NT],
                                                   f32x4_t (&gacc)[NG], float (&bsum)[MT]) {
    typedef Mma<E> M;
    constexpr int FR = M::BK / 32, FL = M::FL;
    constexpr int NLW = FR * MT * FL, NRW = FR * NT * FL;   // loads per wave per tile
    constexpr int PER = NLW + NRW;
    const int lane = threadIdx.x & 63;
    const int n = kt_end - kt_begin;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bsum[mt] = 0.0f;
    if (n <= 0) return;
    const FragSrc L0 = make_frag_src<E>(c.left0, mrow0, lane);
    const FragSrc L1 = make_frag_src<E>(c.left1, mrow0, lane);
    const FragSrc R0 = make_frag_src<E>(c.right0, n0, lane);
    const FragSrc R1 = make_frag_src<E>(c.right1, n0, lane);
    float bs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bs[mt] = 0.0f;

    // k-tile of walk step i (steps past the walk: its first tile, loaded empty)
    auto tile = [&](int i) __attribute__((always_inline)) {
        int t = i + rot;
        if (t >= n) t -= n;
        return i < n ? kt_begin + t : kt_begin;
    };
    auto load = [&](int i, u32x4_t* regs) __attribute__((always_inline)) {
        const int kt = tile(i);
        const bool ph0 = kt < c.nkt0;
        const int64_t k0 = (int64_t)(ph0 ? kt : kt - c.nkt0) * M::BK;
        load_frags<E, MT>(select_src(ph0, L0, L1), k0, regs, i < n);
        load_frags<E, NT>(select_src(ph0, R0, R1), k0, regs + NLW, i < n);
    };
    auto compute = [&](const u32x4_t* regs, bool base, bool gram) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < FR; ++ks) {
            typename M::frag_t a[MT], b[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                a[mt] = M::frag_from_regs(regs + (ks * MT + mt) * FL);
                if (base) bs[mt] += M::frag_sumsq(a[mt]);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                b[nt] = M::frag_from_regs(regs + NLW + (ks * NT + nt) * FL);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) M::mma(acc[mt][nt], a[mt], b[nt]);
            }
            if constexpr (GIP) {
                if (gram) {
                    int q = 0;
#pragma unroll
                    for (int b1 = 0; b1 < NT; ++b1)
#pragma unroll
                        for (int b2 = b1; b2 < NT; ++b2) M::mma(gacc[q++], b[b1], b[b2]);
                }
            }
        }
    };
    static_assert(D >= 2 && (D - 1) * PER < 64, "register ring depth");
    // step t waits until only steps t + 1 .. t + D - 2 are in flight, then
    // step t + D - 1 goes into the set of step t - 1 (already consumed)
    const int nsteps = (n + D - 1) / D * D;
    u32x4_t sets[D][PER];
#pragma unroll
    for (int j = 0; j < D - 1; ++j) load(j, sets[j]);
    for (int i = 0; i < nsteps; i += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int t = i + j;
            wait_vmcnt<(D - 2) * PER>();
            load(t + D - 1, sets[(j + D - 1) % D]);
            const bool ph0 = tile(t) < c.nkt0;
            compute(sets[j], want_base && ph0, ph0);
        }
    }
    wait_vmcnt<0>();   // the empty loads issued past the walk
    if (want_base) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float v = bs[mt];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            bsum[mt] = v;
        }
    }
}

template <typename E, int WM, int WN, int MT, int NT, bool ALIGNED>
__device__ __forceinline__ void mainloop(const Contraction& c, int64_t m0, int64_t n0, int kt_begin, int kt_end,
                                         int rot, float* base_dst, int64_t d_out, f32x4_t (&acc)[MT][NT],
                                         char* smem) {
    if constexpr (ALIGNED) {
        f32x4_t none[1];
        mainloop_dma<E, WM, WN, MT, NT, false>(c, m0, n0, kt_begin, kt_end, rot, base_dst, d_out, acc, smem, none);
    }
    else
        mainloop_staged<E, WM, WN, MT, NT>(c, m0, n0, kt_begin, kt_end, base_dst, d_out, acc, smem);
}

// ------------------------------------------------------------- W0 pass
// Balanced K split of the large-tile pass (dora_balance.h): each workgroup
// walks one or more segments (k-tile ranges of one m-tile), each with its
// own epilogue and partial slot.  nwg = 0: the uniform split.

struct W0PassArgs {
    Contraction c;
    const void* B;          // [d_out, r], for the row-dot epilogue
    int64_t d_out, r;
    int ksplit, n_mtiles, n_ntiles;
    int xcd_map;            // workgroups on one XCD share (n-tile, k-chunk)
    float* part_base;       // [ksplit][d_out]
    float* part_cross;      // [n_ntiles * ksplit][d_out]
    float half_s;           // s / 2, for the Gram term formed inside the pass
    Balance bal;            // large-tile pass only
};

template <int WM, int WN, int MT, int NT, bool ALIGNED>
struct W0Form {
    static constexpr bool WIDE = ALIGNED && WM == 1 && WN >= 4 && MT == 8;
    static constexpr bool NARROW = ALIGNED && WN == 1;
};

// Register sets per wave of the narrow loops: two, i.e. one k-tile in flight
// while the previous one is computed.  Measured on MI355X at r <= 64: two
// sets were the fastest or within 2% of it on every shape tried (4096^2
// r = 32: 16.7 us against 17.6 with four; 28672 x 8192 r = 32: 130 against
// 131; 8192^2 r = 64: 70.7 against 74.1), three and six were slower: with
// hundreds of waves streaming W0, more requests in flight per wave only add
// contention in the memory system.
constexpr int kNarrowDepth = 2;

// bf16 tiles whose one n-tile covers r <= 64 (narrow, and the wide 64-column
// tile) form the Gram term inside the W0 pass.  The norm's Gram term is a sum over
// K of per-chunk terms,
//   B_i G B_i^T = sum_c B_i (A_c A_c^T) B_i^T,
// so each K-chunk workgroup builds G_c from the A fragments it already
// holds and adds (s/2) B G_c to its U accumulators before the row dot with
// B, exactly as the extended contraction adds B Gs with the whole Gram.  No
// Gram kernels run and the contraction has no Gs k-tiles.  A narrow wave
// holds all of the tile's A rows and builds every upper 16 x 16 block of
// G_c; wide waves split the blocks (mainloop_dma).  Every m-tile's
// workgroups build the same G_c, so the in-pass Gram grows with d_out while
// the Gram kernels do not: measured on MI355X, the wide 128-column tile lost
// with it (8192^2 r = 128 54.8 -> 61.7 us, 28672 x 8192 153.0 -> 194.8 us;
// 4096^2 33.7 -> 32.6 us), the 64-column one won everywhere (4096^2 r = 64
// 30.2 -> 25.3 us, r = 40 30.0 -> 25.0, 8192 x 4096 r = 64 34.5 -> 29.7,
// 8192^2 48.2 -> 44.6, 1024 x 8192 32.6 -> 25.6).
template <typename E, int WN, int NT, bool ALIGNED>
struct GramInPass {
    static constexpr bool NARROW = ALIGNED && WN == 1 && NT <= 4 && sizeof(E) == 2;
    static constexpr bool WIDE = ALIGNED && WN == 4 && NT == 1 && sizeof(E) == 2;
    static constexpr bool value = NARROW || WIDE;
    static constexpr int NBLK = WN * NT;                        // 16-row blocks of A in the tile
    static constexpr int NG = NARROW ? NT * (NT + 1) / 2 : (WIDE ? NT * NBLK : 1);
    static constexpr int RP = WIDE ? NBLK * 16 : (NT <= 2 ? 32 : 64);   // K of the B Gs product (narrow: zero-padded)
    static constexpr int PITCH = RP * 2 + 16;                   // Gs tile row bytes in LDS
    static constexpr int BYTES = value ? RP * PITCH : 0;
};

// One operand as the 128-byte-row DMA sees it; lane l moves slot l % 8 of row
// l / 8 of an 8-row group (1 KiB per instruction, eight whole lines).  The
// row and K offsets of an instruction are wave-uniform, so they move the
// buffer's base address (scalar registers) while the per-lane part stays one
// fixed VGPR; the buffer is shrunk by the same amount, so rows past the
// operand still read zeros.
struct Dma64 {
    uint32_t base_lo, base_hi;     // address of the workgroup's first row
    int bytes;                     // bytes from there to the operand's end (clamped to 31 bits)
    int ld_bytes, kmax_bytes;
};

__device__ __forceinline__ Dma64 make_dma64(const Operand& o, int64_t row0) {
    Dma64 d;
    const int64_t ldb = o.ld * 2;
    const uint64_t base = reinterpret_cast<uint64_t>(static_cast<const char*>(o.p) + row0 * ldb);
    int64_t bytes = (o.rows - row0) * ldb;
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7ffffff0) bytes = 0x7ffffff0;
    d.base_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    d.base_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
    d.bytes = __builtin_amdgcn_readfirstlane((int)bytes);
    d.ld_bytes = __builtin_amdgcn_readfirstlane((int)ldb);
    d.kmax_bytes = __builtin_amdgcn_readfirstlane((int)(o.kmax * 2));
    return d;
}

// The register-free K walk of the narrow forms (bf16, aligned, the Gram
// term formed in the pass).  Each wave moves its own 64-element k-tiles of
// W0 (its MT * 16 rows from mrow0) and of A (NT * 16 rows from n0, zeros past
// r) by LDS DMA into a private ring of D stages: whole 128-byte rows, so
// every request to L2 is one full line (register-fed fragment loads can only
// ask for 64 bytes of a row at a time, and a CU keeps only so many requests
// in flight).  The fragments are read from the ring with the 128-byte-row
// swizzle; per k-tile the MFMAs, base term and Gram blocks are those of the
// register-fed loop, and so is the rotated walk.  A wave waits only for its
// own loads, so the walk has no barriers.
template <int MT, int NT, int NWAVES, int D>
struct NarrowRing {
    static constexpr int ROWS = (MT + NT) * 16;
    static constexpr int STAGE = ROWS * 128;             // bytes per stage
    static constexpr int PER = ROWS / 8;                 // DMA instructions per stage
    static constexpr int BYTES = NWAVES * D * STAGE;
    static_assert(D >= 2 && (D - 2) * PER < 64, "vmcnt range");
};

template <int MT, int NT, int NG, int D>
__device__ __forceinline__ void mainloop_narrow_dma(const Contraction& c, int64_t mrow0, int64_t n0, int kt_begin,
                                                    int kt_end, int rot, bool want_base, char* ring,
                                                    f32x4_t (&acc)[MT][NT], f32x4_t (&gacc)[NG],
                                                    float (&bsum)[MT]) {
    typedef Mma<bf16_t> M;
    typedef NarrowRing<MT, NT, 1, D> RR;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = kt_end - kt_begin;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bsum[mt] = 0.0f;
    if (n <= 0) return;
    const Dma64 W = make_dma64(c.left0, mrow0);
    const Dma64 A = make_dma64(c.right0, n0);
    // lane l moves slot l % 8 of row l / 8 of an 8-row group, carrying
    // logical chunk slot ^ swz(row) = (l % 8) ^ (l / 8) ^ (group parity)
    const int ce = ((lane & 7) ^ (lane >> 3)) * 16, co = ce ^ 16;
    const int we = (lane >> 3) * W.ld_bytes + ce, wo = (lane >> 3) * W.ld_bytes + co;
    const int ae = (lane >> 3) * A.ld_bytes + ce, ao = (lane >> 3) * A.ld_bytes + co;
    char* mine = ring + wave * D * RR::STAGE;
    // aux: the load's cache policy (W0 is read once: non-temporal)
    auto group = [&](const Dma64& d, int g, int lane_off, int chunk_b, int k0b, char* dst, auto aux)
        __attribute__((always_inline)) {
        const int kleft = d.kmax_bytes - k0b;
        const int voff = chunk_b < kleft ? lane_off : kOutOfRange;
        const int off = g * 8 * d.ld_bytes + k0b;
        const int left = d.bytes > off ? d.bytes - off : 0;
        const uint64_t addr = (((uint64_t)d.base_hi << 32) | d.base_lo) + (uint32_t)off;
        i32x4_t rs;
        rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
        rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
        rs[2] = __builtin_amdgcn_readfirstlane(left);
        rs[3] = 0x00020000;
        raw_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff, 0, 0, decltype(aux)::value);
    };
    // k-tile of walk step i (the walk starts at a rotated tile)
    auto tile = [&](int i) __attribute__((always_inline)) {
        int t = i + rot;
        if (t >= n) t -= n;
        return kt_begin + t;
    };
    // step i's loads into stage i % D; steps past the walk load zeros
    auto issue = [&](int i) __attribute__((always_inline)) {
        const bool valid = i < n;
        const int k0b = tile(valid ? i : 0) * 128;
        char* st = mine + (i % D) * RR::STAGE;
#pragma unroll
        for (int g = 0; g < MT * 2; ++g)
            group(W, g, valid ? ((g & 1) ? wo : we) : kOutOfRange, (g & 1) ? co : ce, k0b, st + g * 1024,
                  IntC<kCachePolicyNT>{});
#pragma unroll
        for (int g = 0; g < NT * 2; ++g)
            group(A, g, valid ? ((g & 1) ? ao : ae) : kOutOfRange, (g & 1) ? co : ce, k0b,
                  st + MT * 16 * 128 + g * 1024, IntC<0>{});
    };
    const int fr = lane & 15, q = lane >> 4, sw = swz(fr);
    const float on = want_base ? 1.0f : 0.0f;
    float bs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) bs[mt] = 0.0f;
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(i);
    for (int t = 0; t < n; ++t) {
        wait_vmcnt<(D - 2) * RR::PER>();        // step t landed
        __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): this wave's reads of step t - 1 are done
        issue(t + D - 1);                      // into step t - 1's stage
        const char* st = mine + (t % D) * RR::STAGE;
#pragma unroll
        for (int ks = 0; ks < M::BK / 32; ++ks) {
            M::frag_t af[MT], b[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                af[mt] = M::load_frag_swz(st + (mt * 16 + fr) * 128, ks, q, sw);
                bs[mt] = fmaf(on, M::frag_sumsq(af[mt]), bs[mt]);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                b[nt] = M::load_frag_swz(st + (MT * 16 + nt * 16 + fr) * 128, ks, q, sw);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) M::mma(acc[mt][nt], af[mt], b[nt]);
            }
            int g = 0;
#pragma unroll
            for (int b1 = 0; b1 < NT; ++b1)
#pragma unroll
                for (int b2 = b1; b2 < NT; ++b2) M::mma(gacc[g++], b[b1], b[b2]);
        }
    }
    wait_vmcnt<0>();   // the empty loads issued past the walk
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        float v = bs[mt];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        bsum[mt] = v;
    }
}

// The narrowest register-fed form (r <= 16) is held to three workgroups per
// CU (168 VGPRs, no spills): tall projections run several rounds of its
// workgroups, and with the Gram blocks it would otherwise drop to two.
template <typename E, int WM, int WN, int MT, int NT, bool ALIGNED>
__global__ __launch_bounds__(WM * WN * 64, (ALIGNED && WN == 1 && NT == 1) ? 3 : 1) void w0_pass(W0PassArgs a) {
    typedef Tile<E, WM, WN, MT, NT> TL;
    typedef W0Form<WM, WN, MT, NT, ALIGNED> F;
    static_assert(!ALIGNED || F::WIDE || F::NARROW, "aligned W0 pass needs the wide or narrow form");
    constexpr int RED_BYTES = WN * TL::BM * 4;
    // epilogue staging of the workgroup's B tile: rows padded by 16 bytes so
    // that the four row groups one fragment read touches use distinct banks
    constexpr int B_SLOTS = TL::BN * (int)sizeof(E) / 16 + 1;   // 16-byte slots per row
    constexpr int B_PITCH = B_SLOTS * 16;
    constexpr int B_BYTES = ALIGNED ? TL::BM * B_PITCH : 0;
    constexpr int EPI = B_BYTES + RED_BYTES;
    typedef GramInPass<E, WN, NT, ALIGNED> GIP;
    constexpr int EPI_ALL = EPI + GIP::BYTES;
    constexpr int WIDE_BYTES = TL::DMA_BYTES;
    // the narrow form with the Gram term in the pass walks K through per-wave
    // LDS-DMA rings (mainloop_narrow_dma): two workgroups per CU at r <= 32,
    // one at r <= 64
    constexpr bool RING = F::NARROW && GIP::value;
    constexpr int RING_D = NT == 1 ? 3 : 2;
    constexpr int RING_BYTES = RING ? NarrowRing<MT, NT, WM, RING_D>::BYTES : 0;
    constexpr int MAIN = F::WIDE ? WIDE_BYTES : (F::NARROW ? RING_BYTES : TL::STAGED_BYTES);
    __shared__ __attribute__((aligned(1024))) char smem[MAIN > EPI_ALL ? MAIN : EPI_ALL];

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
    f32x4_t gacc[GIP::NG];
#pragma unroll
    for (int q = 0; q < GIP::NG; ++q) gacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    float* base_dst = base_rows ? a.part_base + (int64_t)kc * a.d_out : nullptr;
    // rotated start of the K walk (see mainloop_dma)
    const int nk = kt_end - kt_begin;
    const int rot = nk > 0 ? (int)(((unsigned)id * 7u + ((unsigned)id >> 3) * 3u) % (unsigned)nk) : 0;
    if constexpr (F::WIDE)
        mainloop_dma<E, WM, WN, MT, NT, false, GIP::WIDE, GIP::NG>(a.c, m0, n0, kt_begin, kt_end, rot, base_dst,
                                                                   a.d_out, acc, smem, gacc);
    else if constexpr (F::NARROW) {
        const int64_t mrow0 = m0 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * MT * 16;
        float bsum[MT];
        if constexpr (RING) {
            mainloop_narrow_dma<MT, NT, GIP::NG, RING_D>(a.c, mrow0, n0, kt_begin, kt_end, rot, base_dst != nullptr,
                                                         smem, acc, gacc, bsum);
            __syncthreads();   // every wave is done with the ring before the epilogue reuses it
        } else {
            mainloop_w0_narrow<E, MT, NT, GIP::value, GIP::NG, kNarrowDepth>(a.c, mrow0, n0, kt_begin, kt_end, rot,
                                                                             base_dst != nullptr, acc, gacc, bsum);
        }
        if (base_dst) {
            const int lane = threadIdx.x & 63;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int64_t m = mrow0 + mt * 16 + lane;
                if (lane < 16 && m < a.d_out) base_dst[m] = bsum[mt];
            }
        }
    }
    else
        mainloop_staged<E, WM, WN, MT, NT>(a.c, m0, n0, kt_begin, kt_end, base_dst, a.d_out, acc, smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // cross partial: sum_n B[m][n] * acc[m][n] over this workgroup's columns.
    // acc[mt][nt][j] is row wm*MT*16 + mt*16 + 4*(lane/16) + j, column
    // wn*NT*16 + nt*16 + lane%16 of the tile.
    float* red = reinterpret_cast<float*>(smem + B_BYTES);   // [WN][BM]
    if constexpr (ALIGNED) {
        // Stage B[m0 .., n0 ..] (BM x BN) in LDS with one coalesced DMA pass;
        // rows past d_out and columns past r read zeros.
        const int64_t rb = a.r * (int64_t)sizeof(E);
        const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<const char*>(a.B) + m0 * rb);
        int64_t bytes = (a.d_out - m0) * rb;
        if (bytes > 0x7ffffff0) bytes = 0x7ffffff0;
        i32x4_t rs;
        rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
        rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
        rs[2] = __builtin_amdgcn_readfirstlane((int)bytes);
        rs[3] = 0x00020000;
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        const int colb0 = (int)(n0 * (int64_t)sizeof(E));
        constexpr int NINS = (TL::BM * B_SLOTS + 63) / 64;
#pragma unroll
        for (int k = 0; k < (NINS + TL::NW - 1) / TL::NW; ++k) {
            const int ins = wave_u + k * TL::NW;
            if (NINS % TL::NW == 0 || ins < NINS) {
                const int slot = ins * 64 + lane;
                const int row = slot / B_SLOTS, ch = slot % B_SLOTS;
                const int colb = colb0 + ch * 16;
                const bool ok = ch < B_SLOTS - 1 && row < TL::BM && colb < (int)rb;
                const int voff = ok ? row * (int)rb + colb : kOutOfRange;
                raw_buffer_load_lds(rs, (lds_void_t*)(smem + ins * 1024), 16, voff, 0, 0, 0);
            }
        }
        if constexpr (GIP::WIDE) {
            // each wave stores its blocks of Gs_c = (s/2) G_c as bf16 [RP][RP]
            // and their mirrors; the blocks cover all of it (RP = BN)
            char* gs = smem + B_BYTES + RED_BYTES;
#pragma unroll
            for (int jb = 0; jb < NT; ++jb) {
                const int b1 = wn * NT + jb;
#pragma unroll
                for (int b2 = 0; b2 < GIP::NBLK; ++b2) {
                    if (b2 < b1) continue;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = b1 * 16 + 4 * (lane >> 4) + j, k = b2 * 16 + (lane & 15);
                        const E v = Cvt<E>::from_f(a.half_s * gacc[jb * GIP::NBLK + b2][j]);
                        *reinterpret_cast<E*>(gs + i * GIP::PITCH + k * 2) = v;
                        if (b1 != b2) *reinterpret_cast<E*>(gs + k * GIP::PITCH + i * 2) = v;
                    }
                }
            }
        } else if constexpr (GIP::value) {
            // wave 0 stores Gs_c = (s/2) G_c as bf16 [RP][RP] (zero past BN)
            // from its accumulators (every wave holds the same G_c)
            char* gs = smem + B_BYTES + RED_BYTES;
            if (wave == 0) {
                for (int o = lane * 16; o < GIP::BYTES; o += 64 * 16)
                    *reinterpret_cast<u32x4_t*>(gs + o) = u32x4_t{0u, 0u, 0u, 0u};
                int q = 0;
#pragma unroll
                for (int b1 = 0; b1 < NT; ++b1)
#pragma unroll
                    for (int b2 = b1; b2 < NT; ++b2, ++q)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int i = b1 * 16 + 4 * (lane >> 4) + j, k = b2 * 16 + (lane & 15);
                            const E v = Cvt<E>::from_f(a.half_s * gacc[q][j]);
                            *reinterpret_cast<E*>(gs + i * GIP::PITCH + k * 2) = v;
                            if (b1 != b2) *reinterpret_cast<E*>(gs + k * GIP::PITCH + i * 2) = v;
                        }
            }
        }
        wait_vmcnt<0>();
        __syncthreads();
        if constexpr (GIP::value) {
            // U += B Gs_c: left fragments are this wave's rows of the staged B
            // (K = columns of r, zero at and past BN), right fragments the
            // rows of Gs_c of this wave's columns
            const char* gs = smem + B_BYTES + RED_BYTES;
            typedef Mma<E> M;
#pragma unroll
            for (int ks = 0; ks < GIP::RP / 32; ++ks) {
                const int kk = 32 * ks + 8 * (lane >> 4);
                typename M::frag_t gf[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    gf[nt] = *reinterpret_cast<const typename M::frag_t*>(
                        gs + ((wn * NT + nt) * 16 + (lane & 15)) * GIP::PITCH + kk * 2);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int row = wm * MT * 16 + mt * 16 + (lane & 15);
                    typename M::frag_t bf{};
                    if (kk < TL::BN) bf = *reinterpret_cast<const typename M::frag_t*>(smem + row * B_PITCH + kk * 2);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) M::mma(acc[mt][nt], bf, gf[nt]);
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wm * MT * 16 + mt * 16 + 4 * (lane >> 4) + j;
                const E* brow = reinterpret_cast<const E*>(smem + row * B_PITCH) + wn * NT * 16 + (lane & 15);
                float v = 0.0f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) v = fmaf(Cvt<E>::to_f(brow[nt * 16]), acc[mt][nt][j], v);
                v += __shfl_xor(v, 1);
                v += __shfl_xor(v, 2);
                v += __shfl_xor(v, 4);
                v += __shfl_xor(v, 8);
                if ((lane & 15) == 0) red[wn * TL::BM + row] = v;
            }
        }
    } else {
        const E* Bp = static_cast<const E*>(a.B);
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


// ------------------------------------------------------------- W0 pass, whole rows (low rank)
// bf16, 16-byte aligned operands, r <= 32.  A workgroup owns 16 whole rows
// of W0 and its eight waves split K eight ways (measured: 5-9% faster than
// four waves, by the loads it keeps in flight per CU): each walks its K range
// (U, base and Gram blocks of that range, whose Gram term is a sum over K
// ranges like any other K split) through its own LDS-DMA ring; then it adds
// (s/2) B G_w to its U accumulators and takes the row dots with B.  The
// workgroup adds the waves' base and cross partials in wave order in LDS and
// writes wnorm and g itself: no partials leave the workgroup and no assembly
// kernel runs.
struct W0RowsArgs {
    Contraction c;        // left0 = W0, right0 = A; no second phase
    const void* B;        // [d_out, r]
    const float* m;       // [d_out] or null
    int64_t d_out, r;
    float half_s, two_s, eps;
    float* wnorm;
    float* g;
};

constexpr int kRowsWaves = 8;
constexpr int kRowsPerWg = 16;


// One round of workgroups (rows_form): each holds a CU's LDS for its rings.
template <int NT>
__global__ __launch_bounds__(kRowsWaves * 64) void w0_rows_narrow(W0RowsArgs a) {
    typedef bf16_t E;
    typedef Mma<E> M;
    typedef GramInPass<E, 1, NT, true> GIP;
    static_assert(GIP::value, "the whole-row form forms the Gram term in the pass");
    constexpr int BN = NT * 16;
    constexpr int B_SLOTS = BN * 2 / 16 + 1;                      // 16-byte slots per staged B row (+1 zero pad)
    constexpr int B_PITCH = B_SLOTS * 16;
    constexpr int B_NINS = (kRowsPerWg * B_SLOTS + 63) / 64;      // DMA instructions staging B
    constexpr int GS_OFF = B_NINS * 1024;                         // the DMA fills whole 1 KiB blocks
    constexpr int RED_OFF = GS_OFF + kRowsWaves * GIP::BYTES;
    constexpr int EPI = RED_OFF + 2 * kRowsWaves * kRowsPerWg * 4;
    // the K walk's ring follows the staged B and is reused by the Gs tiles
    // and the reduction once the walk is done
    constexpr int RING_OFF = GS_OFF;
    typedef NarrowRing<1, NT, kRowsWaves, NT == 1 ? 4 : 3> RR;
    constexpr int RING_END = RING_OFF + RR::BYTES;
    constexpr int LDS = RING_END > EPI ? RING_END : EPI;
    __shared__ __attribute__((aligned(1024))) char smem[LDS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t m0 = (int64_t)blockIdx.x * kRowsPerWg;
    const int nkt = a.c.nkt0;
    const int kt_begin = (int)((int64_t)wave * nkt / kRowsWaves);
    const int kt_end = (int)((int64_t)(wave + 1) * nkt / kRowsWaves);

    f32x4_t acc[1][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[0][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t gacc[GIP::NG];
#pragma unroll
    for (int q = 0; q < GIP::NG; ++q) gacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float bsum = 0.0f;
    // m of this workgroup's rows, requested before the K walk so that its
    // latency hides under it (loads retire in issue order, so the walk's
    // first wait covers it)
    float m_row = 0.0f;
    if (threadIdx.x < kRowsPerWg && a.m && m0 + threadIdx.x < a.d_out) m_row = a.m[m0 + threadIdx.x];
    // B rows [m0, m0 + 16), columns [0, BN) (zeros past r and past d_out),
    // staged by wave 0 ahead of the K walk, which uses no LDS
    if (wave == 0) {
        const int64_t rb = a.r * 2;
        const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<const char*>(a.B) + m0 * rb);
        int64_t bytes = (a.d_out - m0) * rb;
        if (bytes > 0x7ffffff0) bytes = 0x7ffffff0;
        i32x4_t rs;
        rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
        rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
        rs[2] = __builtin_amdgcn_readfirstlane((int)bytes);
        rs[3] = 0x00020000;
#pragma unroll
        for (int ins = 0; ins < B_NINS; ++ins) {
            const int slot = ins * 64 + lane;
            const int row = slot / B_SLOTS, ch = slot % B_SLOTS;
            const int colb = ch * 16;
            const bool ok = ch < B_SLOTS - 1 && row < kRowsPerWg && colb < (int)rb;
            const int voff = ok ? row * (int)rb + colb : kOutOfRange;
            raw_buffer_load_lds(rs, (lds_void_t*)(smem + ins * 1024), 16, voff, 0, 0, 0);
        }
    }
    {
        float bs[1];
        mainloop_narrow_dma<1, NT, GIP::NG, (NT == 1 ? 4 : 3)>(a.c, m0, 0, kt_begin, kt_end, 0, true,
                                                                smem + RING_OFF, acc, gacc, bs);
        bsum = bs[0];
        __syncthreads();   // every wave is done with the ring
    }

    // this wave's Gs_w = (s/2) G_w as bf16 [RP][RP], zero past BN
    {
        char* gs = smem + GS_OFF + wave * GIP::BYTES;
        for (int o = lane * 16; o < GIP::BYTES; o += 64 * 16)
            *reinterpret_cast<u32x4_t*>(gs + o) = u32x4_t{0u, 0u, 0u, 0u};
        int q = 0;
#pragma unroll
        for (int b1 = 0; b1 < NT; ++b1)
#pragma unroll
            for (int b2 = b1; b2 < NT; ++b2, ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = b1 * 16 + 4 * (lane >> 4) + j, k = b2 * 16 + (lane & 15);
                    const E v = Cvt<E>::from_f(a.half_s * gacc[q][j]);
                    *reinterpret_cast<E*>(gs + i * GIP::PITCH + k * 2) = v;
                    if (b1 != b2) *reinterpret_cast<E*>(gs + k * GIP::PITCH + i * 2) = v;
                }
    }
    wait_vmcnt<0>();
    __syncthreads();
    // U_w += B Gs_w, then the row dots with B
    {
        const char* gs = smem + GS_OFF + wave * GIP::BYTES;
        const int kk = 8 * (lane >> 4);
        typename M::frag_t bf{};
        if (kk < BN) bf = *reinterpret_cast<const typename M::frag_t*>(smem + (lane & 15) * B_PITCH + kk * 2);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const typename M::frag_t gf =
                *reinterpret_cast<const typename M::frag_t*>(gs + (nt * 16 + (lane & 15)) * GIP::PITCH + kk * 2);
            M::mma(acc[0][nt], bf, gf);
        }
    }
    float* red = reinterpret_cast<float*>(smem + RED_OFF);   // [2][waves][16]: base, cross
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 4 * (lane >> 4) + j;
        const E* brow = reinterpret_cast<const E*>(smem + row * B_PITCH) + (lane & 15);
        float v = 0.0f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) v = fmaf(Cvt<E>::to_f(brow[nt * 16]), acc[0][nt][j], v);
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        if ((lane & 15) == 0) red[(kRowsWaves + wave) * kRowsPerWg + row] = v;
    }
    if (lane < kRowsPerWg) red[wave * kRowsPerWg + lane] = bsum;
    __syncthreads();
    if (threadIdx.x < kRowsPerWg) {
        const int row = threadIdx.x;
        const int64_t i = m0 + row;
        if (i < a.d_out) {
            float base = red[row], cd = red[kRowsWaves * kRowsPerWg + row];
#pragma unroll
            for (int w = 1; w < kRowsWaves; ++w) {
                base += red[w * kRowsPerWg + row];
                cd += red[(kRowsWaves + w) * kRowsPerWg + row];
            }
            const float n2 = fmaxf(fmaf(a.two_s, cd, base), 0.0f);
            const float wn = sqrtf(n2);
            a.wnorm[i] = wn;
            if (a.m) a.g[i] = m_row / fmaxf(wn, a.eps);
        }
    }
}

// ------------------------------------------------------------- W0 pass, 256 x 384 tiles
// Large-tile form of the W0 pass for bf16 operands, used when r > 128.  A
// workgroup owns 256 rows of W0 and 384 columns of r: every A tile that
// crosses L2 feeds twice as many MFMAs as with 128-row tiles, which halves
// the L2 -> CU traffic of A, the larger of the two streams per k-tile.
// Eight waves in a 2 x 4 grid each accumulate a 128 x 96 block with 32x32x16
// MFMAs (4 x 3 blocks of 32 x 32, 192 accumulators per lane); one 16-deep
// step of K needs only 7 operand registers per lane, so two waves fit on
// every SIMD and cover each other's LDS and memory waits.  Tiles are 64
// elements of K (whole 128-byte rows, so every DMA request is a full line):
// W0 | B and A | Gs share a two-stage ring that fills the CU's 160 KB of LDS.

struct Big {
    static constexpr int WG_PER_CU = 1;                 // workgroups resident on one CU
    static constexpr int WM = WG_PER_CU == 2 ? 1 : 2, WN = 4, NW = WM * WN, NTH = NW * 64;
    static constexpr int MT = 4, NT = 3;   // 32 x 32 blocks per wave
    static constexpr int WROWS = MT * 32;  // rows of one wave row
    static constexpr int BM = WM * WROWS, BN = WN * NT * 32, BK = 64;
    static constexpr int KS = BK / 16;     // 32 x 32 x 16 MFMA steps per k-tile
    static constexpr int STAGES = 2;       // ring stages, each a k-tile of both operands
    static constexpr int ER = WM * 32;     // epilogue rows per round
    static constexpr int ROWB = BK * 2;    // bytes of K per tile row: one whole 128-byte line
    static constexpr int LBYTES = BM * ROWB, RBYTES = BN * ROWB;
    static constexpr int STAGE = LBYTES + RBYTES;
    static constexpr int RING = STAGES * STAGE;
    static constexpr int LPW = BM / 8 / NW, RPW = BN / 8 / NW;   // DMA instructions (8 rows each) per wave per tile
    // epilogue: two staging buffers of 64 B rows (rows padded by 16 bytes)
    // and the per-row partials of all four rounds
    static constexpr int EB_SLOTS = BN * 2 / 16 + 1;
    static constexpr int EB_PITCH = EB_SLOTS * 16;
    // a staging buffer is filled by whole 1 KiB DMA instructions
    static constexpr int EB_BYTES = (ER * EB_PITCH + 1023) / 1024 * 1024;
    static constexpr int EPI_BYTES = 2 * EB_BYTES + MT * WN * ER * 4;
    static constexpr int LDS_BYTES = RING > EPI_BYTES ? RING : EPI_BYTES;
    static_assert(BM / 8 % NW == 0 && BN / 8 % NW == 0, "DMA groups split evenly across waves");
    static_assert(NW % 2 == 0, "a wave's DMA groups all have the parity of the wave");
    static_assert(LBYTES % 1024 == 0 && RBYTES % 1024 == 0, "ring stages hold whole 1 KiB DMA instructions");
    static_assert(MT == WN, "each wave sums the base term of one 32-row block");
    static_assert(LPW + RPW < 64, "vmcnt range");
};



// Enqueue rows [0, ROWS) of a 128-byte K slab into LDS at dst.  `d` is the
// phase's operand (scalar fields), k0b the slab's byte offset along K.  Lane
// l moves slot l % 8 of row l / 8 of each 8-row group: lane_off =
// (l / 8) * ld_bytes + chunk_b, where chunk_b is the byte offset of the
// logical chunk that slot holds (slot ^ swz(row); the groups a wave issues
// all have the wave's parity, so one chunk serves them all); a lane_off of
// kOutOfRange turns the whole load into zeros.  Chunks past the operand's K
// extent read zeros.  Row and K offsets fit 31 bits: a workgroup's rows of
// any operand span less than 2^30 bytes.  AUX is the loads' cache policy:
// the left operand (W0, then B) is read once and goes non-temporal, which
// measured 2-4% faster at 28672 x 8192, 36864 x 8192, 28672 x 16384 and
// 27648 x 5120, r = 384, and no slower at 8192^2 and 4096^2.
template <int ROWS, int AUX>
__device__ __forceinline__ void dma128_tile(const Dma64& d, int lane_off, int chunk_b, int k0b, char* dst,
                                            int wave) {
    constexpr int PER = ROWS / 8 / Big::NW;
    const int ldb = d.ld_bytes, bytes = d.bytes, kmax = d.kmax_bytes;
    const uint64_t base = ((uint64_t)d.base_hi << 32) | d.base_lo;
    const bool full = k0b + Big::ROWB <= kmax;
    const int voff = full ? lane_off : (chunk_b < kmax - k0b ? lane_off : kOutOfRange);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int grp = wave + q * Big::NW;
        const int off = grp * 8 * ldb + k0b;
        const int left = bytes > off ? bytes - off : 0;
        const uint64_t addr = base + (uint32_t)off;
        i32x4_t rs;
        rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
        rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
        rs[2] = __builtin_amdgcn_readfirstlane(left);
        rs[3] = 0x00020000;
        raw_buffer_load_lds(rs, (lds_void_t*)(dst + grp * 1024), 16, voff, 0, 0, AUX);
    }
}

// One segment of the large-tile pass: rows of m-tile mtile, columns of
// n-tile ntile, k-tiles [kt_begin, kt_end); its partials go to slot kc.
__device__ __forceinline__ void w0_pass_big_seg(const W0PassArgs& a, const int id, const int mtile, const int ntile,
                                                const int kc, const int kt_begin, const int kt_end, char* smem) {
    typedef Big G;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / G::WN, wn = wave % G::WN;
    const int64_t m0 = (int64_t)mtile * G::BM, n0 = (int64_t)ntile * G::BN;
    const Contraction& c = a.c;
    const int n = kt_end - kt_begin;
    float* base_dst = ntile == 0 ? a.part_base + (int64_t)kc * a.d_out : nullptr;
    const int rot = n > 0 ? (int)(((unsigned)id * 7u + ((unsigned)id >> 3) * 3u) % (unsigned)n) : 0;

    f32x16_t acc[G::MT][G::NT];
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mt][nt][e] = 0.0f;
    float bs = 0.0f;

    if (n > 0) {
        const Dma64 L0 = make_dma64(c.left0, m0);
        const Dma64 L1 = make_dma64(c.left1, m0);
        const Dma64 R0 = make_dma64(c.right0, n0);
        const Dma64 R1 = make_dma64(c.right1, n0);
        // per-lane DMA offsets; the two operands of a phase share a row pitch
        // (W0 and A: d_in; B and Gs: r, a multiple of 8 on this path)
        const int dchunk = ((lane & 7) ^ (lane >> 3) ^ (wave & 1)) * 16;
        const int doff0 = (lane >> 3) * L0.ld_bytes + dchunk;
        const int doff1 = (lane >> 3) * L1.ld_bytes + dchunk;
        // fragment byte offsets inside a tile: row (l % 32) of a 32-row block,
        // logical chunk 2 ks + l / 32 for MFMA step ks, i.e. fo0 ^ (ks << 5)
        const int fo0 = (lane & 31) * G::ROWB + (((lane >> 5) ^ swz(lane & 31)) << 4);
        const int lrow0 = wm * G::WROWS * G::ROWB, rrow0 = wn * 96 * G::ROWB;
        const float base_on = base_dst != nullptr ? 1.0f : 0.0f;

        // k-tile visited at step i (the walk starts at a rotated tile)
        auto tile = [&](int i) __attribute__((always_inline)) {
            int t = i + rot;
            if (t >= n) t -= n;
            return kt_begin + t;
        };
        // Loads of step i into stage i % 2; steps past the last tile still
        // issue (reading zeros into a stage no one reads), so the loop carries
        // no branches.
        auto issue_op = [&](int i, auto rows, int soff, const Dma64& P0, const Dma64& P1)
            __attribute__((always_inline)) {
            const bool valid = i < n;
            const int kt = tile(valid ? i : 0);
            const bool ph0 = kt < c.nkt0;
            Dma64 d;
            d.base_lo = ph0 ? P0.base_lo : P1.base_lo;
            d.base_hi = ph0 ? P0.base_hi : P1.base_hi;
            d.bytes = ph0 ? P0.bytes : P1.bytes;
            d.ld_bytes = ph0 ? P0.ld_bytes : P1.ld_bytes;
            d.kmax_bytes = ph0 ? P0.kmax_bytes : P1.kmax_bytes;
            const int lo = valid ? (ph0 ? doff0 : doff1) : kOutOfRange;
            const int k0b = (ph0 ? kt : kt - c.nkt0) * G::ROWB;
            dma128_tile<decltype(rows)::value, decltype(rows)::value == G::BM ? kCachePolicyNT : 0>(
                d, lo, dchunk, k0b, smem + (i % G::STAGES) * G::STAGE + soff, wave);
        };
        auto issue = [&](int i) __attribute__((always_inline)) {
            issue_op(i, IntC<G::BM>{}, 0, L0, L1);
            issue_op(i, IntC<G::BN>{}, G::LBYTES, R0, R1);
        };
        auto read = [&](int i, int ks, bf16x8_t (&av)[G::MT], bf16x8_t (&bv)[G::NT]) __attribute__((always_inline)) {
            const int fo = fo0 ^ (ks << 5);
            const char* Lt = smem + (i % G::STAGES) * G::STAGE + lrow0 + fo;
            const char* Rt = smem + (i % G::STAGES) * G::STAGE + G::LBYTES + rrow0 + fo;
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt) av[mt] = *reinterpret_cast<const bf16x8_t*>(Lt + mt * 32 * G::ROWB);
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt) bv[nt] = *reinterpret_cast<const bf16x8_t*>(Rt + nt * 32 * G::ROWB);
        };
        // MFMAs over blocks (mt, nt) with lo <= mt * NT + nt < hi.  The right
        // fragments go in the A slot and the left ones in the B slot, so each
        // accumulator block holds U^T: lane l carries row l % 32 of the left
        // block and register e column 8 (e / 4) + 4 (l / 32) + e % 4 of the
        // right block (runs of 4 consecutive columns, read as one 8-byte load
        // of B in the epilogue).
        auto mma = [&](const bf16x8_t (&av)[G::MT], const bf16x8_t (&bv)[G::NT], int lo, int hi)
            __attribute__((always_inline)) {
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt) {
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt) {
                    const int k = mt * G::NT + nt;
                    if (k < lo || k >= hi) continue;
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[nt], av[mt], acc[mt][nt], 0, 0, 0);
                }
            }
        };
        // ||W0_i||^2 from the left fragments: wave wn sums block wn of its
        // rows (a compile-time copy of the loop per wave column); on = 0 for
        // k-tiles of the B | Gs phase or workgroups that own no base rows
        auto base_sum = [&](auto wnc, const bf16x8_t (&av)[G::MT], float on) __attribute__((always_inline)) {
            bs = fmaf(on, Mma<bf16_t>::frag_sumsq(av[decltype(wnc)::value]), bs);
        };
        auto base_on_at = [&](int i) __attribute__((always_inline)) {
            return tile(i) < c.nkt0 ? base_on : 0.0f;
        };

        // Software pipeline over k-tiles, two stages: tile j + 1 loads while
        // tile j is computed.  Tile j: its four MFMA steps, the fragments of
        // each next step read while the previous step's MFMAs run (two
        // register sets), all but the last HOLD MFMAs of step 3.  Then wait
        // for tile j + 1 (this wave's loads; its fragment reads of tile j are
        // complete), barrier (every wave's loads of tile j + 1 landed, every
        // wave is done with tile j's stage), enqueue tile j + 2 into that
        // stage, read tile j + 1's step-0 fragments, and only then issue the
        // held-back MFMAs, which keep the matrix pipe busy across the barrier
        // and the LDS latency.  (Enqueueing tile j + 2 earlier, behind a
        // second barrier once step 3's fragments are read, measured 2-4%
        // slower.)
        constexpr int HOLD = 2;
        constexpr int ALL = G::MT * G::NT;
        // Order of one step's MFMAs and the next step's fragment reads: one
        // MFMA, then the MT + NT fragment reads, then the other MFMAs, so the
        // reads' LDS latency runs under the matrix pipe instead of after it.
        // Measured 3% faster at 28672 x 8192 and 27648 x 5120, r = 384, and
        // no slower at 8192^2 and 4096^2.
        auto interleave = []() __attribute__((always_inline)) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, G::MT + G::NT, 0);  // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, ALL - 1, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        auto main_loop = [&](auto wnc) __attribute__((always_inline)) {
            bf16x8_t a0[G::MT], b0[G::NT], a1[G::MT], b1[G::NT];
            issue(0);
            issue(1);
            wait_vmcnt<G::LPW + G::RPW>();   // tile 0 landed; tile 1 may be in flight
            __builtin_amdgcn_s_barrier();
            read(0, 0, a0, b0);
            for (int j = 0; j < n - 1; ++j) {
                const float on = base_on_at(j);
                mma(a0, b0, 0, ALL);
                read(j, 1, a1, b1);
                base_sum(wnc, a0, on);
                interleave();
                mma(a1, b1, 0, ALL);
                read(j, 2, a0, b0);
                base_sum(wnc, a1, on);
                interleave();
                mma(a0, b0, 0, ALL);
                read(j, 3, a1, b1);
                base_sum(wnc, a0, on);
                interleave();
                mma(a1, b1, 0, ALL - HOLD);
                base_sum(wnc, a1, on);
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<0>();
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                issue(j + 2);
                read(j + 1, 0, a0, b0);
                __builtin_amdgcn_sched_barrier(0);
                mma(a1, b1, ALL - HOLD, ALL);
            }
            {
                const float on = base_on_at(n - 1);
                mma(a0, b0, 0, ALL);
                base_sum(wnc, a0, on);
                __builtin_amdgcn_sched_barrier(0);
                read(n - 1, 1, a1, b1);
                mma(a1, b1, 0, ALL);
                base_sum(wnc, a1, on);
                __builtin_amdgcn_sched_barrier(0);
                read(n - 1, 2, a0, b0);
                mma(a0, b0, 0, ALL);
                base_sum(wnc, a0, on);
                __builtin_amdgcn_sched_barrier(0);
                read(n - 1, 3, a1, b1);
                mma(a1, b1, 0, ALL);
                base_sum(wnc, a1, on);
            }
            wait_vmcnt<0>();   // trailing zero loads land before LDS is reused
        };
        switch (wn) {
            case 0: main_loop(IntC<0>{}); break;
            case 1: main_loop(IntC<1>{}); break;
            case 2: main_loop(IntC<2>{}); break;
            default: main_loop(IntC<3>{}); break;
        }
    }
    __syncthreads();   // ring free for the epilogue

    // base partial: lanes l and l + 32 hold the two K halves of row l % 32 of
    // block wn of this wave's 128 rows
    const float base_part = bs + __shfl_xor(bs, 32);   // row l % 32 of block wn, lanes < 32

    // cross partial: sum_n B[m][n] U[m][n] over this workgroup's columns.
    // acc[mt][nt][e] is U at row mt*32 + l%32 of the wave's 128 rows and
    // column nt*32 + 8 (e/4) + 4 (l/32) + e%4 of its 96.  Round mt handles row
    // block mt of both row halves (64 rows): its B rows are staged in LDS
    // (double buffered, the next round's DMA overlaps this round's dots);
    // every lane dots its row with 4-column runs of B (one 8-byte read each),
    // adds the other half-wave's columns of the same row, and the four column
    // waves' partials are added in order.
    {
        const int64_t rb = a.r * 2;
        const int colb0 = (int)(n0 * 2);
        const uint64_t baddr = reinterpret_cast<uint64_t>(static_cast<const char*>(a.B) + m0 * rb);
        int64_t bbytes = (a.d_out - m0) * rb;
        if (bbytes < 0) bbytes = 0;
        if (bbytes > 0x7ffffff0) bbytes = 0x7ffffff0;
        i32x4_t brs;
        brs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)baddr);
        brs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(baddr >> 32));
        brs[2] = __builtin_amdgcn_readfirstlane((int)bbytes);
        brs[3] = 0x00020000;
        constexpr int ER = G::ER;                             // rows per round
        constexpr int EBUF = G::EB_BYTES;                     // one staging buffer
        float* red = reinterpret_cast<float*>(smem + 2 * EBUF);   // [MT][WN][ER]
        // staged row r of round mt is tile row (r / 32) * WROWS + mt * 32 + r % 32
        auto stage_b = [&](int mt, char* buf) __attribute__((always_inline)) {
            constexpr int NINS = (ER * G::EB_SLOTS + 63) / 64;
#pragma unroll
            for (int k = 0; k < (NINS + G::NW - 1) / G::NW; ++k) {
                const int ins = wave + k * G::NW;
                if (ins < NINS) {
                    const int slot = ins * 64 + lane;
                    const int row = slot / G::EB_SLOTS, ch = slot % G::EB_SLOTS;
                    const int trow = (row >> 5) * G::WROWS + mt * 32 + (row & 31);
                    const int colb = colb0 + ch * 16;
                    const bool ok = ch < G::EB_SLOTS - 1 && row < ER && colb < (int)rb;
                    const int voff = ok ? trow * (int)rb + colb : kOutOfRange;
                    raw_buffer_load_lds(brs, (lds_void_t*)(buf + ins * 1024), 16, voff, 0, 0, 0);
                }
            }
        };
        stage_b(0, smem);
        const int srow = wm * 32 + (lane & 31);               // this lane's staged row
        const int colh = 4 * (lane >> 5);                      // its column offset in a run of 8
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
            wait_vmcnt<0>();
            __syncthreads();   // round mt's B landed; round mt - 1's readers are done
            if (mt + 1 < G::MT) stage_b(mt + 1, smem + ((mt + 1) & 1) * EBUF);
            const bf16_t* brow =
                reinterpret_cast<const bf16_t*>(smem + (mt & 1) * EBUF + srow * G::EB_PITCH) + wn * 96 + colh;
            float x = 0.0f;
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    typedef bf16_t bf16x4_t __attribute__((ext_vector_type(4)));
                    const bf16x4_t bq = *reinterpret_cast<const bf16x4_t*>(brow + nt * 32 + 8 * q);
#pragma unroll
                    for (int c = 0; c < 4; ++c) x = fmaf(static_cast<float>(bq[c]), acc[mt][nt][4 * q + c], x);
                }
            }
            x += __shfl_xor(x, 32);   // the other half-wave holds the row's other columns
            if (lane < 32) red[mt * G::WN * ER + wn * ER + srow] = x;
        }
        __syncthreads();
    }

    // Publish this workgroup's partials: the base term of rows
    // wm*WROWS + wn*32 + l (l < 32), and for every row the sum of the four
    // column waves' dots, in wave order.
    {
        const float* red = reinterpret_cast<const float*>(smem + 2 * G::EB_BYTES);
        if (base_dst) {
            const int64_t mrow = m0 + wm * G::WROWS + wn * 32 + lane;
            if (lane < 32 && mrow < a.d_out) base_dst[mrow] = base_part;
        }
        for (int t = threadIdx.x; t < G::BM; t += G::NTH) {
            const int mt = t / G::ER, r = t % G::ER;
            const int64_t mrow = m0 + (r >> 5) * G::WROWS + mt * 32 + (r & 31);
            if (mrow < a.d_out) {
                const float* rd = red + mt * G::WN * G::ER;
                float v = rd[r];
#pragma unroll
                for (int w = 1; w < G::WN; ++w) v += rd[w * G::ER + r];
                a.part_cross[((int64_t)ntile * a.ksplit + kc) * a.d_out + mrow] = v;
            }
        }
    }
}

// Uniform K split: one segment per workgroup, K-chunks mapped to XCDs.  This
// form keeps the segment body outside any loop: wrapped in the balanced
// form's segment loop, the body's register allocation spills (256 VGPRs and
// 60 bytes of scratch per lane, and 9% more time at 8192^2), so that loop
// lives in its own kernel.
__device__ __forceinline__ void w0_pass_big_body(const W0PassArgs& a, const int id, char* smem) {
    const int nkt = a.c.nkt0 + a.c.nkt1;
    const int Q = a.n_ntiles * a.ksplit;
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
    const int kc = q % a.ksplit;
    w0_pass_big_seg(a, id, mtile, q / a.ksplit, kc, (int)((int64_t)kc * nkt / a.ksplit),
                    (int)((int64_t)(kc + 1) * nkt / a.ksplit), smem);
}

// Balanced K split (Balance): the workgroup's segments in walk order.
__device__ __forceinline__ void w0_pass_big_body_balanced(const W0PassArgs& a, const int id, char* smem) {
    bool first = true;
    balance_segments(a.bal, id, [&](const BalanceSeg& s) {
        if (!first) __syncthreads();   // the previous segment's epilogue is done with LDS
        first = false;
        w0_pass_big_seg(a, id, s.mt, 0, s.slot, s.kt_begin, s.kt_end, smem);
    });
}

// ------------------------------------------------------------- Gram
constexpr int kGramTile = 64;   // WM = WN = 2, MT = NT = 2

struct GramArgs {
    Contraction c;     // left0 = right0 = A
    int ntiles, nsplit, nupper;
    int64_t rnp;       // ntiles * 64
    float* part;       // [nsplit][rnp][rnp]; only tiles with ti <= tj are written
};

template <typename E, bool ALIGNED>
__global__ __launch_bounds__(256) void gram_partial(GramArgs a) {
    typedef Tile<E, 2, 2, 2, 2> TL;
    __shared__ __attribute__((aligned(1024))) char smem[ALIGNED ? TL::DMA_BYTES : TL::STAGED_BYTES];
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
    mainloop<E, 2, 2, 2, 2, ALIGNED>(a.c, (int64_t)ti * kGramTile, (int64_t)tj * kGramTile, kt_begin, kt_end,
                                     0, nullptr, 0, acc, smem);
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

// Gram partials for bf16 operands with 16-byte aligned rows.  Split s of the
// K range runs on XCD s % 8 (workgroup ids are dealt to XCDs round-robin), so
// each XCD streams only its own K-slices of A and the whole of A crosses HBM
// once.  Each workgroup walks its slice through an LDS ring of NS stages
// (left and right 64-row tiles, 16 KB a stage), NS - 1 tiles ahead.  A single
// call runs one round of workgroups and uses 8 stages; a group's Gram runs
// several members' workgroups and uses 4, so that two workgroups share a CU.
// The ring depth does not change the order of the K walk, so both give the
// same partials bit for bit.
template <int NS>
constexpr int gram_split_lds() {
    return NS * (Tile<bf16_t, 2, 2, 2, 2>::LBYTES + Tile<bf16_t, 2, 2, 2, 2>::RBYTES);
}
constexpr int kGramStages = 8, kGramStagesGroup = 4;

template <int NS>
__device__ __forceinline__ void gram_split_bf16_body(const GramArgs& a, const int id, char* smem) {
    typedef Tile<bf16_t, 2, 2, 2, 2> TL;
    typedef Mma<bf16_t> M;
    constexpr int STAGE = TL::LBYTES + TL::RBYTES;   // 8 KB + 8 KB
    constexpr int LPW = 2 * (TL::BM / 8 / TL::NW);   // DMA instructions per wave per tile (left + right)
    static_assert(LPW * (NS - 2) < 64, "vmcnt range");
    static_assert(NS * STAGE == gram_split_lds<NS>(), "LDS size");
    const int xcd = id % kNumXCD, slot = id / kNumXCD;
    const int split = xcd + kNumXCD * (slot / a.nupper);
    if (split >= a.nsplit) return;
    int u = slot % a.nupper, ti = 0;
    while (u >= a.ntiles - ti) {
        u -= a.ntiles - ti;
        ++ti;
    }
    const int tj = ti + u;
    const int nkt = a.c.nkt0;
    const int kt_begin = (int)((int64_t)split * nkt / a.nsplit);
    const int n = (int)((int64_t)(split + 1) * nkt / a.nsplit) - kt_begin;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / 2, wn = wave % 2;
    const int q = lane >> 4;
    const DmaSrc L = make_dma_src<bf16_t>(a.c.left0, (int64_t)ti * kGramTile, lane);
    const DmaSrc R = make_dma_src<bf16_t>(a.c.left0, (int64_t)tj * kGramTile, lane);
    constexpr int TKB = 128;
    // the K walk starts at a tile that differs between the workgroups of a
    // split, so that the six tiles sharing a row block do not request the
    // same lines at the same time
    const int rot = n > 0 ? (int)((unsigned)(slot * 5) % (unsigned)n) : 0;
    auto issue = [&](int i) __attribute__((always_inline)) {
        char* st = smem + (i % NS) * STAGE;
        int t = i + rot;
        if (t >= n) t -= n;
        const int k0b = (kt_begin + t) * TKB;
        dma_tile<TL::BM, 0, TL::NW>(L, k0b, st, wave, TKB);
        dma_tile<TL::BN, 0, TL::NW>(R, k0b, st + TL::LBYTES, wave, TKB);
    };
    int lrow[2], lsw[2], rrow[2], rsw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        lrow[t] = wm * 32 + t * 16 + (lane & 15);
        lsw[t] = swz(lrow[t]);
        rrow[t] = wn * 32 + t * 16 + (lane & 15);
        rsw[t] = swz(rrow[t]);
    }
    f32x4_t acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Tiles move in groups of GT = NS / 2: group g + 1 loads while group g
    // is computed, with two barriers per group.
    constexpr int GT = NS / 2;
    const int ngroups = (n + GT - 1) / GT;
    auto issue_group = [&](int grp) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < GT; ++t)
            if (grp * GT + t < n) issue(grp * GT + t);
    };
    issue_group(0);
    issue_group(1);
    for (int grp = 0; grp < ngroups; ++grp) {
        // group grp landed (only group grp + 1, if full, may be in flight)
        if ((grp + 2) * GT <= n)
            wait_vmcnt<LPW * GT>();
        else
            wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int t = 0; t < GT; ++t) {
            const int jj = grp * GT + t;
            if (jj >= n) break;
            const char* Lt = smem + (jj % NS) * STAGE;
            const char* Rt = Lt + TL::LBYTES;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                M::frag_t av[2], bv[2];
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) {
                    av[q2] = M::load_frag_swz(Lt + lrow[q2] * 128, ks, q, lsw[q2]);
                    bv[q2] = M::load_frag_swz(Rt + rrow[q2] * 128, ks, q, rsw[q2]);
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) M::mma(acc[mt][nt], av[mt], bv[nt]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's reads of group grp are done
        __builtin_amdgcn_s_barrier();         // every wave's are: the group's stages are free
        issue_group(grp + 2);
    }

    // Write the partial tile as coalesced 16-byte row segments staged through
    // LDS (the ring is free).
    float* tl = reinterpret_cast<float*>(smem);   // [64][TP]
    constexpr int TP = kGramTile + 4;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int ii = wm * 32 + mt * 16 + 4 * (lane >> 4) + jj;
                const int kk = wn * 32 + nt * 16 + (lane & 15);
                tl[ii * TP + kk] = acc[mt][nt][jj];
            }
    __syncthreads();
    float* out = a.part + (int64_t)split * a.rnp * a.rnp;
    const int tid = threadIdx.x;
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
        const int e = rep * 256 + tid;        // 1024 segments of 4 floats
        const int row = e >> 4, c4 = (e & 15) * 4;
        f32x4_t v;
        v[0] = tl[row * TP + c4];
        v[1] = tl[row * TP + c4 + 1];
        v[2] = tl[row * TP + c4 + 2];
        v[3] = tl[row * TP + c4 + 3];
        *reinterpret_cast<f32x4_t*>(out + ((int64_t)ti * kGramTile + row) * a.rnp + (int64_t)tj * kGramTile + c4) = v;
    }
}

// Gs[i][j] = (s/2) * sum_split G[i][j] for i < r, j < r; zero for r <= j < ldg.
// The partials hold only the upper 64 x 64 tiles (ti <= tj); G is symmetric,
// so an element of a lower tile is read at its mirror position.  A workgroup
// owns kGfRows rows of one 64 x 64 tile of Gs.  A lower tile reads 64 rows of
// kGfRows columns of its mirror (64-byte pieces) and transposes them through
// LDS, so reads and writes are both coalesced (a pitch of 66 floats keeps the
// transposing writes of 32 lanes on distinct banks).  Each element sums its
// split partials in split order.
constexpr int kGfRows = 16;
constexpr int kGfPerTile = kGramTile / kGfRows;
static_assert(kGfRows * kGramTile == 4 * 256, "four elements per thread");

template <typename E>
__device__ __forceinline__ void gram_finalize_body(const float* __restrict__ part, int nsplit, int64_t rnp,
                                                   int64_t r, int64_t ldg, float half_s, E* __restrict__ gs,
                                                   const int id, float (*tr)[kGramTile + 2]) {
    const int ntiles = (int)(rnp / kGramTile);
    const int tile = id / kGfPerTile, x0 = (id % kGfPerTile) * kGfRows;
    const int ti = tile / ntiles, tj = tile % ntiles;
    const bool mirror = ti > tj;   // uniform over the workgroup
    const int t = threadIdx.x;
    const int64_t stride = rnp * rnp;
    int64_t src[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = e * 256 + t;
        if (!mirror)   // row idx / 64 of the block, column idx % 64
            src[e] = ((int64_t)ti * kGramTile + x0 + idx / kGramTile) * rnp + (int64_t)tj * kGramTile + idx % kGramTile;
        else           // mirror row idx / 16, column x0 + idx % 16
            src[e] = ((int64_t)tj * kGramTile + idx / kGfRows) * rnp + (int64_t)ti * kGramTile + x0 + idx % kGfRows;
    }
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int sp = 0; sp < nsplit; sp += 8) {
        float x[4][8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e][q] = sp + q < nsplit ? part[(int64_t)(sp + q) * stride + src[e]] : 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (sp + q < nsplit) sum[e] += x[e][q];
    }
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = half_s * sum[e];
    if (mirror) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = e * 256 + t;
            tr[idx % kGfRows][idx / kGfRows] = v[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = e * 256 + t;
            v[e] = tr[idx / kGramTile][idx % kGramTile];
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = e * 256 + t;
        const int64_t i = (int64_t)ti * kGramTile + x0 + idx / kGramTile;
        const int64_t j = (int64_t)tj * kGramTile + idx % kGramTile;
        if (i < r && j < ldg) gs[i * ldg + j] = Cvt<E>::from_f(j < r ? v[e] : 0.0f);
    }
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
__device__ __forceinline__ void norm_finalize_body(const float* __restrict__ pbase, int nbase,
                                                  const float* __restrict__ pcross, int ncross, int64_t d_out,
                                                  float two_s, const float* __restrict__ m, float eps,
                                                  float* __restrict__ wnorm, float* __restrict__ g, const int64_t i,
                                                  const Balance bal = Balance{1, 0, 1}) {
    if (i >= d_out) return;
    if (bal.nwg > 0) nbase = ncross = bal.slots((int)(i / Big::BM));   // this row's m-tile's slots
    // m is loaded ahead of the partials, so both come back in one memory
    // round trip; partials are loaded in batches of 16 (both kinds together)
    // before they are summed, each kind in partial order
    const float mi = m ? m[i] : 0.0f;
    float base = 0.0f, cd = 0.0f;
    const int total = nbase + ncross;
    for (int c0 = 0; c0 < total; c0 += 16) {
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int c = c0 + t;
            x[t] = c < nbase ? pbase[(int64_t)c * d_out + i]
                             : (c < total ? pcross[(int64_t)(c - nbase) * d_out + i] : 0.0f);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int c = c0 + t;
            if (c < nbase)
                base += x[t];
            else if (c < total)
                cd += x[t];
        }
    }
    const float n2 = fmaxf(fmaf(two_s, cd, base), 0.0f);
    const float wn = sqrtf(n2);
    wnorm[i] = wn;
    if (m) g[i] = mi / fmaxf(wn, eps);
}

// ------------------------------------------------------------- launches
// Kernels of one norm, and of a group of norms in one launch per stage.  A
// group runs each stage of every member in a single grid: member j owns
// workgroups [start[j], start[j+1]), and its starts are multiples of the XCD
// count, so member-local workgroup ids keep their XCD.
template <bool BAL>
__global__ __launch_bounds__(Big::NTH, Big::WG_PER_CU * Big::NW / 4) void w0_pass_big(W0PassArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[Big::LDS_BYTES];
    if constexpr (BAL)
        w0_pass_big_body_balanced(a, blockIdx.x, smem);
    else
        w0_pass_big_body(a, blockIdx.x, smem);
}

__global__ __launch_bounds__(256) void gram_split_bf16(GramArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[gram_split_lds<kGramStages>()];
    gram_split_bf16_body<kGramStages>(a, blockIdx.x, smem);
}

template <typename E>
__global__ __launch_bounds__(256) void gram_finalize(const float* __restrict__ part, int nsplit, int64_t rnp,
                                                     int64_t r, int64_t ldg, float half_s, E* __restrict__ gs) {
    __shared__ float tr[kGfRows][kGramTile + 2];
    gram_finalize_body<E>(part, nsplit, rnp, r, ldg, half_s, gs, blockIdx.x, tr);
}

__global__ __launch_bounds__(256) void norm_finalize(const float* __restrict__ pbase, int nbase,
                                                     const float* __restrict__ pcross, int ncross, int64_t d_out,
                                                     float two_s, const float* __restrict__ m, float eps,
                                                     float* __restrict__ wnorm, float* __restrict__ g,
                                                     Balance bal) {
    norm_finalize_body(pbase, nbase, pcross, ncross, d_out, two_s, m, eps, wnorm, g,
                       (int64_t)blockIdx.x * 256 + threadIdx.x, bal);
}

struct GramFinArgs {
    const float* part;
    int nsplit;
    int64_t rnp, r, ldg;
    float half_s;
    void* gs;
};

struct NormFinArgs {
    const float* pbase;
    const float* pcross;
    int nbase, ncross;
    int64_t d_out;
    float two_s, eps;
    const float* m;
    float* wnorm;
    float* g;
    Balance bal;
};

template <typename A>
struct Group {
    A a[kMaxNormGroup];
    int start[kMaxNormGroup + 1];
    int n;
};

// member owning workgroup id (wave-uniform; at most kMaxNormGroup compares)
template <typename A>
__device__ __forceinline__ int group_member(const Group<A>& g, int id) {
    int j = 0;
    while (j + 1 < g.n && id >= g.start[j + 1]) ++j;
    return j;
}

template <bool BAL>
__global__ __launch_bounds__(Big::NTH, Big::WG_PER_CU * Big::NW / 4) void w0_pass_big_group(Group<W0PassArgs> g) {
    __shared__ __attribute__((aligned(1024))) char smem[Big::LDS_BYTES];
    const int j = group_member(g, blockIdx.x);
    if (BAL && g.a[j].bal.nwg > 0)
        w0_pass_big_body_balanced(g.a[j], blockIdx.x - g.start[j], smem);
    else
        w0_pass_big_body(g.a[j], blockIdx.x - g.start[j], smem);
}

__global__ __launch_bounds__(256) void gram_split_bf16_group(Group<GramArgs> g) {
    __shared__ __attribute__((aligned(1024))) char smem[gram_split_lds<kGramStagesGroup>()];
    const int j = group_member(g, blockIdx.x);
    gram_split_bf16_body<kGramStagesGroup>(g.a[j], blockIdx.x - g.start[j], smem);
}

__global__ __launch_bounds__(256) void gram_finalize_group(Group<GramFinArgs> g) {
    __shared__ float tr[kGfRows][kGramTile + 2];
    const int j = group_member(g, blockIdx.x);
    const GramFinArgs& a = g.a[j];
    gram_finalize_body<bf16_t>(a.part, a.nsplit, a.rnp, a.r, a.ldg, a.half_s, static_cast<bf16_t*>(a.gs),
                               blockIdx.x - g.start[j], tr);
}

__global__ __launch_bounds__(256) void norm_finalize_group(Group<NormFinArgs> g) {
    const int j = group_member(g, blockIdx.x);
    const NormFinArgs& a = g.a[j];
    norm_finalize_body(a.pbase, a.nbase, a.pcross, a.ncross, a.d_out, a.two_s, a.m, a.eps, a.wnorm, a.g,
                       (int64_t)(blockIdx.x - g.start[j]) * 256 + threadIdx.x, a.bal);
}

// ------------------------------------------------------------- configs
struct TileCfg {
    int wm, wn, mt, nt;
};
// Ordered by the width BN of the slice of r a workgroup covers.
constexpr TileCfg kCfgs[] = {
    {4, 1, 2, 1},    // narrow, BM 128, BN 16
    {4, 1, 2, 2},    // narrow, BM 128, BN 32
    {4, 1, 2, 4},    // narrow, BM 128, BN 64
    {1, 4, 8, 1},    // wide,   BM 128, BN 64
    {1, 4, 8, 2},    // wide,   BM 128, BN 128
    {1, 4, 8, 3},    // wide,   BM 128, BN 192
    {1, 4, 8, 6},    // wide,   BM 128, BN 384
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);
// bf16 at 32 < r <= 64: the narrow tile walks K through per-wave LDS-DMA
// rings (96 KB per workgroup, one per CU), each wave with its own copy of
// the A tile; where its workgroups take more than one round, the wide tile
// of the same BN, whose four waves share one A tile in LDS, runs instead.
// Measured on MI355X (norm per call, both forming the Gram term in the
// pass): one round, narrow against wide, 4096^2 r = 64 19.3 against 25.6 us,
// r = 48 19.2 against 25.4, 1024 x 8192 r = 64 19.8 against 26.0; two or
// more rounds, wide against narrow, 8192^2 r = 64 45.1 against 50.1, r = 40
// 44.7 against 48.8, 8192 x 4096 30.1 against 32.8, 16384 x 4096 r = 48 52.6
// against 58.9, 28672 x 8192 r = 64 143.1 against 156.8.
constexpr int kNarrow64Cfg = 2;

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
        case 5: return launch_w0_cfg<E, 5, AL>(a, grid, st);
        default:
            if constexpr (sizeof(E) == 2) return launch_w0_cfg<E, 6, AL>(a, grid, st);
            return hipErrorInvalidValue;
    }
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// LDS-DMA paths: 16-byte aligned rows, and byte offsets inside one tile of
// rows that fit the 31-bit buffer offsets.
template <typename E>
bool operands_aligned(const NormPlan& p, const void* W0, const void* A, const void* B) {
    constexpr int VEC = Mma<E>::VEC;
    const int64_t span =
        (int64_t)(p.bm > p.bn ? p.bm : p.bn) * (p.d_in > p.ldg ? p.d_in : p.ldg) * (int64_t)sizeof(E);
    return p.d_in % VEC == 0 && p.r % VEC == 0 && al16(W0) && al16(A) && al16(B) && span < (1LL << 30);
}

// Whether this plan's W0 pass forms the Gram term itself (the kernel-side
// condition is GramInPass for the same tile configuration).
template <typename E>
bool gram_in_pass(const NormPlan& p, bool aligned) {
    if (p.big || p.cfg < 0) return false;
    const TileCfg t = kCfgs[p.cfg];
    return sizeof(E) == 2 && aligned && ((t.wn == 1 && t.nt <= 4) || (t.wn == 4 && t.nt == 1));
}

// Whether the norm runs as the single whole-row kernel (w0_rows_narrow):
// when its 16-row workgroups make exactly one round (4081 <= d_out <= 4096)
// and W0 has at most 2^25 elements.  Measured on MI355X at r <= 32, both
// forms walking K through LDS-DMA rings: 4096^2 r = 16 10.7 against 14.8 us
// for the K-split pass plus assembly, r = 32 12.8 against 17.2 us, 4096 x
// 8192 r = 16 16.2 against 22.5 us.  With more rows (several rounds, the
// whole-row kernel then feeding registers directly) the K-split pass is as
// fast or faster: 16384 x 2048 r = 16 20.5 against 21.1 us, 8192 x 4096
// r = 24 21.6 against 26.4 us, 6144^2 r = 16 a tie; and so it is below one
// workgroup per CU (2048 x 8192 r = 16 17.5 against 19.0 us with the
// register-fed kernels).
constexpr int64_t kRowsFormMaxElems = int64_t(1) << 25;
constexpr int64_t kRowsFormMinRows = int64_t(kRowsPerWg) * (kNumCU - 1) + 1;
constexpr int64_t kRowsFormMaxRows = int64_t(kRowsPerWg) * kNumCU;

template <typename E>
bool rows_form(const NormPlan& p, bool aligned) {
    return gram_in_pass<E>(p, aligned) && kCfgs[p.cfg].wn == 1 && kCfgs[p.cfg].nt <= 2 &&
           p.d_out * p.d_in <= kRowsFormMaxElems &&
           p.d_out >= kRowsFormMinRows &&
           p.d_out <= kRowsFormMaxRows;
}

// Arguments and grids of the three stages of one norm (not base-only).
struct NormLaunch {
    GramArgs ga;
    unsigned ggrid;
    GramFinArgs gf;
    unsigned gfgrid;
    W0PassArgs wa;
    int wgrid;
    NormFinArgs nf;
    unsigned nfgrid;
};

template <typename E>
NormLaunch make_norm_launch(const NormPlan& p, bool aligned, const void* W0, const void* A, const void* B,
                            const float* m, float s, float eps, float* wnorm, float* g, void* ws) {
    char* w = static_cast<char*>(ws);
    const int64_t d_out = p.d_out, d_in = p.d_in, r = p.r;
    NormLaunch L;
    float* gpart = reinterpret_cast<float*>(w + p.off_gpart);
    GramArgs& ga = L.ga;
    ga.c.left0 = Operand{A, d_in, r, d_in};
    ga.c.right0 = ga.c.left0;
    ga.c.left1 = ga.c.right1 = Operand{nullptr, 0, 0, 0};
    ga.c.nkt0 = (int)((d_in + Mma<E>::BK - 1) / Mma<E>::BK);
    ga.c.nkt1 = 0;
    ga.ntiles = p.gram_tiles;
    ga.nsplit = p.gram_split;
    ga.nupper = p.gram_tiles * (p.gram_tiles + 1) / 2;
    ga.rnp = (int64_t)p.gram_tiles * kGramTile;
    ga.part = gpart;
    if (sizeof(E) == 2 && aligned && p.gram_xcd)   // gram_split_bf16
        L.ggrid = (unsigned)(kNumXCD * ((ga.nsplit + kNumXCD - 1) / kNumXCD) * ga.nupper);
    else
        L.ggrid = (unsigned)(ga.nupper * ga.nsplit);
    L.gf = GramFinArgs{gpart, ga.nsplit, ga.rnp, r, p.ldg, 0.5f * s, w + p.off_gs};
    L.gfgrid = (unsigned)(p.gram_tiles * p.gram_tiles * kGfPerTile);

    W0PassArgs& wa = L.wa;
    wa.bal = p.bal_nwg > 0 ? Balance{p.bal_units, p.bal_nwg, p.bal_nkt} : Balance{1, 0, 1};
    wa.c.left0 = Operand{W0, d_in, d_out, d_in};
    wa.c.right0 = Operand{A, d_in, r, d_in};
    wa.c.left1 = Operand{B, r, d_out, r};
    wa.c.right1 = Operand{w + p.off_gs, p.ldg, r, r};
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
    wa.part_base = reinterpret_cast<float*>(w + p.off_pbase);
    wa.part_cross = reinterpret_cast<float*>(w + p.off_pcross);
    wa.half_s = 0.5f * s;
    if (gram_in_pass<E>(p, aligned)) wa.c.nkt1 = 0;   // no Gs k-tiles: the pass forms the Gram term
    if (p.bal_nwg > 0) {
        L.wgrid = p.bal_nwg;
    } else if (wa.xcd_map) {
        const int per = kNumXCD / Q;   // m-tiles per XCD slot
        L.wgrid = kNumXCD * ((p.n_mtiles + per - 1) / per);
    } else {
        L.wgrid = Q * p.n_mtiles;
    }
    L.nf = NormFinArgs{wa.part_base, wa.part_cross, p.ksplit, Q, d_out, 2.0f * s, eps, m, wnorm, g, wa.bal};
    L.nfgrid = (unsigned)((d_out + 255) / 256);
    return L;
}

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
                                                                        wnorm, g, Balance{1, 0, 1});
        return hipGetLastError();
    }
    const bool al = operands_aligned<E>(p, W0, A, B);
    if (p.big && !al) return hipErrorInvalidValue;   // the caller runs the fallback plan
    if (rows_form<E>(p, al)) {
        if constexpr (sizeof(E) == 2) {
            W0RowsArgs ra;
            ra.c.left0 = Operand{W0, d_in, d_out, d_in};
            ra.c.right0 = Operand{A, d_in, r, d_in};
            ra.c.left1 = ra.c.right1 = Operand{nullptr, 0, 0, 0};
            ra.c.nkt0 = p.nkt_w0;
            ra.c.nkt1 = 0;
            ra.B = B;
            ra.m = m;
            ra.d_out = d_out;
            ra.r = r;
            ra.half_s = 0.5f * s;
            ra.two_s = 2.0f * s;
            ra.eps = eps;
            ra.wnorm = wnorm;
            ra.g = g;
            const unsigned grid = (unsigned)((d_out + kRowsPerWg - 1) / kRowsPerWg);
            if (kCfgs[p.cfg].nt == 1)
                w0_rows_narrow<1><<<grid, kRowsWaves * 64, 0, st>>>(ra);
            else
                w0_rows_narrow<2><<<grid, kRowsWaves * 64, 0, st>>>(ra);
            return hipGetLastError();
        }
    }
    const NormLaunch L = make_norm_launch<E>(p, al, W0, A, B, m, s, eps, wnorm, g, ws);

    // 1. Gs = (s/2) A A^T, unless the W0 pass forms the Gram term
    if (!gram_in_pass<E>(p, al)) {
        if (sizeof(E) == 2 && al && p.gram_xcd) {
            gram_split_bf16<<<L.ggrid, 256, 0, st>>>(L.ga);
        } else {
            if (al)
                gram_partial<E, true><<<L.ggrid, 256, 0, st>>>(L.ga);
            else
                gram_partial<E, false><<<L.ggrid, 256, 0, st>>>(L.ga);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        gram_finalize<E><<<L.gfgrid, 256, 0, st>>>(L.gf.part, L.gf.nsplit, L.gf.rnp, L.gf.r, L.gf.ldg, L.gf.half_s,
                                                   static_cast<E*>(L.gf.gs));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // 2. streaming pass over [W0 | B] x [A | Gs]^T with the row-dot epilogue
    if constexpr (sizeof(E) == 2) {
        if (p.big) {
            if (p.bal_nwg > 0)
                w0_pass_big<true><<<L.wgrid, Big::NTH, 0, st>>>(L.wa);
            else
                w0_pass_big<false><<<L.wgrid, Big::NTH, 0, st>>>(L.wa);
            e = hipGetLastError();
        } else {
            e = al ? launch_w0<E, true>(p.cfg, L.wa, L.wgrid, st) : launch_w0<E, false>(p.cfg, L.wa, L.wgrid, st);
        }
    } else {
        e = al ? launch_w0<E, true>(p.cfg, L.wa, L.wgrid, st) : launch_w0<E, false>(p.cfg, L.wa, L.wgrid, st);
    }
    if (e != hipSuccess) return e;

    // 3. assemble
    norm_finalize<<<L.nfgrid, 256, 0, st>>>(L.nf.pbase, L.nf.nbase, L.nf.pcross, L.nf.ncross, L.nf.d_out,
                                            L.nf.two_s, L.nf.m, L.nf.eps, L.nf.wnorm, L.nf.g, L.nf.bal);
    return hipGetLastError();
}

}  // namespace

namespace {

// The balanced split is taken when the uniform one fills less than
// kBalanceMaxFill percent of a round and its workgroups walk at least
// kBalanceMinKtiles 64-wide k-tiles (3840 of K).  Measured on MI355X at
// r = 384, with 32-wide k-tiles: 28672 x 8192 (112 m-tiles, 8576 of K per
// workgroup) 240.4 -> 233.2 us; with 1920-2880 of K per workgroup the second
// epilogue costs more than the idle CUs (27648 x 5120 a tie, 14336 x 8192
// 132.1 -> 136.1 us, 28672 x 4096 135.3 -> 139.5 us, 20000 x 8200 188.0 ->
// 190.8 us).
constexpr int64_t kBalanceMaxFill = 95;
constexpr int kBalanceMinKtiles = 60;

NormPlan plan_norm_impl(int64_t d_out, int64_t d_in, int64_t r, int dtype, bool base_only, bool allow_big) {
    NormPlan p{};
    p.dtype = dtype;
    p.d_out = d_out;
    p.d_in = d_in;
    p.r = r;
    p.base_only = base_only;
    const int esz = (int)dtype_size(dtype);
    const int vec = 16 / esz;
    const int gram_bk = dtype == kF32 ? Mma<float>::BK : Mma<bf16_t>::BK;
    if (base_only) {
        p.off_pbase = 0;
        p.bytes = align_up((size_t)d_out * 4, 256);
        return p;
    }
    // 256 x 384 tiles from r = 129: above 128 they beat the 128 x 192 tiles
    // even with a third or more of the tile's columns zero (measured on
    // MI355X: 8192^2 r = 160 84.1 -> 69.3 us, r = 192 84.0 -> 70.9 us, 5120^2
    // r = 192 63.3 -> 42.9 us, 4096^2 r = 192 37.4 -> 36.3 us); at r <= 128
    // the zero columns' MFMAs cost more than the tiles save (8192^2 r = 128
    // 55.3 against 66.1 us, 28672 x 8192 r = 128 160.1 against 188.9 us).
    p.big = allow_big && dtype == kBF16 && r > 128;
    int ks = 1;
    if (p.big) {
        p.cfg = -1;
        p.bm = Big::BM;
        p.bn = Big::BN;
        p.bk = Big::BK;
        p.n_mtiles = (int)((d_out + p.bm - 1) / p.bm);
        p.n_ntiles = (int)((r + p.bn - 1) / p.bn);
        p.nkt_w0 = (int)((d_in + p.bk - 1) / p.bk);
        p.nkt_g = (int)((r + p.bk - 1) / p.bk);
        const int nkt = p.nkt_w0 + p.nkt_g;
        // Measured: a single round of workgroups beats several, whose every
        // round pays the cold start and the epilogue again; so split K as far
        // as one round allows, keeping >= 4 k-tiles (256 of K) per workgroup.
        const int64_t tiles = (int64_t)p.n_mtiles * p.n_ntiles;
        const int64_t round = (int64_t)kNumCU * Big::WG_PER_CU;
        ks = tiles >= round ? 1 : (int)(round / tiles);
        if (ks > 64) ks = 64;
        while (ks > 1 && nkt / ks < 4) --ks;
        // A uniform split that leaves CUs idle (112 m-tiles in two K-chunks
        // use 224 of 256) is traded for equal ranges over all CUs when the
        // workgroups are long: some then run two segments, i.e. two
        // epilogues.
        if (p.n_ntiles == 1 && tiles < round && tiles * ks * 100 < round * kBalanceMaxFill &&
            nkt / ks >= kBalanceMinKtiles) {
            const Balance b{tiles * nkt, (int)round, nkt};
            p.bal_nwg = b.nwg;
            p.bal_nkt = nkt;
            p.bal_units = b.units;
            int most = 1;
            for (int mt = 0; mt < p.n_mtiles; ++mt) most = b.slots(mt) > most ? b.slots(mt) : most;
            ks = most;   // partial slots per row
        }
    } else {
        // widest configuration this dtype instantiates (fp32 fragments double
        // the register footprint, so fp32 stops at BN = 192)
        const int max_cfg = dtype == kF32 ? 5 : kNumCfgs - 1;
        int cfg = 0;
        while (cfg < max_cfg && kCfgs[cfg].wn * kCfgs[cfg].nt * 16 < r) ++cfg;
        auto tiles_for = [&](int c) {
            p.cfg = c;
            p.bm = kCfgs[c].wm * kCfgs[c].mt * 16;
            p.bn = kCfgs[c].wn * kCfgs[c].nt * 16;
            p.bk = gram_bk;
            p.n_mtiles = (int)((d_out + p.bm - 1) / p.bm);
            p.n_ntiles = (int)((r + p.bn - 1) / p.bn);
            p.nkt_w0 = (int)((d_in + p.bk - 1) / p.bk);
            p.nkt_g = (int)((r + p.bk - 1) / p.bk);
            const int nkt = p.nkt_w0 + p.nkt_g;
            // k-split: W0 is cut into ks K-stripes per m-tile.  Workgroup ids
            // place stripe c on XCD c % 8, and streaming W0 measures near the
            // HBM roofline when every XCD owns its own stripe (ks a multiple
            // of 8) but ~40% lower with 4 stripes; beyond that, split further
            // only to give >= 2 workgroups per CU.  Every stripe keeps >= 8
            // k-tiles.
            ks = 1;
            while (ks < kNumXCD && nkt / (2 * ks) >= 8) ks *= 2;
            while (ks < 64 && (int64_t)p.n_mtiles * p.n_ntiles * ks < 2 * kNumCU && nkt / (2 * ks) >= 8) ks *= 2;
        };
        tiles_for(cfg);
        if (cfg == kNarrow64Cfg && dtype == kBF16 && (int64_t)p.n_mtiles * ks > kNumCU) tiles_for(cfg + 1);
    }
    p.ksplit = ks;
    // Gram
    const int gram_nkt = (int)((d_in + gram_bk - 1) / gram_bk);
    p.gram_tiles = (int)((r + kGramTile - 1) / kGramTile);
    const int nupper = p.gram_tiles * (p.gram_tiles + 1) / 2;
    int gs = (kNumCU + nupper - 1) / nupper;
    const int max_split = gram_nkt / 4 > 1 ? gram_nkt / 4 : 1;
    if (gs > max_split) gs = max_split;
    if (gs < 1) gs = 1;
    // bf16: splits in whole multiples of the XCD count, one K-slice per XCD
    // (at most 256 / nupper workgroups' worth, each >= 4 k-tiles)
    p.gram_xcd = false;
    if (dtype == kBF16 && gram_nkt >= 4 * kNumXCD) {
        int x = kNumXCD;
        while (x + kNumXCD <= 64 && (int64_t)(x + kNumXCD) * nupper <= kNumCU && gram_nkt / (x + kNumXCD) >= 4)
            x += kNumXCD;
        gs = x;
        p.gram_xcd = true;
    }
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

}  // namespace

// The large-tile plan needs 16-byte aligned operands; calls whose pointers
// are not aligned run the fallback plan, so the workspace covers both.
NormPlan plan_norm(int64_t d_out, int64_t d_in, int64_t r, int dtype, bool base_only) {
    NormPlan p = plan_norm_impl(d_out, d_in, r, dtype, base_only, true);
    p.bytes_needed = p.bytes;
    if (p.big) {
        const NormPlan f = plan_norm_impl(d_out, d_in, r, dtype, base_only, false);
        if (f.bytes > p.bytes_needed) p.bytes_needed = f.bytes;
    }
    return p;
}

hipError_t launch_norm(const NormPlan& p, const void* W0, const void* A, const void* B, const float* m, float s,
                       float eps, float* wnorm, float* g, void* workspace, hipStream_t stream) {
    if (p.dtype == kF32) return norm_typed<float>(p, W0, A, B, m, s, eps, wnorm, g, workspace, stream);
    if (p.big && !operands_aligned<bf16_t>(p, W0, A, B)) {
        const NormPlan f = plan_norm_impl(p.d_out, p.d_in, p.r, p.dtype, p.base_only, false);
        return norm_typed<bf16_t>(f, W0, A, B, m, s, eps, wnorm, g, workspace, stream);
    }
    return norm_typed<bf16_t>(p, W0, A, B, m, s, eps, wnorm, g, workspace, stream);
}

size_t norm_group_workspace_bytes(int n, const int64_t* d_out, const int64_t* d_in, int64_t r, int dtype) {
    size_t total = 0;
    for (int j = 0; j < n; ++j) total += align_up(plan_norm(d_out[j], d_in[j], r, dtype, false).bytes_needed, 256);
    return total;
}

// One call for several norms that share r (for example all projections of
// one layer).  When every member takes the aligned bf16 large-tile path, each
// stage runs once for the whole group (four launches in all); otherwise the
// members run one after another.  Either way a member's kernels, tiling and
// summation order are those of its own single call, so the results are
// bitwise the same.
hipError_t launch_norm_group(int n, const NormMember* mem, int64_t r, int dtype, float eps, void* workspace,
                             hipStream_t st) {
    static_assert(sizeof(Group<W0PassArgs>) <= 4096 && sizeof(Group<GramArgs>) <= 4096, "kernel argument size");
    NormPlan plans[kMaxNormGroup];
    char* wsj[kMaxNormGroup];
    size_t off = 0;
    bool grouped = dtype == kBF16;
    for (int j = 0; j < n; ++j) {
        const NormMember& M = mem[j];
        plans[j] = plan_norm(M.d_out, M.d_in, r, dtype, M.s == 0.0f);
        wsj[j] = static_cast<char*>(workspace) + off;
        off += align_up(plan_norm(M.d_out, M.d_in, r, dtype, false).bytes_needed, 256);
        grouped = grouped && plans[j].big && plans[j].gram_xcd && !plans[j].base_only &&
                  operands_aligned<bf16_t>(plans[j], M.W0, M.A, M.B);
    }
    if (!grouped) {
        for (int j = 0; j < n; ++j) {
            const NormMember& M = mem[j];
            const hipError_t e = launch_norm(plans[j], M.W0, M.A, M.B, M.m, M.s, eps, M.wnorm, M.g, wsj[j], st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    Group<GramArgs> gg;
    Group<GramFinArgs> gf;
    Group<W0PassArgs> gw;
    Group<NormFinArgs> gn;
    gg.n = gf.n = gw.n = gn.n = n;
    gg.start[0] = gf.start[0] = gw.start[0] = gn.start[0] = 0;
    auto pad8 = [](int x) { return (x + kNumXCD - 1) / kNumXCD * kNumXCD; };
    NormLaunch L[kMaxNormGroup];
    for (int j = 0; j < n; ++j) {
        const NormMember& M = mem[j];
        L[j] = make_norm_launch<bf16_t>(plans[j], true, M.W0, M.A, M.B, M.m, M.s, eps, M.wnorm, M.g, wsj[j]);
        gf.a[j] = L[j].gf;
        gf.start[j + 1] = gf.start[j] + (int)L[j].gfgrid;
        gn.a[j] = L[j].nf;
        gn.start[j + 1] = gn.start[j] + (int)L[j].nfgrid;
    }
    // Gram and W0 pass: members with the longest workgroups (most k-tiles per
    // K-chunk) go first, so the short workgroups of the others fill the last
    // round's idle CUs instead of the long ones running alone at the end (a
    // stable order: ties keep member order).  Each member keeps its own plan,
    // so its result is unchanged.
    auto longest_first = [&](auto kt_per_wg, int (&ord)[kMaxNormGroup]) {
        for (int i = 0; i < n; ++i) {
            int k = i;
            while (k > 0 && kt_per_wg(ord[k - 1]) < kt_per_wg(i)) {
                ord[k] = ord[k - 1];
                --k;
            }
            ord[k] = i;
        }
    };
    int og[kMaxNormGroup], ow[kMaxNormGroup];
    longest_first([&](int j) { return (L[j].ga.c.nkt0 + L[j].ga.nsplit - 1) / L[j].ga.nsplit; }, og);
    longest_first(
        [&](int j) {
            if (plans[j].bal_nwg > 0) return (int)((plans[j].bal_units + plans[j].bal_nwg - 1) / plans[j].bal_nwg);
            const int nkt = plans[j].nkt_w0 + plans[j].nkt_g;
            return (nkt + plans[j].ksplit - 1) / plans[j].ksplit;
        },
        ow);
    for (int i = 0; i < n; ++i) {
        gg.a[i] = L[og[i]].ga;
        gg.start[i + 1] = gg.start[i] + pad8((int)L[og[i]].ggrid);
        gw.a[i] = L[ow[i]].wa;
        gw.start[i + 1] = gw.start[i] + pad8(L[ow[i]].wgrid);
    }
    hipError_t e;
    gram_split_bf16_group<<<gg.start[n], 256, 0, st>>>(gg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gram_finalize_group<<<gf.start[n], 256, 0, st>>>(gf);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bool any_bal = false;
    for (int j = 0; j < n; ++j) any_bal = any_bal || plans[j].bal_nwg > 0;
    if (any_bal)
        w0_pass_big_group<true><<<gw.start[n], Big::NTH, 0, st>>>(gw);
    else
        w0_pass_big_group<false><<<gw.start[n], Big::NTH, 0, st>>>(gw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    norm_finalize_group<<<gn.start[n], 256, 0, st>>>(gn);
    return hipGetLastError();
}

}  // namespace dora
