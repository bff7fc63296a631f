// DoRA merge for serving on gfx950: W_merged = diag(g) (W0 + s B A).
//
// "LoRA & DoRA: The Math, Memory, and Trade-offs" §6 gives the merged DoRA
// weight m (W0 + sBA) / ||W0 + sBA||_row, an ordinary matrix with no adapter
// left at inference; "Scaling DoRA" §4 computes g = m / max(wnorm, eps) once
// from the factored norm, so the merge takes g as an input and never forms a
// norm of its own.
//
// Mapping onto the chip.  B A is a dense contraction over K = r, so it runs on
// MFMA; the rest (read W0, scale, write W) is a stream over d_out x d_in that
// bounds the call.  Both MFMA operands must hold K contiguously per lane: B
// does ([d_out][r] row-major), A does not ([r][d_in]), so transpose_a first
// writes A^T into the workspace as [d_in][r_pad], zero-padded to whole 64-byte
// k-tiles (the tail k-tile then needs no masking on that side).  With bf16
// and r <= 32 (one k-tile) the tile kernel builds that A^T tile from A itself
// and no transpose runs.
//
// merge_tile: one workgroup per 128 x 128 output tile, 4 waves (2 x 2), each a
// 64 x 64 block of 32 x 32 MFMA tiles with fp32 accumulators.  k-tiles of 64
// bytes per row (32 bf16 or 16 fp32) of both operands are staged through LDS
// (register-prefetched double buffer, swizzled rows).  The W0 tile is loaded
// into registers at the start so its HBM latency hides under the MFMA loop;
// the epilogue passes the accumulators through an fp32 LDS tile so that each
// thread finishes whole 16-byte chunks: W = g_i * fmaf(s, acc, W0), rounded
// once.  W may alias W0 exactly: every element is read and written by the
// same thread of the same workgroup.
#include "dora_device.h"
#include "dora_gfx950.h"
#include "dora_launch.h"

namespace dora {
namespace {

constexpr int kNumXCD = 8;

// ------------------------------------------------------------ transpose A
constexpr int kTrTile = 64;

template <typename E>
__global__ __launch_bounds__(256) void transpose_a(const E* __restrict__ A, int64_t r, int64_t d_in,
                                                   E* __restrict__ At, int64_t r_pad) {
    __shared__ E tile[kTrTile][kTrTile + 2];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * kTrTile, k0 = (int64_t)blockIdx.y * kTrTile;
#pragma unroll
    for (int i = 0; i < kTrTile / 4; ++i) {
        const int64_t k = k0 + ty + 4 * i, n = n0 + tx;
        tile[ty + 4 * i][tx] = (k < r && n < d_in) ? A[k * d_in + n] : Cvt<E>::from_f(0.0f);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTrTile / 4; ++i) {
        const int64_t n = n0 + ty + 4 * i, k = k0 + tx;
        if (n < d_in && k < r_pad) At[n * r_pad + k] = tile[tx][ty + 4 * i];
    }
}

// 16-byte form (d_in a multiple of the vector width, A 16-byte aligned): each
// thread loads whole 16-byte runs of a row of A, scatters them into an LDS
// tile held n-major, and stores whole 16-byte runs of a row of A^T.
template <typename E>
__global__ __launch_bounds__(256) void transpose_a_vec(const E* __restrict__ A, int64_t r, int64_t d_in,
                                                       E* __restrict__ At, int64_t r_pad) {
    constexpr int VEC = 16 / sizeof(E);
    constexpr int CPR = kTrTile / VEC;          // 16-byte runs per tile row
    constexpr int PITCH = kTrTile + VEC;        // elements per LDS row (16-byte aligned rows)
    __shared__ __attribute__((aligned(16))) E tile[kTrTile][PITCH];   // [n][k]
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kTrTile, k0 = (int64_t)blockIdx.y * kTrTile;
#pragma unroll
    for (int i = 0; i < kTrTile * CPR / 256; ++i) {
        const int c = tid + 256 * i, kr = c / CPR, cc = c % CPR;
        const int64_t k = k0 + kr, n = n0 + (int64_t)cc * VEC;
        Pack<E> v;
        v.u = (k < r && n < d_in) ? *reinterpret_cast<const u32x4_t*>(A + k * d_in + n) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < VEC; ++e) tile[cc * VEC + e][kr] = v.e[e];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTrTile * CPR / 256; ++i) {
        const int c = tid + 256 * i, nr = c / CPR, kc = c % CPR;
        const int64_t n = n0 + nr, k = k0 + (int64_t)kc * VEC;
        if (n < d_in && k < r_pad)
            *reinterpret_cast<u32x4_t*>(At + n * r_pad + k) = *reinterpret_cast<const u32x4_t*>(&tile[nr][kc * VEC]);
    }
}

// bf16 form: a thread loads 16 bytes from each of two adjacent k-rows of A,
// packs each column's (k, k + 1) pair into one 32-bit word and writes it to
// an LDS tile held n-major with a 33-word pitch (a wave's writes then fall
// in 64 distinct banks); it then reads 4 words (8 k-values) of one n and
// stores them as one 16-byte run of A^T.
constexpr int kTrPitchW = kTrTile / 2 + 1;          // words per LDS row of the bf16 tile

__global__ __launch_bounds__(256) void transpose_a_bf16(const bf16_t* __restrict__ A, int64_t r, int64_t d_in,
                                                        bf16_t* __restrict__ At, int64_t r_pad) {
    __shared__ uint32_t tile[kTrTile][kTrPitchW];   // [n][k / 2]
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kTrTile, k0 = (int64_t)blockIdx.y * kTrTile;
    {
        const int cc = tid & 7, kp = tid >> 3;       // 8 column chunks x 32 k-pairs
        const int64_t n = n0 + (int64_t)cc * 8, k = k0 + 2 * kp;
        Pack<bf16_t> lo, hi;
        lo.u = (k < r && n < d_in) ? *reinterpret_cast<const u32x4_t*>(A + k * d_in + n) : u32x4_t{0u, 0u, 0u, 0u};
        hi.u = (k + 1 < r && n < d_in) ? *reinterpret_cast<const u32x4_t*>(A + (k + 1) * d_in + n)
                                       : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, lo.e[e]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, hi.e[e]) << 16);
            tile[cc * 8 + e][kp] = w;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i, nr = c >> 3, kc = c & 7;
        const int64_t n = n0 + nr, k = k0 + (int64_t)kc * 8;
        if (n < d_in && k < r_pad) {
            u32x4_t v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = tile[nr][kc * 4 + j];
            *reinterpret_cast<u32x4_t*>(At + n * r_pad + k) = v;
        }
    }
}

// A^T as the tile kernel's LDS stages hold it: block (nt, kt) is rows
// nt*128 .. nt*128 + 127 of A^T (columns of A) by K values kt*32 .. kt*32 + 31,
// 64 bytes per row, with the row's 16-byte chunk c at slot c ^ swz64(row).
// Blocks are 8 KB and contiguous, so every DMA instruction of a stage copies
// 1 KiB of consecutive bytes (eight whole 128-byte lines) instead of sixteen
// 64-byte row pieces.  Rows past d_in and K past r are zeros.  The transpose
// goes through LDS as in transpose_a_bf16.
constexpr int kTileRows = 128, kTileK = 32;
constexpr int kTilePad = 256;   // rows of A^T written: whole tiles of either tile kernel

__global__ __launch_bounds__(256) void transpose_a_tiles_bf16(const bf16_t* __restrict__ A, int64_t r,
                                                              int64_t d_in, char* __restrict__ At, int64_t r_pad,
                                                              int64_t n_pad) {
    __shared__ uint32_t tile[kTrTile][kTrPitchW];   // [n][k / 2]
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kTrTile, k0 = (int64_t)blockIdx.y * kTrTile;
    {
        const int cc = tid & 7, kp = tid >> 3;
        const int64_t n = n0 + (int64_t)cc * 8, k = k0 + 2 * kp;
        Pack<bf16_t> lo, hi;
        lo.u = (k < r && n < d_in) ? *reinterpret_cast<const u32x4_t*>(A + k * d_in + n) : u32x4_t{0u, 0u, 0u, 0u};
        hi.u = (k + 1 < r && n < d_in) ? *reinterpret_cast<const u32x4_t*>(A + (k + 1) * d_in + n)
                                       : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, lo.e[e]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, hi.e[e]) << 16);
            tile[cc * 8 + e][kp] = w;
        }
    }
    __syncthreads();
    const int64_t nk = r_pad / kTileK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i, nr = c >> 3, kc = c & 7;
        const int64_t n = n0 + nr, k = k0 + (int64_t)kc * 8;
        if (n < n_pad && k < r_pad) {
            u32x4_t v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = tile[nr][kc * 4 + j];
            const int rr = (int)(n % kTileRows), ch = (int)((k % kTileK) / 8);
            const int64_t blk = (n / kTileRows) * nk + k / kTileK;
            *reinterpret_cast<u32x4_t*>(At + (blk * kTileRows + rr) * 64 + ((ch ^ swz64(rr)) << 4)) = v;
        }
    }
}

// ------------------------------------------------------------- MFMA traits
// A k-tile holds 64 bytes of K per row.  In each of its two MFMA k-steps a
// lane supplies the 16-byte chunk 2*step + lane/32 of its row, for both
// operands, so every product pairs matching K.
template <typename E> struct MergeMma;

template <> struct MergeMma<bf16_t> {
    static constexpr int KT = 32;
    __device__ __forceinline__ static void mma(f32x16_t& c, u32x4_t a, u32x4_t b) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};

template <> struct MergeMma<float> {
    static constexpr int KT = 16;
    // four K=2 products: element i of the chunk, lanes < 32 and >= 32 hold
    // two different chunks, so each K value enters exactly once
    __device__ __forceinline__ static void mma(f32x16_t& c, u32x4_t a, u32x4_t b) {
        const f32x4_t av = __builtin_bit_cast(f32x4_t, a), bv = __builtin_bit_cast(f32x4_t, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[i], c, 0, 0, 0);
    }
};

constexpr int kBM = 128, kBN = 128, kNTh = 256;
constexpr int kRowB = 64;                                // bytes per LDS row per k-tile
constexpr int kStageB = (kBM + kBN) * kRowB;             // 16 KB
constexpr int kEpiPitch = kBN + 8;                       // floats per LDS row of the epilogue tile
constexpr int kEpiB = kBM * kEpiPitch * 4;               // 69,632 B
constexpr int kLdsB = kEpiB > 2 * kStageB ? kEpiB : 2 * kStageB;

struct MergeArgs {
    const void* W0;
    const void* At;
    const void* B;
    const float* g;
    void* W;
    float s;
    int64_t d_out, d_in, r, r_pad;
    int n_mt, n_nt;   // output tiles along d_out and d_in
    int per_xcd;      // tiles per XCD slice (grid = 8 * per_xcd)
};

// workgroup -> output tile: consecutive workgroups go to consecutive XCDs;
// each XCD takes one contiguous slice of the tile list, which runs through
// panels of 8 row-tiles column by column, so the workgroups resident on one
// XCD share a few row-tiles of B and column-tiles of A^T in its L2.
__device__ __forceinline__ bool merge_tile_of(const MergeArgs& a, int& mt, int& nt) {
    const int id = blockIdx.x;
    const int t = (id % kNumXCD) * a.per_xcd + id / kNumXCD;
    if (t >= a.n_mt * a.n_nt) return false;
    constexpr int PM = 8;
    const int panel = t / (PM * a.n_nt);
    const int u = t - panel * PM * a.n_nt;
    const int pm = min(PM, a.n_mt - panel * PM);
    mt = panel * PM + u % pm;
    nt = u / pm;
    return true;
}

template <typename E, bool ALIGNED>
__device__ __forceinline__ u32x4_t load_b_chunk(const E* B, int64_t row, int64_t k, const MergeArgs& a) {
    constexpr int VEC = 16 / sizeof(E);
    if (ALIGNED) {
        if (row < a.d_out && k < a.r) return *reinterpret_cast<const u32x4_t*>(B + row * a.r + k);
        return u32x4_t{0u, 0u, 0u, 0u};
    } else {
        Pack<E> v;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v.e[e] = (row < a.d_out && k + e < a.r) ? B[row * a.r + k + e] : Cvt<E>::from_f(0.0f);
        return v.u;
    }
}

template <typename E, bool ALIGNED>
__global__ __launch_bounds__(kNTh, 2) void merge_tile(MergeArgs a) {
    int mt, nt;
    if (!merge_tile_of(a, mt, nt)) return;
    constexpr int VEC = 16 / sizeof(E);
    constexpr int KT = MergeMma<E>::KT;
    constexpr int CPR = kBN / VEC;                       // 16-byte chunks per output row
    constexpr int NOUT = kBM * CPR / kNTh;               // output chunks per thread
    __shared__ __attribute__((aligned(16))) char lds[kLdsB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)mt * kBM, n0 = (int64_t)nt * kBN;
    const E* W0 = static_cast<const E*>(a.W0);
    const E* B = static_cast<const E*>(a.B);
    const E* At = static_cast<const E*>(a.At);

    // W0 tile into registers now; consumed by the epilogue
    u32x4_t w0v[NOUT];
#pragma unroll
    for (int i = 0; i < NOUT; ++i) {
        const int c = tid + kNTh * i, row = c / CPR, cc = c % CPR;
        const int64_t gm = m0 + row, gn = n0 + (int64_t)cc * VEC;
        if (ALIGNED) {
            w0v[i] = (gm < a.d_out && gn < a.d_in)
                         ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W0 + gm * a.d_in + gn))
                         : u32x4_t{0u, 0u, 0u, 0u};
        } else {
            Pack<E> v;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                v.e[e] = (gm < a.d_out && gn + e < a.d_in) ? W0[gm * a.d_in + gn + e] : Cvt<E>::from_f(0.0f);
            w0v[i] = v.u;
        }
    }

    // k-tile staging: 2 chunks of B rows and 2 of A^T rows per thread
    const int nk = (int)(a.r_pad / KT);
    u32x4_t lreg[2], rreg[2];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + kNTh * i, row = c >> 2, q = c & 3;
            const int64_t k = (int64_t)kt * KT + q * VEC;
            lreg[i] = load_b_chunk<E, ALIGNED>(B, m0 + row, k, a);
            const int64_t gn = n0 + row;
            rreg[i] = gn < a.d_in ? *reinterpret_cast<const u32x4_t*>(At + gn * a.r_pad + k)
                                  : u32x4_t{0u, 0u, 0u, 0u};
        }
    };
    auto store_tile = [&](int buf) {
        char* st = lds + buf * kStageB;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + kNTh * i, row = c >> 2, q = c & 3;
            *reinterpret_cast<u32x4_t*>(st + row * kRowB + ((q ^ swz64(row)) << 4)) = lreg[i];
            *reinterpret_cast<u32x4_t*>(st + (kBM + row) * kRowB + ((q ^ swz64(row)) << 4)) = rreg[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    load_tile(0);
    store_tile(0);
    if (nk > 1) load_tile(1);
    __syncthreads();
    const int fr = lane & 31, fh = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const char* st = lds + (kt & 1) * kStageB;
#pragma unroll
        for (int step = 0; step < 2; ++step) {
            const int q = 2 * step + fh;
            u32x4_t av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + fr;
                av[i] = *reinterpret_cast<const u32x4_t*>(st + row * kRowB + ((q ^ swz64(row)) << 4));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wn * 64 + j * 32 + fr;
                bv[j] = *reinterpret_cast<const u32x4_t*>(st + (kBM + row) * kRowB + ((q ^ swz64(row)) << 4));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) MergeMma<E>::mma(acc[i][j], av[i], bv[j]);
        }
        if (kt + 1 < nk) store_tile((kt + 1) & 1);
        if (kt + 2 < nk) load_tile(kt + 2);
        __syncthreads();
    }

    // epilogue: accumulators -> fp32 LDS tile -> whole 16-byte output chunks
    float* epi = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                const int col = wn * 64 + j * 32 + fr;
                epi[row * kEpiPitch + col] = acc[i][j][e];
            }
    __syncthreads();
    E* W = static_cast<E*>(a.W);
    const float s = a.s;
#pragma unroll
    for (int i = 0; i < NOUT; ++i) {
        const int c = tid + kNTh * i, row = c / CPR, cc = c % CPR;
        const int64_t gm = m0 + row, gn = n0 + (int64_t)cc * VEC;
        if (gm >= a.d_out || gn >= a.d_in) continue;
        const float gi = a.g[gm];
        const float* src = epi + row * kEpiPitch + cc * VEC;
        Pack<E> w, o;
        w.u = w0v[i];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o.e[e] = Cvt<E>::from_f(gi * fmaf(s, src[e], Cvt<E>::to_f(w.e[e])));
        if (ALIGNED) {
            __builtin_nontemporal_store(o.u, reinterpret_cast<u32x4_t*>(W + gm * a.d_in + gn));
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (gn + e < a.d_in) W[gm * a.d_in + gn + e] = o.e[e];
        }
    }
}

// ------------------------------------------------- LDS-DMA form (aligned)
// The k-tiles of both operands move global -> LDS by DMA through a ring of
// kRing stages; lane l of a DMA instruction moves slot l % 4 of row l / 4 of
// a 16-row group (1 KiB).  Each wave issues kDmaPerWave instructions per
// stage.  The W0 tile is loaded into registers right after the last real
// stage is issued: vector-memory loads retire in issue order, so earlier
// waits would otherwise also wait for W0; issued last, its HBM latency hides
// under the remaining k-tiles, and the waits below let it stay in flight.
constexpr int kRing = 3;
constexpr int kDmaPerWave = (kBM + kBN) / 16 / (kNTh / 64);
constexpr int kEpiRows = 64;                              // epilogue in two 64-row halves
// The DMA kernel's accumulators hold transposed blocks (see merge_tile_dma),
// so a lane writes four consecutive floats of one row; a pitch of 4 mod 64
// banks keeps those 16-byte writes free of bank conflicts.
constexpr int kEpiPitchT = kBN + 4;
static_assert(kRing * kStageB >= kEpiRows * kEpiPitchT * 4, "epilogue half fits in the ring");

struct DmaOp {
    uint32_t base_lo, base_hi;   // first row of the workgroup's tile
    int bytes;                   // from there to the operand's end (clamped to 31 bits)
    int ld_bytes, kmax_bytes;
};

__device__ __forceinline__ DmaOp make_dma_op(const void* p, int64_t ld_bytes, int64_t rows, int64_t row0,
                                             int64_t kmax_bytes) {
    DmaOp d;
    const uint64_t base = reinterpret_cast<uint64_t>(static_cast<const char*>(p) + row0 * ld_bytes);
    int64_t bytes = (rows - row0) * ld_bytes;
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7ffffff0) bytes = 0x7ffffff0;
    d.base_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    d.base_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
    d.bytes = __builtin_amdgcn_readfirstlane((int)bytes);
    d.ld_bytes = __builtin_amdgcn_readfirstlane((int)ld_bytes);
    d.kmax_bytes = __builtin_amdgcn_readfirstlane((int)kmax_bytes);
    return d;
}

// DMA of 16-row group `grp` of k-tile kt into LDS at dst.  lane_off is the
// lane's byte offset inside the group ((l / 4) rows and the chunk its slot
// holds, chunk_b); the group and k-tile offsets move the scalar base, and the
// record count shrinks with it, so rows past the operand read zeros.  Chunks
// past K (kmax) read zeros.  Offsets fit 31 bits: a tile spans 128 rows.
__device__ __forceinline__ void dma_group(const DmaOp& d, int grp, int kt, int lane_off, int chunk_b, char* dst) {
    const int k0b = kt * kRowB;
    const int voff = chunk_b < d.kmax_bytes - k0b ? lane_off : kOutOfRange;
    const int off = grp * 16 * d.ld_bytes + k0b;
    const int left = d.bytes > off ? d.bytes - off : 0;
    const uint64_t addr = (((uint64_t)d.base_hi << 32) | d.base_lo) + (uint32_t)off;
    i32x4_t rs;
    rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
    rs[2] = __builtin_amdgcn_readfirstlane(left);
    rs[3] = kRsrcWord3;
    raw_buffer_load_lds(rs, (lds_void_t*)(dst + grp * 1024), 16, voff, 0, 0, 0);
}

// Wait until a stage has landed while `after` later stages (and, if w0, the
// NW0 W0 loads) may stay in flight.  Both are wave-uniform run-time values;
// each combination gets its own immediate.
template <int NW0, int A>
__device__ __forceinline__ void wait_stage(int after, bool w0) {
    if constexpr (A < 0) {
        wait_vmcnt<0>();
    } else {
        if (after == A) {
            if (w0)
                wait_vmcnt<A * kDmaPerWave + NW0>();
            else
                wait_vmcnt<A * kDmaPerWave>();
            return;
        }
        wait_stage<NW0, A - 1>(after, w0);
    }
}

// DMA of one 1 KiB run of a tiled operand block into LDS at dst.
__device__ __forceinline__ void dma_run(const char* src, int lane, char* dst) {
    const uint64_t addr = reinterpret_cast<uint64_t>(src);
    i32x4_t rs;
    rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(addr >> 32));
    rs[2] = 1024;
    rs[3] = kRsrcWord3;
    raw_buffer_load_lds(rs, (lds_void_t*)dst, 16, lane * 16, 0, 0, 0);
}

// TILED: a.At holds A^T in the stage layout of transpose_a_tiles_bf16.
template <typename E, bool DIRECT, bool TILED = false>
__global__ __launch_bounds__(kNTh, sizeof(E) == 2 ? 3 : 2) void merge_tile_dma(MergeArgs a) {
    int mt, nt;
    if (!merge_tile_of(a, mt, nt)) return;
    constexpr int VEC = 16 / sizeof(E);
    constexpr int CPR = kBN / VEC;
    constexpr int NH = kEpiRows * CPR / kNTh;           // output chunks per thread per half
    constexpr int NW0 = 2 * NH;                         // W0 chunks per thread
    constexpr int NLD = 2 * NW0;                        // loads issued with them: W0 chunk and g of its row
    __shared__ __attribute__((aligned(1024))) char lds[kRing * kStageB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)mt * kBM, n0 = (int64_t)nt * kBN;
    const int esz = (int)sizeof(E);
    const DmaOp lop = make_dma_op(a.B, a.r * esz, a.d_out, m0, a.r * esz);
    const DmaOp rop = make_dma_op(a.At, a.r_pad * esz, a.d_in, n0, a.r_pad * esz);
    const int grow = lane >> 2, slot = lane & 3;
    const int chunk_b = (slot ^ swz64(grow)) * 16;
    const int loff = grow * lop.ld_bytes + chunk_b, roff = grow * rop.ld_bytes + chunk_b;
    const int nk = (int)(a.r_pad / MergeMma<E>::KT);

    auto issue = [&](int kt) {
        char* st = lds + (kt % kRing) * kStageB;
        if constexpr (DIRECT) {
            // low rank (r <= 32, one k-tile): the A^T tile is built from A in
            // place of a transpose launch.  A thread loads a 16-byte run of one
            // row k of A (8 consecutive columns n) and scatters it into the
            // swizzled rows n of the stage; rows k >= r give the zero padding.
#pragma unroll
            for (int q = 0; q < kDmaPerWave / 2; ++q) dma_group(lop, wave + q * (kNTh / 64), kt, loff, chunk_b, st);
            constexpr int KT = MergeMma<E>::KT, NCH = kBN / VEC;
            char* rst = st + kBM * kRowB;
            const E* A = static_cast<const E*>(a.At);
#pragma unroll 1
            for (int c0 = 0; c0 < KT * NCH; c0 += kNTh) {
                const int c = c0 + tid, k = c / NCH, n8 = (c % NCH) * VEC;
                const int64_t gn = n0 + n8;
                Pack<E> v;
                v.u = (k < a.r && gn < a.d_in) ? *reinterpret_cast<const u32x4_t*>(A + (int64_t)k * a.d_in + gn)
                                               : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int nn = n8 + e;
                    *reinterpret_cast<E*>(rst + nn * kRowB + (((k / VEC) ^ swz64(nn)) << 4) + (k % VEC) * (int)sizeof(E)) =
                        v.e[e];
                }
            }
            return;
        }
        const char* rblk = static_cast<const char*>(a.At) + ((int64_t)nt * nk + kt) * (kBN * kRowB);
#pragma unroll
        for (int q = 0; q < kDmaPerWave / 2; ++q) {
            const int grp = wave + q * (kNTh / 64);
            dma_group(lop, grp, kt, loff, chunk_b, st);
            if constexpr (TILED)
                dma_run(rblk + grp * 1024, lane, st + kBM * kRowB + grp * 1024);
            else
                dma_group(rop, grp, kt, roff, chunk_b, st + kBM * kRowB);
        }
    };
    const E* W0 = static_cast<const E*>(a.W0);
    // W0 chunks and the g of their rows, loaded unconditionally (addresses
    // clamped into the tensors) so that every wave issues the same count
    u32x4_t w0v[NW0];
    float gv[NW0];
    auto issue_w0 = [&]() {
#pragma unroll
        for (int i = 0; i < NW0; ++i) {
            const int h = i / NH, c = tid + kNTh * (i % NH);
            const int64_t gm = min(m0 + h * kEpiRows + c / CPR, a.d_out - 1);
            const int64_t gn = min(n0 + (int64_t)(c % CPR) * VEC, a.d_in - VEC);
            w0v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W0 + gm * a.d_in + gn));
            gv[i] = a.g[gm];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    for (int t = 0; t < kRing - 1; ++t)
        if (t < nk) issue(t);
    // W0 goes out in iteration kt_w0, right after the last real stage
    const int kt_w0 = max(0, nk - kRing);
    const int fr = lane & 31, fh = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        // stage kt has landed once only the stages issued after it (and the
        // W0 loads, if issued) are outstanding
        const int after = min(nk, kt + kRing - 1) - kt - 1;
        wait_stage<NLD, kRing - 2>(after, kt > kt_w0);
        lds_barrier();
        if (kt + kRing - 1 < nk) issue(kt + kRing - 1);
        if (kt == kt_w0) issue_w0();
        const char* st = lds + (kt % kRing) * kStageB;
#pragma unroll
        for (int step = 0; step < 2; ++step) {
            const int q = 2 * step + fh;
            u32x4_t av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + fr;
                av[i] = *reinterpret_cast<const u32x4_t*>(st + row * kRowB + ((q ^ swz64(row)) << 4));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wn * 64 + j * 32 + fr;
                bv[j] = *reinterpret_cast<const u32x4_t*>(st + (kBM + row) * kRowB + ((q ^ swz64(row)) << 4));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) MergeMma<E>::mma(acc[i][j], bv[j], av[i]);
        }
    }
    lds_barrier();   // every wave is done with the ring

    // epilogue, one 64-row half at a time: accumulators -> fp32 LDS tile ->
    // whole 16-byte chunks of W.  The MFMAs above take A^T's fragment first,
    // so acc[i][j] is the transposed block: lane l owns row l % 32 of row
    // block i and, in registers 4g .. 4g + 3, columns 8g + 4 (l / 32) .. + 3
    // of column block j, one 16-byte LDS write each.
    float* epi = reinterpret_cast<float*>(lds);
    E* W = static_cast<E*>(a.W);
    const float s = a.s;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (wm == h) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int row = i * 32 + fr;
                        const int col = wn * 64 + j * 32 + 8 * g + 4 * fh;
                        *reinterpret_cast<f32x4_t*>(epi + row * kEpiPitchT + col) =
                            f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                    acc[i][j][4 * g + 3]};
                    }
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const int c = tid + kNTh * i, row = c / CPR, cc = c % CPR;
            const int64_t gm = m0 + h * kEpiRows + row, gn = n0 + (int64_t)cc * VEC;
            if (gm < a.d_out && gn < a.d_in) {
                const float gi = gv[h * NH + i];
                const float* src = epi + row * kEpiPitchT + cc * VEC;
                Pack<E> w, o;
                w.u = w0v[h * NH + i];
#pragma unroll
                for (int e = 0; e < VEC; ++e) o.e[e] = Cvt<E>::from_f(gi * fmaf(s, src[e], Cvt<E>::to_f(w.e[e])));
                __builtin_nontemporal_store(o.u, reinterpret_cast<u32x4_t*>(W + gm * a.d_in + gn));
            }
        }
        lds_barrier();
    }
}

// ------------------------------------------------- large tiles (bf16, aligned)
// The same pipeline on 256 x 256 output tiles with 8 waves in a 2 x 4 grid,
// each a 128 x 64 block (4 x 2 blocks of 32 x 32).  Per output element the
// operand tiles that cross L2 -> LDS halve against 128 x 128 tiles (6 against
// 12 bytes at r = 384), and each k-step's fragment reads feed 8 MFMAs per
// wave instead of 4.  One workgroup per CU: 96 KB of ring, the W0 tile (128
// KB) prefetched into registers after the last stage, the epilogue in four
// 64-row rounds through the ring's LDS.
struct BigMerge {
    static constexpr int BM = 256, BN = 256, WM = 2, WN = 4, NW = WM * WN, NTH = NW * 64;
    static constexpr int WR = BM / WM, WC = BN / WN;     // rows, columns of one wave
    static constexpr int MT = WR / 32, NT = WC / 32;      // 32 x 32 blocks of one wave
    static constexpr int STAGE = (BM + BN) * kRowB;      // 32 KB
    static constexpr int LDMA = BM / 16 / NW, RDMA = BN / 16 / NW;   // DMA groups per wave and stage
    static constexpr int DMA = LDMA + RDMA;
    static constexpr int ER = 64;                        // epilogue rows per round
    static constexpr int ROUNDS = BM / ER;
    static constexpr int PITCH = BN + 4;                 // floats per epilogue row (16-byte writes, no conflicts)
    static constexpr int CPR = BN / 8;                   // 16-byte chunks per output row
    static constexpr int NH = ER * CPR / NTH;            // output chunks per thread per round
    static constexpr int NW0 = ROUNDS * NH;
    static_assert(BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "DMA groups split evenly across waves");
    static_assert(kRing * STAGE >= ER * PITCH * 4, "an epilogue round fits in the ring");
    static_assert(ER % 32 == 0 && WR % ER == 0, "a round takes whole row blocks of one wave row");
};

template <int NW0, int A>
__device__ __forceinline__ void wait_stage_big(int after, bool w0) {
    if constexpr (A < 0) {
        wait_vmcnt<0>();
    } else {
        if (after == A) {
            if (w0)
                wait_vmcnt<A * BigMerge::DMA + NW0>();
            else
                wait_vmcnt<A * BigMerge::DMA>();
            return;
        }
        wait_stage_big<NW0, A - 1>(after, w0);
    }
}

// TILED: a.At holds A^T in the stage layout of transpose_a_tiles_bf16 (a
// 256-row stage is two consecutive 128-row blocks).
template <bool TILED>
__global__ __launch_bounds__(BigMerge::NTH, 1) void merge_tile_big(MergeArgs a) {
    typedef bf16_t E;
    typedef BigMerge G;
    int mt, nt;
    if (!merge_tile_of(a, mt, nt)) return;
    constexpr int VEC = 8;
    constexpr int NLD = G::NW0 + 1;                      // W0 chunks and one g per thread
    static_assert(G::NTH >= G::BM, "one thread per tile row fetches its g");
    __shared__ __attribute__((aligned(1024))) char lds[kRing * G::STAGE + G::BM * 4];
    float* gsm = reinterpret_cast<float*>(lds + kRing * G::STAGE);   // g of the tile's rows

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / G::WN, wn = wave % G::WN;
    const int64_t m0 = (int64_t)mt * G::BM, n0 = (int64_t)nt * G::BN;
    const DmaOp lop = make_dma_op(a.B, a.r * 2, a.d_out, m0, a.r * 2);
    const DmaOp rop = make_dma_op(a.At, a.r_pad * 2, a.d_in, n0, a.r_pad * 2);
    const int grow = lane >> 2, slot = lane & 3;
    const int chunk_b = (slot ^ swz64(grow)) * 16;
    const int loff = grow * lop.ld_bytes + chunk_b, roff = grow * rop.ld_bytes + chunk_b;
    const int nk = (int)(a.r_pad / MergeMma<E>::KT);

    auto issue = [&](int kt) {
        char* st = lds + (kt % kRing) * G::STAGE;
#pragma unroll
        for (int q = 0; q < G::LDMA; ++q) dma_group(lop, wave + q * G::NW, kt, loff, chunk_b, st);
#pragma unroll
        for (int q = 0; q < G::RDMA; ++q) {
            const int grp = wave + q * G::NW;
            if constexpr (TILED) {
                const int64_t blk = ((int64_t)nt * (G::BN / kTileRows) + grp / 8) * nk + kt;
                dma_run(static_cast<const char*>(a.At) + blk * (kTileRows * kRowB) + (grp % 8) * 1024, lane,
                        st + G::BM * kRowB + grp * 1024);
            } else {
                dma_group(rop, grp, kt, roff, chunk_b, st + G::BM * kRowB);
            }
        }
    };
    const E* W0 = static_cast<const E*>(a.W0);
    // W0 chunks and the g of one tile row per thread, loaded unconditionally
    // (addresses clamped into the tensors) so that every wave issues the same
    // count; g goes to LDS when the epilogue starts
    u32x4_t w0v[G::NW0];
    float grow_v;
    auto issue_w0 = [&]() {
#pragma unroll
        for (int i = 0; i < G::NW0; ++i) {
            const int h = i / G::NH, c = tid + G::NTH * (i % G::NH);
            const int64_t gm = min(m0 + h * G::ER + c / G::CPR, a.d_out - 1);
            const int64_t gn = min(n0 + (int64_t)(c % G::CPR) * VEC, a.d_in - VEC);
            w0v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W0 + gm * a.d_in + gn));
        }
        grow_v = a.g[min(m0 + (tid % G::BM), a.d_out - 1)];
    };

    f32x16_t acc[G::MT][G::NT];
#pragma unroll
    for (int i = 0; i < G::MT; ++i)
#pragma unroll
        for (int j = 0; j < G::NT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    for (int t = 0; t < kRing - 1; ++t)
        if (t < nk) issue(t);
    const int kt_w0 = max(0, nk - kRing);
    const int fr = lane & 31, fh = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int after = min(nk, kt + kRing - 1) - kt - 1;
        wait_stage_big<NLD, kRing - 2>(after, kt > kt_w0);
        lds_barrier();
        if (kt + kRing - 1 < nk) issue(kt + kRing - 1);
        if (kt == kt_w0) issue_w0();
        const char* st = lds + (kt % kRing) * G::STAGE;
#pragma unroll
        for (int step = 0; step < 2; ++step) {
            const int q = 2 * step + fh;
            u32x4_t av[G::MT], bv[G::NT];
#pragma unroll
            for (int i = 0; i < G::MT; ++i) {
                const int row = wm * G::WR + i * 32 + fr;
                av[i] = *reinterpret_cast<const u32x4_t*>(st + row * kRowB + ((q ^ swz64(row)) << 4));
            }
#pragma unroll
            for (int j = 0; j < G::NT; ++j) {
                const int row = wn * G::WC + j * 32 + fr;
                bv[j] = *reinterpret_cast<const u32x4_t*>(st + (G::BM + row) * kRowB + ((q ^ swz64(row)) << 4));
            }
#pragma unroll
            for (int i = 0; i < G::MT; ++i)
#pragma unroll
                for (int j = 0; j < G::NT; ++j) MergeMma<E>::mma(acc[i][j], bv[j], av[i]);
        }
    }
    lds_barrier();   // every wave is done with the ring

    // epilogue, one 64-row round at a time (as in merge_tile_dma: acc[i][j]
    // is the transposed block, lane l owning row l % 32 of row block i and
    // columns 8g + 4 (l / 32) .. + 3 of column block j in registers 4g ..)
    float* epi = reinterpret_cast<float*>(lds);
    E* W = static_cast<E*>(a.W);
    const float s = a.s;
    if (tid < G::BM) gsm[tid] = grow_v;
#pragma unroll
    for (int h = 0; h < G::ROUNDS; ++h) {
#pragma unroll
        for (int i = 0; i < G::MT; ++i) {
            if (wm * G::WR + i * 32 >= h * G::ER && wm * G::WR + i * 32 < (h + 1) * G::ER) {
#pragma unroll
                for (int j = 0; j < G::NT; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int row = wm * G::WR + i * 32 - h * G::ER + fr;
                        const int col = wn * G::WC + j * 32 + 8 * g + 4 * fh;
                        *reinterpret_cast<f32x4_t*>(epi + row * G::PITCH + col) =
                            f32x4_t{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                    }
            }
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < G::NH; ++i) {
            const int c = tid + G::NTH * i, row = c / G::CPR, cc = c % G::CPR;
            const int64_t gm = m0 + h * G::ER + row, gn = n0 + (int64_t)cc * VEC;
            if (gm < a.d_out && gn < a.d_in) {
                const float gi = gsm[h * G::ER + row];
                const float* src = epi + row * G::PITCH + cc * VEC;
                Pack<E> w, o;
                w.u = w0v[h * G::NH + i];
#pragma unroll
                for (int e = 0; e < VEC; ++e) o.e[e] = Cvt<E>::from_f(gi * fmaf(s, src[e], Cvt<E>::to_f(w.e[e])));
                __builtin_nontemporal_store(o.u, reinterpret_cast<u32x4_t*>(W + gm * a.d_in + gn));
            }
        }
        lds_barrier();
    }
}

inline const bf16_t* A_bf16(const void* p) { return static_cast<const bf16_t*>(p); }

// Large tiles run one workgroup per CU, so a tile's W0 stream and epilogue
// overlap nothing of its own; with several tiles per CU the 128 x 128 kernel,
// three workgroups per CU hiding each other's phases, is faster (measured on
// MI355X at r = 384: 8192^2 104 against 110 us, 5120 x 27648 219 against 229
// us).  When the large grid is a single round that fills most CUs, its
// halved operand traffic wins (4096^2 35.6 -> 29.3 us, 2048 x 8192 37.5 ->
// 30.9 us, 2560 x 5120 32.6 -> 28.8 us); at 192 tiles it ties (3072 x 4096)
// and at 128 it loses (1024 x 8192 21.6 against 26.9 us).
constexpr int64_t kMergeBigMinTiles = 200, kMergeBigMaxTiles = 256;

template <typename E>
hipError_t merge_typed(const void* W0, const void* A, const void* B, const float* g, float s, int64_t d_out,
                       int64_t d_in, int64_t r, void* W, void* workspace, hipStream_t st) {
    constexpr int KT = MergeMma<E>::KT;
    const int64_t r_pad = (r + KT - 1) / KT * KT;
    E* At = static_cast<E*>(workspace);
    constexpr int VEC = 16 / sizeof(E);
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const dim3 tgrid((unsigned)((d_in + kTrTile - 1) / kTrTile), (unsigned)((r_pad + kTrTile - 1) / kTrTile));
    const bool aligned = d_in % VEC == 0 && r % VEC == 0 && al16(W0) && al16(B) && al16(W);
    // bf16 with one k-tile of r: the tile kernel stages A^T from A itself
    const bool a_direct = sizeof(E) == 2 && aligned && al16(A) && r_pad == KT;
    // 256 x 256 tiles where they make one round of workgroups
    const int64_t big_tiles = ((d_out + BigMerge::BM - 1) / BigMerge::BM) * ((d_in + BigMerge::BN - 1) / BigMerge::BN);
    const bool big = sizeof(E) == 2 && aligned && !a_direct && big_tiles >= kMergeBigMinTiles &&
                     big_tiles <= kMergeBigMaxTiles;
    // the bf16 tile kernels read A^T as contiguous stage blocks
    const bool tiled = sizeof(E) == 2 && aligned && !a_direct && al16(A);
    const int64_t n_pad = (d_in + kTilePad - 1) / kTilePad * kTilePad;
    if (a_direct) {
    } else if (tiled) {
        if constexpr (sizeof(E) == 2)
            transpose_a_tiles_bf16<<<dim3((unsigned)(n_pad / kTrTile), tgrid.y), 256, 0, st>>>(
                A_bf16(A), r, d_in, reinterpret_cast<char*>(At), r_pad, n_pad);
    } else if (d_in % VEC == 0 && al16(A)) {
        if constexpr (sizeof(E) == 2)
            transpose_a_bf16<<<tgrid, 256, 0, st>>>(A_bf16(A), r, d_in, reinterpret_cast<bf16_t*>(At), r_pad);
        else
            transpose_a_vec<E><<<tgrid, 256, 0, st>>>(static_cast<const E*>(A), r, d_in, At, r_pad);
    }
    else
        transpose_a<E><<<tgrid, 256, 0, st>>>(static_cast<const E*>(A), r, d_in, At, r_pad);

    const int64_t bm = big ? BigMerge::BM : kBM, bn = big ? BigMerge::BN : kBN;
    MergeArgs a;
    a.W0 = W0;
    a.At = a_direct ? static_cast<const E*>(A) : At;   // merge_tile_dma<E, true> reads A [r][d_in]
    a.B = B;
    a.g = g;
    a.W = W;
    a.s = s;
    a.d_out = d_out;
    a.d_in = d_in;
    a.r = r;
    a.r_pad = r_pad;
    a.n_mt = (int)((d_out + bm - 1) / bm);
    a.n_nt = (int)((d_in + bn - 1) / bn);
    const int64_t tiles = (int64_t)a.n_mt * a.n_nt;
    a.per_xcd = (int)((tiles + kNumXCD - 1) / kNumXCD);
    const unsigned grid = (unsigned)(a.per_xcd * kNumXCD);
    if (big) {
        if (tiled)
            merge_tile_big<true><<<grid, BigMerge::NTH, 0, st>>>(a);
        else
            merge_tile_big<false><<<grid, BigMerge::NTH, 0, st>>>(a);
    } else if (a_direct) {
        if constexpr (sizeof(E) == 2) merge_tile_dma<E, true><<<grid, kNTh, 0, st>>>(a);
    } else if (tiled) {
        if constexpr (sizeof(E) == 2) merge_tile_dma<E, false, true><<<grid, kNTh, 0, st>>>(a);
    } else if (aligned) {
        merge_tile_dma<E, false><<<grid, kNTh, 0, st>>>(a);
    }
    else {
        merge_tile<E, false><<<grid, kNTh, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

size_t merge_workspace_bytes(int64_t d_in, int64_t r, int dtype) {
    const int64_t kt = dtype == kF32 ? MergeMma<float>::KT : MergeMma<bf16_t>::KT;
    const int64_t r_pad = (r + kt - 1) / kt * kt;
    const int64_t n_pad = (d_in + kTilePad - 1) / kTilePad * kTilePad;   // tiled A^T covers whole tiles
    return align_up((size_t)n_pad * (size_t)r_pad * dtype_size(dtype), 256);
}

hipError_t launch_merge(const void* W0, const void* A, const void* B, const float* g, float s, int64_t d_out,
                        int64_t d_in, int64_t r, int dtype, void* W, void* workspace, hipStream_t stream) {
    if (dtype == kF32) return merge_typed<float>(W0, A, B, g, s, d_out, d_in, r, W, workspace, stream);
    return merge_typed<bf16_t>(W0, A, B, g, s, d_out, d_in, r, W, workspace, stream);
}

}  // namespace dora
