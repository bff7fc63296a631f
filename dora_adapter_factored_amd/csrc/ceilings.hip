// Ceiling measurements for the DoRA kernels on gfx950: what the chip
// sustains for the operations the hot path is built from, measured with
// kernels that do nothing else.  They are context for the hot path's
// roofline fractions, not part of it, and live in their own library
// (libdora_ceilings.so) so the product library's ABI stays the method's.
//
//  - MFMA only: the W0 pass's instruction and wave tile (32 x 32 x 16 bf16,
//    a 4 x 3 block tile per wave, 192 accumulator registers, 8 waves a
//    workgroup, one workgroup a CU), and the same work as 16 x 16 x 32
//    blocks (8 x 6 per wave); operands stay in registers, nothing touches
//    memory inside the loop.
//  - streams in the compose kernels' access patterns: 2 reads + 1 write and
//    3 reads + 2 writes of 16-byte packets, non-temporal, grid-strided.
//  - read rate of one CU: every workgroup reads its own region (or all read
//    one region, which then sits in L2) with up to 8 waves of 16-byte loads.
//  - the W0 pass's streaming pattern without MFMA: 256 workgroups of 256
//    rows x one K-chunk, K-chunk c on XCD c, 64-byte row pieces per k-tile
//    through a 4-stage LDS-DMA ring with a barrier per tile, the walk over
//    K rotated per workgroup as in the pass, optionally with the 384-row A
//    tile of each k-tile as well.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dora_device.h"
#include "dora_gfx950.h"

namespace dora {
namespace {

// ------------------------------------------------------------- MFMA only
__global__ __launch_bounds__(512) void mfma_32x32x16_loop(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    f32x16_t acc[4][3];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 3; ++n)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[m][n][e] = 0.0f;
    bf16x8_t a[4], b[3];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) a[m][e] = static_cast<bf16_t>((float)((lane + m * 7 + e) & 15) * 0.0625f);
#pragma unroll
    for (int n = 0; n < 3; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) b[n][e] = static_cast<bf16_t>((float)((lane * 3 + n + e) & 15) * 0.0625f);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 3; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[n], a[m], acc[m][n], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 3; ++n)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[m][n][e];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(512) void mfma_16x16x32_loop(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    f32x4_t acc[8][6];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 6; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t a[8], b[6];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) a[m][e] = static_cast<bf16_t>((float)((lane + m * 7 + e) & 15) * 0.0625f);
#pragma unroll
    for (int n = 0; n < 6; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) b[n][e] = static_cast<bf16_t>((float)((lane * 3 + n + e) & 15) * 0.0625f);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int n = 0; n < 6; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b[n], acc[m][n], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 6; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[m][n][e];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// ------------------------------------------------------------- streams
// n16: 16-byte packets per array.  The arithmetic is an integer add per
// word, so only the bytes moved matter.
__global__ __launch_bounds__(256) void stream_r2w1(const u32x4_t* a, const u32x4_t* b, u32x4_t* y, int64_t n16) {
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 2 * step) {
        const bool two = i + step < n16;
        const u32x4_t a0 = __builtin_nontemporal_load(a + i), b0 = __builtin_nontemporal_load(b + i);
        u32x4_t a1 = a0, b1 = b0;
        if (two) {
            a1 = __builtin_nontemporal_load(a + i + step);
            b1 = __builtin_nontemporal_load(b + i + step);
        }
        __builtin_nontemporal_store(a0 + b0, y + i);
        if (two) __builtin_nontemporal_store(a1 + b1, y + i + step);
    }
}

__global__ __launch_bounds__(256) void stream_r2w2(const u32x4_t* a, const u32x4_t* b, u32x4_t* y, u32x4_t* z,
                                                   int64_t n16) {
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += step) {
        const u32x4_t a0 = __builtin_nontemporal_load(a + i), b0 = __builtin_nontemporal_load(b + i);
        __builtin_nontemporal_store(a0 + b0, y + i);
        __builtin_nontemporal_store(a0 ^ b0, z + i);
    }
}

__global__ __launch_bounds__(256) void stream_r3w2(const u32x4_t* a, const u32x4_t* b, const u32x4_t* c, u32x4_t* y,
                                                   u32x4_t* z, int64_t n16) {
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += step) {
        const u32x4_t a0 = __builtin_nontemporal_load(a + i), b0 = __builtin_nontemporal_load(b + i);
        const u32x4_t c0 = __builtin_nontemporal_load(c + i);
        __builtin_nontemporal_store(a0 + b0, y + i);
        __builtin_nontemporal_store(a0 ^ c0, z + i);
    }
}

// The same three streams, blocked: workgroup w owns packets
// [w * 256 * kStreamU, (w + 1) * 256 * kStreamU) and every thread issues all
// of its kStreamU loads per input before its stores (the compose kernels'
// shape: many workgroups, several 16-byte loads in flight per thread).
constexpr int kStreamU = 4;

template <int PATTERN>
__global__ __launch_bounds__(256) void stream_blocked(const u32x4_t* a, const u32x4_t* b, const u32x4_t* c,
                                                      u32x4_t* y, u32x4_t* z, int64_t n16) {
    const int64_t i0 = (int64_t)blockIdx.x * (256 * kStreamU) + threadIdx.x;
    u32x4_t av[kStreamU], bv[kStreamU], cv[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
        const int64_t i = i0 + (int64_t)u * 256;
        if (i < n16) {
            av[u] = __builtin_nontemporal_load(a + i);
            bv[u] = __builtin_nontemporal_load(b + i);
            if (PATTERN == 1) cv[u] = __builtin_nontemporal_load(c + i);
        }
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
        const int64_t i = i0 + (int64_t)u * 256;
        if (i < n16) {
            __builtin_nontemporal_store(av[u] + bv[u], y + i);
            if (PATTERN == 1) __builtin_nontemporal_store(av[u] ^ cv[u], z + i);
            if (PATTERN == 2) __builtin_nontemporal_store(av[u] ^ bv[u], z + i);
        }
    }
}

// ------------------------------------------------------------- one CU's read rate
// Workgroup w reads bytes_per_wg bytes starting at w * stride (stride 0: all
// workgroups read the same region), reps times, 8 loads of 16 bytes in
// flight per thread, and writes an XOR of what it read.
__global__ __launch_bounds__(512) void cu_read(const u32x4_t* buf, int64_t bytes_per_wg, int64_t stride, int reps,
                                               uint32_t* out) {
    const u32x4_t* p = buf + (int64_t)blockIdx.x * (stride / 16);
    const int64_t n16 = bytes_per_wg / 16;
    u32x4_t x = u32x4_t{0u, 0u, 0u, 0u};
    for (int r = 0; r < reps; ++r) {
        for (int64_t i0 = threadIdx.x; i0 < n16; i0 += 8 * (int64_t)blockDim.x) {
            u32x4_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int64_t i = i0 + k * (int64_t)blockDim.x;
                v[k] = i < n16 ? p[i] : u32x4_t{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) x ^= v[k];
        }
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// ------------------------------------------------------------- the W0 pass's stream
// 256 workgroups: 32 row tiles of 256 rows x 8 K-chunks, chunk c on XCD c
// (workgroup ids are dealt to XCDs round robin).  Each k-tile moves 256 rows
// x 64 bytes of W0 (and, with_a, 384 rows x 64 bytes of A) into a 4-stage
// LDS ring by DMA, three tiles ahead; a barrier per tile; every thread reads
// 16 bytes of the landed tile so the data is consumed.  AMODE 1 reads A
// row-major ([r][d_in], each k-tile 384 pieces of 64 bytes a row apart), as
// the W0 pass does; AMODE 2 reads the same bytes k-tile-major ([k-tile][r][32
// elements], each k-tile's A tile one contiguous 24 KB run).  AMODE 3 moves
// what AMODE 1 moves with K cut into seven chunks over 224 workgroups: chunk
// x < 7 on XCD x for m-tiles [0, 28), the last XCD taking m-tiles 28..31 of
// every chunk; each CU then walks 8/7 as many k-tiles while each XCD moves
// the same bytes as in the eight-chunk layout.
constexpr int kRows = 256, kArows = 384, kStages = 4, kRowB = 64;
constexpr int kStageBytes = (kRows + kArows) * kRowB;

template <int AMODE>
__global__ __launch_bounds__(512) void w0_stream(const bf16_t* W0, const bf16_t* A, int64_t d_out, int64_t d_in,
                                                 int64_t r, uint32_t* out) {
    // DMA instructions per wave per tile: 16 (W0) and 24 (A) groups of 16 rows over 8 waves
    constexpr int PER = kRows / 16 / 8 + (AMODE ? kArows / 16 / 8 : 0);
    constexpr int NCH = AMODE == 3 ? 7 : 8;   // K-chunks
    __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int id = blockIdx.x;
    int kc = id % 8, mtile = id / 8;
    if (AMODE == 3 && kc == 7) {   // the last XCD: 4 m-tiles of each chunk
        kc = mtile / 4;
        mtile = 28 + mtile % 4;
    }
    const int64_t m0 = (int64_t)mtile * kRows;
    const int nkt = (int)((d_in * 2 + kRowB - 1) / kRowB);
    const int kt0 = (int)((int64_t)kc * nkt / NCH), kt1 = (int)((int64_t)(kc + 1) * nkt / NCH);
    const int n = kt1 - kt0;
    // the walk starts at a rotated k-tile, as the W0 pass's does (workgroups
    // reading the same column offset of a power-of-two pitch at the same time
    // pile onto a few memory channels)
    const int rot = n > 0 ? (int)(((unsigned)id * 7u + ((unsigned)id >> 3) * 3u) % (unsigned)n) : 0;
    auto rsrc = [&](const bf16_t* p, int64_t row0, int64_t rows) {
        const uint64_t base = reinterpret_cast<uint64_t>(p + row0 * d_in);
        int64_t bytes = (rows - row0) * d_in * 2;
        if (bytes < 0) bytes = 0;
        if (bytes > 0x7ffffff0) bytes = 0x7ffffff0;
        i32x4_t rs;
        rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
        rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
        rs[2] = __builtin_amdgcn_readfirstlane((int)bytes);
        rs[3] = kRsrcWord3;
        return rs;
    };
    const i32x4_t rw = rsrc(W0, m0, d_out), ra = rsrc(A, 0, r);
    const int ldb = (int)(d_in * 2);
    // lane l moves 16 bytes (slot l % 4) of row l / 4 of a 16-row group
    const int loff = (lane >> 2) * ldb + (lane & 3) * 16;
    // steps past the last tile still issue (zeros), so every wait below
    // leaves exactly the two younger tiles in flight
    auto issue = [&](int i) __attribute__((always_inline)) {
        const bool valid = i < n;
        int t = (valid ? i : 0) + rot;
        if (t >= n) t -= n;
        const int kb = (kt0 + t) * kRowB;
        const bool in = valid && kb + (lane & 3) * 16 < ldb;
        char* st = smem + (i % kStages) * kStageBytes;
#pragma unroll
        for (int g0 = 0; g0 < kRows / 16; g0 += 8) {
            const int g = g0 + wave;
            raw_buffer_load_lds(rw, (lds_void_t*)(st + g * 1024), 16, in ? loff + kb + g * 16 * ldb : kOutOfRange, 0,
                                0, 0);
        }
        if (AMODE == 1 || AMODE == 3) {
#pragma unroll
            for (int g0 = 0; g0 < kArows / 16; g0 += 8) {
                const int g = g0 + wave;
                raw_buffer_load_lds(ra, (lds_void_t*)(st + kRows * kRowB + g * 1024), 16,
                                    in ? loff + kb + g * 16 * ldb : kOutOfRange, 0, 0, 0);
            }
        } else if (AMODE == 2) {
            const int tb = (kt0 + t) * kArows * kRowB;   // the k-tile's contiguous A tile
#pragma unroll
            for (int g0 = 0; g0 < kArows / 16; g0 += 8) {
                const int g = g0 + wave;
                raw_buffer_load_lds(ra, (lds_void_t*)(st + kRows * kRowB + g * 1024), 16,
                                    valid ? tb + g * 1024 + lane * 16 : kOutOfRange, 0, 0, 0);
            }
        }
    };
    u32x4_t x = u32x4_t{0u, 0u, 0u, 0u};
    for (int i = 0; i < kStages - 1; ++i) issue(i);
    for (int j = 0; j < n; ++j) {
        wait_vmcnt<2 * PER>();   // tile j landed (j + 1 and j + 2 may be in flight)
        __syncthreads();
        issue(j + kStages - 1);
        const char* st = smem + (j % kStages) * kStageBytes;
        x ^= *reinterpret_cast<const u32x4_t*>(st + threadIdx.x * 16);
    }
    wait_vmcnt<0>();
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace
}  // namespace dora

// C entry points (argument checks only; the caller sizes every buffer as the
// comment on each states).
extern "C" {

// out: 512 floats per workgroup.  kind 0: 32x32x16, kind 1: 16x16x32.
int dora_ceiling_mfma(int kind, int iters, int workgroups, float* out, void* stream) {
    if (!out || iters < 1 || workgroups < 1) return 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == 0)
        dora::mfma_32x32x16_loop<<<workgroups, 512, 0, st>>>(iters, out);
    else if (kind == 1)
        dora::mfma_16x16x32_loop<<<workgroups, 512, 0, st>>>(iters, out);
    else
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// pattern 0: y = f(a, b) (2 reads + 1 write); pattern 1: y, z = f(a, b, c)
// (3 reads + 2 writes); pattern 2: y, z = f(a, b) (2 reads + 2 writes).
// Every array holds bytes bytes, a multiple of 16.  workgroups >= 1: that
// many workgroups stride over the arrays; 0: the blocked form, one
// workgroup per 256 * 4 packets.
int dora_ceiling_stream(int pattern, const void* a, const void* b, const void* c, void* y, void* z, int64_t bytes,
                        int workgroups, void* stream) {
    if (!a || !b || !y || bytes <= 0 || bytes % 16 || workgroups < 0) return 1;
    if ((pattern == 1 && (!c || !z)) || (pattern == 2 && !z) || pattern < 0 || pattern > 2) return 1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    typedef dora::u32x4_t V;
    if (workgroups == 0) {
        const int64_t n16 = bytes / 16, per = 256 * dora::kStreamU;
        const int64_t grid = (n16 + per - 1) / per;
        if (grid > 0x7fffffff) return 1;
        const V *pa = static_cast<const V*>(a), *pb = static_cast<const V*>(b), *pc = static_cast<const V*>(c);
        V *py = static_cast<V*>(y), *pz = static_cast<V*>(z);
        if (pattern == 0)
            dora::stream_blocked<0><<<(unsigned)grid, 256, 0, st>>>(pa, pb, pc, py, pz, n16);
        else if (pattern == 1)
            dora::stream_blocked<1><<<(unsigned)grid, 256, 0, st>>>(pa, pb, pc, py, pz, n16);
        else
            dora::stream_blocked<2><<<(unsigned)grid, 256, 0, st>>>(pa, pb, pc, py, pz, n16);
        return hipGetLastError() == hipSuccess ? 0 : 4;
    }
    if (pattern == 0) {
        dora::stream_r2w1<<<workgroups, 256, 0, st>>>(static_cast<const V*>(a), static_cast<const V*>(b),
                                                      static_cast<V*>(y), bytes / 16);
    } else if (pattern == 2) {
        if (!z) return 1;
        dora::stream_r2w2<<<workgroups, 256, 0, st>>>(static_cast<const V*>(a), static_cast<const V*>(b),
                                                      static_cast<V*>(y), static_cast<V*>(z), bytes / 16);
    } else if (pattern == 1) {
        if (!c || !z) return 1;
        dora::stream_r3w2<<<workgroups, 256, 0, st>>>(static_cast<const V*>(a), static_cast<const V*>(b),
                                                      static_cast<const V*>(c), static_cast<V*>(y),
                                                      static_cast<V*>(z), bytes / 16);
    } else {
        return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// buf holds at least (workgroups - 1) * stride + bytes_per_wg bytes; out
// holds waves * 64 words per workgroup.
int dora_ceiling_cu_read(const void* buf, int64_t bytes_per_wg, int64_t stride, int reps, int workgroups, int waves,
                         void* out, void* stream) {
    if (!buf || !out || bytes_per_wg < 16 || bytes_per_wg % 16 || stride < 0 || stride % 16 || reps < 1 ||
        workgroups < 1 || waves < 1 || waves > 8)
        return 1;
    dora::cu_read<<<workgroups, waves * 64, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const dora::u32x4_t*>(buf), bytes_per_wg, stride, reps, static_cast<uint32_t*>(out));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// W0 [d_out, d_in] and A [r, d_in] bf16, d_in a multiple of 8 and d_out up
// to 32 row tiles of 256 (rows of A past r read zeros); out holds 256 x 512
// words.  with_a: 0 W0 alone, 1 A row-major, 2 A k-tile-major (offsets past
// A's r * d_in elements read zeros), 3 as 1 in seven K-chunks on 224
// workgroups (d_out exactly 32 row tiles).
int dora_ceiling_w0_stream(const void* W0, const void* A, int64_t d_out, int64_t d_in, int64_t r, int with_a,
                           void* out, void* stream) {
    if (!W0 || !A || !out || d_out < 1 || d_out > 32 * 256 || d_in < 8 || d_in % 8 || r < 1 ||
        r * d_in * 2 >= (int64_t)1 << 31 || (int64_t)256 * d_in * 2 >= (int64_t)1 << 31)
        return 1;
    const auto* w = static_cast<const dora::bf16_t*>(W0);
    const auto* a = static_cast<const dora::bf16_t*>(A);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t* o = static_cast<uint32_t*>(out);
    if (with_a == 1)
        dora::w0_stream<1><<<256, 512, 0, st>>>(w, a, d_out, d_in, r, o);
    else if (with_a == 2)
        dora::w0_stream<2><<<256, 512, 0, st>>>(w, a, d_out, d_in, r, o);
    else if (with_a == 0)
        dora::w0_stream<0><<<256, 512, 0, st>>>(w, a, d_out, d_in, r, o);
    else if (with_a == 3 && d_out == 32 * 256)
        dora::w0_stream<3><<<224, 512, 0, st>>>(w, a, d_out, d_in, r, o);
    else
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
