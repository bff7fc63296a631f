// gfx950 memory primitives shared by the MFMA kernels: LDS DMA (buffer
// loads that write LDS directly), vector-memory waits, and the chunk swizzle
// of 64-byte LDS rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Buffer load of 4 dwords per lane straight into LDS (M0-based destination,
// lane l writes 16 bytes at dst + 16 l).  An offset at or beyond the buffer's
// size reads zeros.
__device__ void raw_buffer_load_lds(i32x4_t rsrc, lds_void_t* lds, int size, int voffset, int soffset,
                                    int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// A per-lane buffer offset that is always out of range: the load reads zeros.
constexpr int kOutOfRange = (int)0x80000000;

// Cache-policy operand of a buffer load on gfx940-class chips: the NT
// (non-temporal) bit, for data read exactly once.  Its lines are the first
// the caches drop, so data that is re-read (the A tile every workgroup of an
// XCD streams) keeps its place in L2.
constexpr int kCachePolicyNT = 2;

// Buffer resource word 3 used for raw byte-addressed buffers here.
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt on vector-memory operations only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).  Vector-memory
// loads retire in issue order, so vmcnt <= N means every load but the N most
// recent has landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt on LDS / scalar-memory operations only (lgkmcnt = 0).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads it does not wait for
// outstanding global loads and stores (on gfx9 one counter covers both), so
// stores issued before it stay in flight.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Chunk swizzle of 64-byte rows: logical chunk c of row i sits in slot
// c ^ swz64(i).  For a fixed chunk, the 16 rows of any aligned 16-row block
// map to 16 distinct (row mod 4, slot) pairs and the even (odd) rows of any
// aligned 8 rows to 4 distinct slots, so 16-lane (64-bank) and 8-lane
// (32-bank) phases of a fragment read are conflict-free.  It depends only on
// the row modulo 16, the height of one DMA group.
__device__ __forceinline__ int swz64(int row) { return ((row >> 2) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1); }

}  // namespace dora
