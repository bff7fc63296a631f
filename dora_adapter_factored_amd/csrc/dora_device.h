// Device-side helpers shared by the gfx950 kernels: element conversions and
// 16-byte vector access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// fp32 <-> element conversions.  float -> bf16/f16 rounds to nearest even.
template <typename T> struct Cvt;
template <> struct Cvt<float> {
    __device__ __forceinline__ static float to_f(float x) { return x; }
    __device__ __forceinline__ static float from_f(float x) { return x; }
};
template <> struct Cvt<bf16_t> {
    __device__ __forceinline__ static float to_f(bf16_t x) { return static_cast<float>(x); }
    __device__ __forceinline__ static bf16_t from_f(float x) { return static_cast<bf16_t>(x); }
};
template <> struct Cvt<f16_t> {
    __device__ __forceinline__ static float to_f(f16_t x) { return static_cast<float>(x); }
    __device__ __forceinline__ static f16_t from_f(float x) { return static_cast<f16_t>(x); }
};

// A 16-byte packet of elements of T (8 bf16/f16 or 4 fp32).
template <typename T> struct Pack {
    static constexpr int N = 16 / sizeof(T);
    union {
        u32x4_t u;
        T e[N];
    };
};

template <typename T>
__device__ __forceinline__ Pack<T> load_pack(const T* p) {
    Pack<T> v;
    v.u = *reinterpret_cast<const u32x4_t*>(p);
    return v;
}

// Streaming variants: the data is touched once per call.
template <typename T>
__device__ __forceinline__ Pack<T> load_pack_stream(const T* p) {
    Pack<T> v;
    v.u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return v;
}

template <typename T>
__device__ __forceinline__ void store_pack_stream(T* p, const Pack<T>& v) {
    __builtin_nontemporal_store(v.u, reinterpret_cast<u32x4_t*>(p));
}

}  // namespace dora
