// device_util.h - small device helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfsdp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // one 16-byte granule

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 packed in one word (lo in bits 15:0), round to
// nearest, ties to even, by gfx950's conversion instruction
// (v_cvt_pk_bf16_f32: one instruction for both values, where a software
// rounding takes about six).  Finite values, denormals and infinities round
// exactly as round-to-nearest-even defines (checked against a software
// rounding on every fp32 bit pattern); a NaN stays a NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// One float -> bfloat16 bits, as pack_bf16x2.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// Storage-type traits of the Newton-Schulz buffers: uint16_t holds bf16 bits.
template <typename T> struct Store;
template <> struct Store<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static uint16_t cvt(float f) { return f32_to_bf16(f); }
};
template <> struct Store<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static float cvt(float f) { return f; }
};

// Element offsets into a Newton-Schulz buffer of ld columns stored in panel
// blocks of 256 rows x 128 bytes (CB columns of T; layout.h describes the
// layout).  Offsets fit in 32 bits: the planner keeps every buffer below
// 2 GiB.
template <typename T> struct Panel {
    static constexpr int CB = 128 / int(sizeof(T));  // columns per block
    static constexpr int BE = 256 * CB;              // elements per block
    // element (r, c)
    __device__ __forceinline__ static uint32_t off(int r, int c, int ld) {
        return uint32_t((r >> 8) * (ld / CB) + c / CB) * uint32_t(BE) + uint32_t((r & 255) * CB + (c % CB));
    }
    // from element (r, c) with c % CB == 0 to (r, c + dc), 0 <= dc
    __host__ __device__ static constexpr uint32_t dcol(int dc) { return uint32_t(dc / CB) * BE + uint32_t(dc % CB); }
};

// Parameter / gradient element access by runtime dtype (0 = fp32, 1 = bf16).
__device__ __forceinline__ float load_elem(const void* base, int dtype, int64_t i) {
    return dtype == 1 ? bf16_to_f32(static_cast<const uint16_t*>(base)[i]) : static_cast<const float*>(base)[i];
}
__device__ __forceinline__ void store_elem(void* base, int dtype, int64_t i, float v) {
    if (dtype == 1)
        static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
    else
        static_cast<float*>(base)[i] = v;
}

// Sum over a 64-lane wavefront (fixed butterfly order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Largest k in [0, n) with begin[k] <= x, for a non-decreasing prefix array.
__device__ __forceinline__ int upper_index(const int32_t* begin, int n, int x) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (begin[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace mfsdp
