// common.hpp -- device helpers shared by the libbin1 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bin1 {

constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float h2f(uint16_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, h);
    return (float)v;                         // exact (v_cvt_f32_f16 keeps subnormals)
}

__device__ __forceinline__ uint16_t f2h_rne(float f) {
    _Float16 v = (_Float16)f;                // v_cvt_f16_f32, round to nearest even
    return __builtin_bit_cast(uint16_t, v);
}

// a * b for a, b < 2^24, as one v_mul_u32_u24.  Written as an instruction because the
// compiler fuses a plain (masked) 24-bit product with a following add into a 64-bit
// multiply-add, whose unused high input it may place in a register that a buffer load is
// still filling; the wait-count pass then drains every load in flight at that point.
__device__ __forceinline__ unsigned mul24(unsigned a, unsigned b) {
    unsigned r;
    asm("v_mul_u32_u24 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Sum over the 64 lanes of a wave (butterfly; every lane ends with the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

}  // namespace bin1
