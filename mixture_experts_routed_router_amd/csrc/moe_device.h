// moe_device.h -- device helpers shared by the HIP kernels of libmoe (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_WAVE 64

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t moe_f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float moe_bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Two floats -> packed bf16x2 (low half = a), nearest even.
__device__ __forceinline__ uint32_t moe_pack_bf16x2(float a, float b) {
    return (uint32_t)moe_f32_to_bf16(a) | ((uint32_t)moe_f32_to_bf16(b) << 16);
}

__device__ __forceinline__ int moe_lane_id() { return (int)(threadIdx.x & (MOE_WAVE - 1)); }

// Wave-wide sum of an int.
__device__ __forceinline__ int moe_wave_sum_i32(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
    return v;
}

__device__ __forceinline__ float moe_wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, MOE_WAVE);
    return v;
}

// Local index of global expert e in { begin + j*stride : j < E_loc }, or -1.
__device__ __forceinline__ int moe_local_index(int e, int begin, int stride, int E_loc) {
    int d = e - begin;
    if (d < 0) return -1;
    int l = d / stride;
    if (l * stride != d || l >= E_loc) return -1;
    return l;
}
