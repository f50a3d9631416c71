// Internal helpers shared by the ttsbb HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttsbb {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
// Native 16-byte vector: stays an SSA value (HIP's uint4 class is copied through memory).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (bf16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Sum over aligned groups of `G` lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// (value, index) argmax step: larger value wins, equal values keep the lower index.
__device__ __forceinline__ void argmax_merge(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o, WAVE);
        int i2 = __shfl_xor(i, o, WAVE);
        argmax_merge(v, i, v2, i2);
    }
}

// Block-wide sum for blockDim.x == 256 (4 waves); `red` is __shared__ float[4].
__device__ __forceinline__ float block_sum_256(float v, float *red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return t;
}

__device__ __forceinline__ void raise_flag(int *flag, int code) {
    if (flag) atomicOr(flag, code);
}

}  // namespace ttsbb
