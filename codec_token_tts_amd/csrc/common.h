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


// Sum over aligned groups of `G` lanes (G a power of two <= 64).
// Cross-lane move inside a 16-lane row through DPP (a VALU operand modifier, no LDS
// round trip).  Every control used here reads a lane of the same row, so no lane is out
// of range.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- 7 - i inside each 8-lane half row
constexpr int DPP_MIRROR = 0x140;      // lane i <- 15 - i inside each 16-lane row
constexpr int DPP_ROR8 = 0x128;        // lane i <- (i + 8) mod 16 inside each 16-lane row

// Sum over aligned groups of G lanes; every lane of a group ends with the same value.
// Up to 16 lanes the steps are DPP (pair, quad, half row, row); wider groups finish
// with butterfly shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
    if constexpr (G >= 2) v += dpp_f<DPP_XOR1>(v);
    if constexpr (G >= 4) v += dpp_f<DPP_XOR2>(v);
    if constexpr (G >= 8) v += dpp_f<DPP_HALF_MIRROR>(v);
    if constexpr (G >= 16) v += dpp_f<DPP_MIRROR>(v);
#pragma unroll
    for (int o = 16; o < G; o <<= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Whole-wave sum / maximum (all 64 lanes active): DPP inside each 16-lane row, then the
// four row results are read into scalar registers and combined, so no step goes through
// LDS.  Every lane receives the result.
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<16>(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
    v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
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

// Fragment-major layout of a bf16 activation operand of at most 64 rows, as the skinny
// decode GEMM loads it: for each 32-wide K step kc and 16-row tile rt (of mt tiles), one
// contiguous 1 KB block whose 16-byte chunk l holds row rt * 16 + l % 16, elements
// kc * 32 + 8 (l / 16) .. +7.  A wave then reads each operand fragment as one contiguous
// 1 KB load instead of 16 row segments.  Element index of (row r, column k):
__device__ __forceinline__ int64_t frag_index(int r, int k, int mt) {
    return ((int64_t)(k >> 5) * mt + (r >> 4)) * 512 + (((k >> 3) & 3) * 16 + (r & 15)) * 8 + (k & 7);
}

__device__ __forceinline__ void raise_flag(int *flag, int code) {
    if (flag) atomicOr(flag, code);
}

}  // namespace ttsbb
