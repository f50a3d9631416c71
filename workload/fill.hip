// Device side of the seeded input generator in workload/gen.py (same definition, bit for
// bit): element e of stream s under seed is word e % 4 of Philox4x32-10 with counter
// (e/4 lo, e/4 hi, s, 0) and key (seed lo, seed hi); a normal variate is the integer
// Irwin-Hall k = b0 + b1 + b2 + c - 1535 (10-bit b's) of that word times fp32(std/512).  Holds no model
// arithmetic.  Used to fill large synthetic inputs (KV caches, tables) in device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
        const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

__device__ __forceinline__ uint32_t word_at(uint64_t seed, uint32_t stream, uint64_t e) {
    const uint64_t b = e >> 2;
    uint32_t c[4] = {(uint32_t)b, (uint32_t)(b >> 32), stream, 0u};
    philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const int j = (int)(e & 3);
    return j == 0 ? c[0] : j == 1 ? c[1] : j == 2 ? c[2] : c[3];
}

__device__ __forceinline__ float normal_at(uint64_t seed, uint32_t stream, uint64_t e, float scale) {
    const uint32_t w = word_at(seed, stream, e);
    const int k = (int)(w & 1023u) + (int)((w >> 10) & 1023u) + (int)((w >> 20) & 1023u) +
                  (int)((w >> 30) & 1u) - 1535;
    return __fmul_rn((float)k, scale);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void fill_normal_kernel(void *dst, int64_t n, uint64_t seed, uint32_t stream, uint64_t start,
                                   float scale, int bf16) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float v = normal_at(seed, stream, start + (uint64_t)i, scale);
        if (bf16) reinterpret_cast<uint16_t *>(dst)[i] = bf16_rne(v);
        else reinterpret_cast<float *>(dst)[i] = v;
    }
}

// pool_layer [n_pages][2][hkv][page][hd]; page_owner[p] = b * max_pages + j (or -1)
__global__ void fill_kv_kernel(void *pool, int64_t n, int hkv, int page, int hd,
                               const int32_t *page_owner, int max_pages, const int32_t *lengths,
                               int64_t pos_stride, uint64_t seed, uint32_t stream_k, uint32_t stream_v,
                               float scale, int bf16) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t t = i;
        const int d = (int)(t % hd); t /= hd;
        const int slot = (int)(t % page); t /= page;
        const int h = (int)(t % hkv); t /= hkv;
        const int kv = (int)(t % 2); t /= 2;
        const int pg = (int)t;
        const int owner = page_owner[pg];
        float v = 0.f;
        if (owner >= 0) {
            const int b = owner / max_pages, j = owner % max_pages;
            const int64_t p = (int64_t)j * page + slot;
            if (p < lengths[b]) {
                const uint64_t e = (uint64_t)(((b * pos_stride + p) * hkv + h) * hd + d);
                v = normal_at(seed, kv ? stream_v : stream_k, e, scale);
            }
        }
        if (bf16) reinterpret_cast<uint16_t *>(pool)[i] = bf16_rne(v);
        else reinterpret_cast<float *>(pool)[i] = v;
    }
}

// Plain 16-byte-per-thread copy: the reference kernel of known traffic against which the
// hardware byte counters (FETCH_SIZE, WRITE_SIZE) are scaled.
__global__ void copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

int grid_for(int64_t n) {
    int64_t g = (n + 255) / 256;
    return (int)(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int wl_fill_normal(void *dst, int64_t n, uint64_t seed,
                                                                     uint32_t stream, uint64_t start,
                                                                     float scale, int bf16, void *hip_stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)hip_stream, dst, n,
                       seed, stream, start, scale, bf16);
    return hipPeekAtLastError() == hipSuccess ? 0 : -1;
}

extern "C" __attribute__((visibility("default"))) int wl_fill_kv(void *pool_layer, int n_pages, int hkv,
                                                                 int page, int hd, const int32_t *page_owner,
                                                                 int max_pages, const int32_t *lengths,
                                                                 int64_t pos_stride, uint64_t seed,
                                                                 uint32_t stream_k, uint32_t stream_v,
                                                                 float scale, int bf16, void *hip_stream) {
    const int64_t n = (int64_t)n_pages * 2 * hkv * page * hd;
    if (n <= 0) return 0;
    hipLaunchKernelGGL(fill_kv_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)hip_stream, pool_layer,
                       n, hkv, page, hd, page_owner, max_pages, lengths, pos_stride, seed, stream_k,
                       stream_v, scale, bf16);
    return hipPeekAtLastError() == hipSuccess ? 0 : -1;
}

// Copies `bytes` (a multiple of 16) from src to dst, both device buffers of at least that size.
extern "C" __attribute__((visibility("default"))) int wl_copy(const void *src, void *dst, int64_t bytes,
                                                              void *hip_stream) {
    if (bytes <= 0 || bytes % 16) return bytes == 0 ? 0 : -1;
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n16)), dim3(256), 0, (hipStream_t)hip_stream,
                       (const uint4 *)src, (uint4 *)dst, n16);
    return hipPeekAtLastError() == hipSuccess ? 0 : -1;
}
