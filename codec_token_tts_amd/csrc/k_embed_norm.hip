// K1 gather-sum codebook embedding, K2 RMSNorm, and small helpers.
//
// K1 (OmniVoice ARCHITECTURE, "Qwen3 0.6B backbone with custom IO": audio rows are
// rows k*1025 + code of the flattened table summed over the codebooks, text rows take
// the text table; ncnn Qwen3-TTS port, "模型结构拆解": the 16 codebook embeddings of a
// frame are summed).  HBM-bound gather: one 256-thread block per output row, each
// thread owns 4 consecutive columns (8-byte bf16 or 16-byte fp32 loads, coalesced per
// table row).  The sum is accumulated in double and rounded once, so the result is the
// correctly rounded fp32 value of the exact sum.
//
// K2 (same page, "GGUF layout": input/post-attention layernorm, llm.norm, eps 1e-6):
// y = x / sqrt(mean(x^2) + eps) * g, one block per row, fp32 statistics, output in
// the operand dtype of the next matrix product.
#include "common.h"
#include "kernels.h"

namespace ttsbb {

template <typename T>
__device__ __forceinline__ void load4(const T *p, float v[4]);
template <>
__device__ __forceinline__ void load4<float>(const float *p, float v[4]) {
    float4 t = *reinterpret_cast<const float4 *>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t *p, float v[4]) {
    uint2 t = *reinterpret_cast<const uint2 *>(p);
    v[0] = __uint_as_float(t.x << 16);
    v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16);
    v[3] = __uint_as_float(t.y & 0xFFFF0000u);
}

template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
    const int r = blockIdx.x;
    const T *tables = reinterpret_cast<const T *>(a.tables);
    for (int c0 = threadIdx.x * 4; c0 < a.hidden; c0 += 256 * 4) {
        const bool text = a.is_text ? (a.is_text[r] != 0) : (r < a.text_prefix);
        float outv[4];
        if (text) {
            int id = a.text_ids[r];
            if (id < 0 || id >= a.text_vocab) {
                if (threadIdx.x == 0 && c0 == 0) raise_flag(a.flag, FLAG_TEXT_ID);
                id = 0;
            }
            load4<T>(reinterpret_cast<const T *>(a.text_table) + (int64_t)id * a.hidden + c0, outv);
        } else {
            // EB codebooks per round: their codes in one round of loads, then their table
            // rows in one more (indices clamped, so every load is unconditional), then the
            // sum in codebook order -- two dependent rounds per EB codebooks, not two per
            // codebook
            constexpr int EB = 16;
            double acc[4] = {0.0, 0.0, 0.0, 0.0};
            bool bad = false;
            const int32_t *crow = a.codes + (int64_t)(r - a.audio_row0) * a.code_row_stride;
            for (int k0 = 0; k0 < a.n_cb; k0 += EB) {
                int code[EB];
#pragma unroll
                for (int u = 0; u < EB; ++u) code[u] = crow[(int64_t)min(k0 + u, a.n_cb - 1) * a.code_cb_stride];
                float v[EB][4];
#pragma unroll
                for (int u = 0; u < EB; ++u) {
                    const int k = min(k0 + u, a.n_cb - 1);
                    const bool ok = code[u] >= 0 && code[u] < a.cb_vocab;
                    bad |= !ok;
                    load4<T>(tables + ((int64_t)k * a.cb_vocab + (ok ? code[u] : 0)) * a.hidden + c0, v[u]);
                }
#pragma unroll
                for (int u = 0; u < EB; ++u) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = k0 + u < a.n_cb ? acc[i] + (double)v[u][i] : acc[i];
                }
            }
            if (bad && threadIdx.x == 0 && c0 == 0) raise_flag(a.flag, FLAG_CODE);
#pragma unroll
            for (int i = 0; i < 4; ++i) outv[i] = (float)acc[i];
        }
        *reinterpret_cast<float4 *>(a.out + (int64_t)r * a.hidden + c0) =
            make_float4(outv[0], outv[1], outv[2], outv[3]);
    }
}

void launch_embed(const EmbedArgs &a, DType dt, hipStream_t s) {
    if (a.n_rows <= 0) return;
    if (dt == DT_BF16)
        hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(a.n_rows), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(embed_kernel<float>, dim3(a.n_rows), dim3(256), 0, s, a);
}

template <typename TO, int NP>
__global__ __launch_bounds__(256) void rmsnorm_kernel(float *x, int ldx, int hidden, const float *g, float eps,
                                                      TO *out, const float *pend, int64_t pend_ld,
                                                      int64_t pend_stride, int out_mt) {
    constexpr int MAXC = 4;  // float4 columns per thread held in registers (hidden <= 4096)
    __shared__ float red[4];
    const int r = blockIdx.x;
    float *xr = x + (int64_t)r * ldx;
    // every load of the row (residual, deferred partials, gains) is issued up front
    float4 v[MAXC], gg[MAXC], pp[NP > 0 ? NP : 1][MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x * 4 + i * 1024;
        if (c >= hidden) continue;
        v[i] = *reinterpret_cast<const float4 *>(xr + c);
#pragma unroll
        for (int z = 0; z < NP; ++z)
            pp[z][i] = *reinterpret_cast<const float4 *>(pend + z * pend_stride + (int64_t)r * pend_ld + c);
        if (g != nullptr) gg[i] = *reinterpret_cast<const float4 *>(g + c);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x * 4 + i * 1024;
        if (c >= hidden) continue;
        if (NP > 0) {  // deferred residual update, in split order
#pragma unroll
            for (int z = 0; z < NP; ++z) {
                v[i].x += pp[z][i].x;
                v[i].y += pp[z][i].y;
                v[i].z += pp[z][i].z;
                v[i].w += pp[z][i].w;
            }
            *reinterpret_cast<float4 *>(xr + c) = v[i];
        }
        ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    }
    if (g == nullptr) return;
    ss = block_sum_256(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)hidden + eps);
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x * 4 + i * 1024;
        if (c >= hidden) continue;
        // fragment-major: the 4 columns c .. c + 3 stay contiguous (c % 4 == 0)
        TO *o = out + (out_mt > 0 ? frag_index(r, c, out_mt) : (int64_t)r * hidden + c);
        o[0] = from_f32<TO>(v[i].x * inv * gg[i].x);
        o[1] = from_f32<TO>(v[i].y * inv * gg[i].y);
        o[2] = from_f32<TO>(v[i].z * inv * gg[i].z);
        o[3] = from_f32<TO>(v[i].w * inv * gg[i].w);
    }
}

template <typename TO>
static void launch_rmsnorm_t(float *x, int ldx, int rows, int hidden, const float *gain, float eps, TO *out,
                             hipStream_t s, const float *pend, int n_pend, int64_t pend_ld, int64_t pend_stride,
                             int out_mt) {
    const dim3 grid(rows), block(256);
    switch (n_pend) {
#define TTSBB_NORM_CASE(NP)                                                                                    \
    case NP:                                                                                                   \
        hipLaunchKernelGGL((rmsnorm_kernel<TO, NP>), grid, block, 0, s, x, ldx, hidden, gain, eps, out, pend, \
                           pend_ld, pend_stride, out_mt);                                                      \
        break;
        TTSBB_NORM_CASE(0)
        TTSBB_NORM_CASE(1)
        TTSBB_NORM_CASE(2)
        TTSBB_NORM_CASE(3)
        TTSBB_NORM_CASE(4)
        TTSBB_NORM_CASE(5)
        TTSBB_NORM_CASE(6)
        TTSBB_NORM_CASE(7)
        TTSBB_NORM_CASE(8)
#undef TTSBB_NORM_CASE
    }
}

// n_pend <= 8 partial buffers, hidden <= 4096 and a multiple of 4 (checked by the caller)
void launch_rmsnorm(float *x, int ldx, int rows, int hidden, const float *gain, float eps, void *out,
                    DType out_dt, hipStream_t s, const float *pend, int n_pend, int64_t pend_ld,
                    int64_t pend_stride, int out_mt) {
    if (rows <= 0) return;
    if (out_dt == DT_BF16)
        launch_rmsnorm_t(x, ldx, rows, hidden, gain, eps, reinterpret_cast<bf16_t *>(out), s, pend, n_pend, pend_ld,
                         pend_stride, out_mt);
    else
        launch_rmsnorm_t(x, ldx, rows, hidden, gain, eps, reinterpret_cast<float *>(out), s, pend, n_pend, pend_ld,
                         pend_stride, 0);
}

__global__ void increment_kernel(int32_t *v, int n, int delta) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) v[i] += delta;
}

void launch_increment(int32_t *v, int n, hipStream_t s, int delta) {
    if (n <= 0) return;
    hipLaunchKernelGGL(increment_kernel, dim3((n + 255) / 256), dim3(256), 0, s, v, n, delta);
}

template <typename T>
__global__ void tap_copy_kernel(const T *src, int64_t s0, int64_t s1, int64_t s2, int d0, int d1,
                                int d2, float *dst) {
    int64_t total = (int64_t)d0 * d1 * d2;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t i2 = i % d2, t = i / d2;
        int64_t i1 = t % d1, i0 = t / d1;
        dst[i] = to_f32<T>(src[i0 * s0 + i1 * s1 + i2 * s2]);
    }
}

void launch_tap_copy(const void *src, DType dt, int64_t s0, int64_t s1, int64_t s2, int d0,
                     int d1, int d2, float *dst, hipStream_t s) {
    int64_t total = (int64_t)d0 * d1 * d2;
    if (total <= 0) return;
    int blocks = (int)((total + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    if (dt == DT_BF16)
        hipLaunchKernelGGL(tap_copy_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s,
                           reinterpret_cast<const bf16_t *>(src), s0, s1, s2, d0, d1, d2, dst);
    else
        hipLaunchKernelGGL(tap_copy_kernel<float>, dim3(blocks), dim3(256), 0, s,
                           reinterpret_cast<const float *>(src), s0, s1, s2, d0, d1, d2, dst);
}

}  // namespace ttsbb
