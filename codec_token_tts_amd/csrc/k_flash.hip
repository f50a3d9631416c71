// K6: bidirectional attention of the MaskGIT pass (OmniVoice ARCHITECTURE, "MaskGIT
// decoder": every step is a full prefill with fully bidirectional attention, no KV
// cache across steps).  Flash-style: keys stream through LDS in blocks of 64 with an
// online softmax, so the S x S score matrix never exists.
//
// Both products run on bf16 MFMA (v_mfma_f32_16x16x32_bf16) in transposed form so
// that a lane's accumulators always belong to one query (column lane % 16):
//   S^T (16 keys x 16 queries) = K (16 x 128) * Q^T (128 x 16)
//   O^T (16 dims x 16 queries) = V^T (16 x 64) * P^T (64 x 16)
// The softmax statistics of a query are then lane-local up to a reduction over the 4
// lanes sharing it, and P^T feeds the second product straight from registers: the
// contraction runs over the 32 keys of a step in the order the lane already holds
// them (keys 4g..4g+3 and 16+4g..16+4g+3 of the step for lane group g), with V^T read
// from LDS in that same key order.  V is stored transposed by K4 ([Hkv][128][s_pad]),
// so each V^T row segment is a contiguous LDS read.
//
// Block = 4 waves = (4/GROUP) query tiles of 16 x GROUP query heads sharing one KV
// head, so the K and V tiles in LDS serve every head of the GQA group.  Scores are
// pre-scaled by log2(e)/sqrt(128) and exponentiated with exp2.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ttsbb {

constexpr int FB = 64;          // keys per block
constexpr int LDKF = 128 + 8;   // K tile row stride (elements)
constexpr int LDVF = FB + 8;    // V^T tile row stride (elements)

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

template <int GROUP>
__global__ __launch_bounds__(256) void flash_kernel(FlashArgs a) {
    constexpr int QT = 4 / GROUP;  // query tiles per block
    __shared__ __attribute__((aligned(16))) bf16_t sK[2][FB * LDKF];
    __shared__ __attribute__((aligned(16))) bf16_t sV[2][128 * LDVF];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int qt = wave / GROUP, jh = wave % GROUP;
    const int hk = blockIdx.y;
    const int head = hk * GROUP + jh;
    const int q0 = blockIdx.x * 16 * QT + qt * 16;
    const int fr = lane & 15, g = lane >> 4, fk = g * 8;
    const int ldq = a.H * 128;

    // Q^T operand: lane -> query q0 + fr, dims ks*32 + fk .. +7
    bf16x8_t qf[4];
    {
        const int qi = q0 + fr;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (qi < a.S)
                qf[ks] = *reinterpret_cast<const bf16x8_t *>(a.q + (int64_t)qi * ldq + head * 128 + ks * 32 + fk);
            else
                qf[ks] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    const bf16_t *kg = a.k + (int64_t)hk * a.s_pad * 128;
    const bf16_t *vg = a.vt + (int64_t)hk * 128 * a.s_pad;
    u32x4_t rk[4], rv[4];
    auto gload = [&](int kb0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ch = tid + 256 * c;
            rk[c] = *reinterpret_cast<const u32x4_t *>(kg + (int64_t)(kb0 + (ch >> 4)) * 128 + (ch & 15) * 8);
            rv[c] = *reinterpret_cast<const u32x4_t *>(vg + (int64_t)(ch >> 3) * a.s_pad + kb0 + (ch & 7) * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ch = tid + 256 * c;
            *reinterpret_cast<u32x4_t *>(&sK[buf][(ch >> 4) * LDKF + (ch & 15) * 8]) = rk[c];
            *reinterpret_cast<u32x4_t *>(&sV[buf][(ch >> 3) * LDVF + (ch & 7) * 8]) = rv[c];
        }
    };

    f32x4_t o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int NB = a.s_pad / FB;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kb = 0; kb < NB; ++kb) {
        const int buf = kb & 1;
        gload(min(kb + 1, NB - 1) * FB);  // unconditional (clamped) so the waits stay counted

        f32x4_t s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8_t ka = *reinterpret_cast<const bf16x8_t *>(&sK[buf][(kt * 16 + fr) * LDKF + ks * 32 + fk]);
                s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ks], s[kt], 0, 0, 0);
            }
        }
        // scale, mask keys past S, block max of this lane's query
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kb * FB + kt * 16 + g * 4 + r;
                const float v = key < a.S ? s[kt][r] * a.scale_log2 : -INFINITY;
                s[kt][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
        const float m_new = fmaxf(m_run, mx);  // finite: every block holds a key < S
        const float sc = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= sc;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d] *= sc;

        bf16x8_t pb[2];
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = exp2f(s[2 * ks2 + h2][r] - m_new);
                    l_run += p;
                    pb[ks2][h2 * 4 + r] = (__bf16)p;
                }
        }
#pragma unroll
        for (int d = 0; d < 8; ++d) {
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                const bf16_t *vrow = &sV[buf][(d * 16 + fr) * LDVF + ks2 * 32 + g * 4];
                const bf16x4_t lo = *reinterpret_cast<const bf16x4_t *>(vrow);
                const bf16x4_t hi = *reinterpret_cast<const bf16x4_t *>(vrow + 16);
                const bf16x8_t va = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ks2], o[d], 0, 0, 0);
            }
        }
        if (kb + 1 < NB) sstore(buf ^ 1);
        __syncthreads();
    }

    l_run += __shfl_xor(l_run, 16, WAVE);
    l_run += __shfl_xor(l_run, 32, WAVE);
    const float inv = 1.0f / l_run;
    const int qi = q0 + fr;
    if (qi < a.S) {
        bf16_t *out = a.out + (int64_t)qi * ldq + head * 128 + g * 4;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            uint2 w;
            w.x = (uint32_t)f32_to_bf16(o[d][0] * inv) | ((uint32_t)f32_to_bf16(o[d][1] * inv) << 16);
            w.y = (uint32_t)f32_to_bf16(o[d][2] * inv) | ((uint32_t)f32_to_bf16(o[d][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(out + d * 16) = w;
        }
    }
}

void launch_flash_attn(const FlashArgs &a, hipStream_t s) {
    if (a.S <= 0) return;
    const int group = a.H / a.Hkv;
    const int qpb = 16 * (4 / group);
    dim3 grid((a.S + qpb - 1) / qpb, a.Hkv);
    if (group == 2) hipLaunchKernelGGL(flash_kernel<2>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(flash_kernel<1>, grid, dim3(256), 0, s, a);
}

}  // namespace ttsbb
