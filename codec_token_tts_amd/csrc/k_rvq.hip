// Codec RVQ decode (OmniVoice ARCHITECTURE, "Audio tokenizer pipeline", decode path:
// e_k = codebook[k].embed[codes[k]], p_k = e_k project_out[k].W^T + bias[k], summed over
// the codebooks; ncnn Qwen3-TTS port, "Codec Decoder的切分": the lookup and projections
// run per frame before the codec body).  fp32 throughout, like the codec's quantizer.
//
//   out[t][n] = sum_k ( sum_d embed[k][codes[k][t]][d] * W[k][n][d] + b[k][n] )
//
// A block computes a tile of 32 frames x 128 outputs (256 threads, 4 x 4 accumulators
// each).  For every codebook and every 64-wide slice of the codebook dimension it
// gathers the tile's 32 embedding rows and the 128 projection rows into LDS (W stored
// transposed so a thread's four outputs are one 16-byte read), then runs the FMAs; the
// sum over codebooks and the bias stay in registers, in codebook order.
#include "common.h"
#include "kernels.h"

namespace ttsbb {

constexpr int RVQ_TF = 32, RVQ_TN = 128, RVQ_TD = 64;

__global__ __launch_bounds__(256) void rvq_decode_kernel(RvqArgs a) {
    __shared__ float sE[RVQ_TF][RVQ_TD + 1];
    __shared__ __attribute__((aligned(16))) float sWt[RVQ_TD][RVQ_TN + 4];
    const int tid = threadIdx.x, tx = tid & 31, ty = tid >> 5;  // outputs tx*4.., frames ty*4..
    const int t0 = blockIdx.x * RVQ_TF, n0 = blockIdx.y * RVQ_TN;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k = 0; k < a.n_q; ++k) {
        const float *emb = a.embed + (int64_t)k * a.cb_size * a.dim;
        const float *w = a.proj_w + (int64_t)k * a.out_dim * a.dim;
        for (int d0 = 0; d0 < a.dim; d0 += RVQ_TD) {
            const int dn = min(RVQ_TD, a.dim - d0);
            __syncthreads();  // the previous slice's reads are done
            for (int i = tid; i < RVQ_TF * RVQ_TD; i += 256) {
                const int f = i / RVQ_TD, d = i % RVQ_TD, t = t0 + f;
                float v = 0.f;
                if (t < a.n_frames && d < dn) {
                    int c = a.codes[(int64_t)k * a.n_frames + t];
                    if (c < 0 || c >= a.cb_size) {
                        if (d == 0) raise_flag(a.flag, FLAG_CODE);
                        c = c < 0 ? 0 : a.cb_size - 1;
                    }
                    v = emb[(int64_t)c * a.dim + d0 + d];
                }
                sE[f][d] = v;
            }
            for (int i = tid; i < RVQ_TN * RVQ_TD; i += 256) {
                const int n = i / RVQ_TD, d = i % RVQ_TD;
                sWt[d][n] = (n0 + n < a.out_dim && d < dn) ? w[(int64_t)(n0 + n) * a.dim + d0 + d] : 0.f;
            }
            __syncthreads();
            for (int d = 0; d < dn; ++d) {
                const float4 wv = *reinterpret_cast<const float4 *>(&sWt[d][tx * 4]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = sE[ty * 4 + i][d];
                    acc[i][0] = fmaf(e, wv.x, acc[i][0]);
                    acc[i][1] = fmaf(e, wv.y, acc[i][1]);
                    acc[i][2] = fmaf(e, wv.z, acc[i][2]);
                    acc[i][3] = fmaf(e, wv.w, acc[i][3]);
                }
            }
        }
        // this codebook's bias, added after its product like p_k = e_k W_k^T + b_k
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            const float bk = n < a.out_dim ? a.proj_b[(int64_t)k * a.out_dim + n] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][j] += bk;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= a.n_frames) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n < a.out_dim) a.out[(int64_t)t * a.out_dim + n] = acc[i][j];
        }
    }
}

void launch_rvq_decode(const RvqArgs &a, hipStream_t s) {
    if (a.n_frames <= 0 || a.out_dim <= 0) return;
    const dim3 grid((a.n_frames + RVQ_TF - 1) / RVQ_TF, (a.out_dim + RVQ_TN - 1) / RVQ_TN);
    hipLaunchKernelGGL(rvq_decode_kernel, grid, dim3(256), 0, s, a);
}

}  // namespace ttsbb
