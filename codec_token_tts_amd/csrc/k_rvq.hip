// Codec RVQ decode (OmniVoice ARCHITECTURE, "Audio tokenizer pipeline", decode path:
// e_k = codebook[k].embed[codes[k]], p_k = e_k project_out[k].W^T + bias[k], summed over
// the codebooks; ncnn Qwen3-TTS port, "Codec Decoder的切分": the lookup and projections
// run per frame before the codec body).  fp32 throughout, like the codec's quantizer.
//
//   out[t][n] = sum_k ( sum_d embed[k][codes[k][t]][d] * W[k][n][d] + b[k][n] )
//
// The whole decode is one product over K = n_q * dim: out = A B^T + sum_k b_k with
// A[t][k*dim + d] = embed[k][codes[k][t]][d] (the gather) and B[n][k*dim + d] = W[k][n][d].
//
// rvq_mfma_kernel (dim % 8 == 0, dim <= 64, n_q <= 32, 16-byte aligned tables): fp32 matrix cores
// (v_mfma_f32_32x32x2_f32).  A block of eight waves owns a 64-frame x 64-output tile: two
// groups of four waves (2 x 2 sub-tiles of 32 x 32) take alternate codebooks.  The tile's
// codes are read, validated and clamped into LDS first.  For each
// codebook a group gathers the tile's 64 embedding rows and 64 projection rows into an LDS
// stage with row-coalesced 16-byte loads (a lane walking a row of its own would touch 64
// lines per load instruction and thrash L1), the next codebook's loads in flight during
// this one's products; in each MFMA the two half-waves take the same offset in the two
// halves of the codebook's dimensions.  Group 1's tile is added onto group 0's through
// LDS, then the biases in codebook order.
//
// rvq_decode_kernel (any shape): a block computes a tile of 32 frames x 128 outputs with
// vector FMAs (256 threads, 4 x 4 accumulators each).  For every codebook and every
// 64-wide slice of the codebook dimension it gathers the tile's 32 embedding rows and the
// 128 projection rows into LDS (W stored transposed so a thread's four outputs are one
// 16-byte read), then runs the FMAs; the sum over codebooks and the bias stay in
// registers, in codebook order.
#include <hip/hip_ext.h>

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

typedef __attribute__((ext_vector_type(16))) float rvq_f32x16;

constexpr int RVQ_G = 2;         // codebook groups: group g takes codebooks g, g + 2, ...
constexpr int RVQ_BT = 64;       // block tile: 64 frames x 64 outputs (2 x 2 waves per group)
constexpr int RVQ_MAXD = 64;     // codebook dimension the LDS stages hold
constexpr int RVQ_MAXQ = 32;     // codebooks whose codes the tile keeps in LDS
constexpr int RVQ_LD = RVQ_MAXD + 4;  // LDS row stride (floats): conflict-free 16-byte reads
constexpr int RVQ_ROWS = 2 * RVQ_BT;  // a stage: 64 embedding rows, then 64 projection rows
constexpr int RVQ_PER = RVQ_ROWS * (RVQ_MAXD / 4) / 256;  // 16-byte loads per thread per stage

// Codebook k's rows of the block's tile into registers, row-coalesced (c4n consecutive
// threads per row): embedding rows of the tile's frames (clamped past the last frame),
// then projection rows of its outputs.  Chunk indices past the stage are clamped to its
// last chunk (loaded and stored again with the same value), so every load is unconditional.
__device__ __forceinline__ void rvq_fetch(const RvqArgs &a, const int *codes_t, int k, int gt, int n0, int c4n,
                                          f32x4_t (&r)[RVQ_PER]) {
#pragma unroll
    for (int j = 0; j < RVQ_PER; ++j) {
        const int idx = min(gt + 256 * j, RVQ_ROWS * c4n - 1);
        const int row = idx / c4n, c = idx % c4n;
        const int code = codes_t[k * RVQ_BT + (row & (RVQ_BT - 1))];  // validated, clamped
        const int n = min(n0 + (row & (RVQ_BT - 1)), a.out_dim - 1);
        const float *src = row < RVQ_BT ? a.embed + ((int64_t)k * a.cb_size + code) * a.dim + c * 4
                                        : a.proj_w + ((int64_t)k * a.out_dim + n) * a.dim + c * 4;
        r[j] = *reinterpret_cast<const f32x4_t *>(src);
    }
}

__device__ __forceinline__ void rvq_put(float *st, int gt, int c4n, const f32x4_t (&r)[RVQ_PER]) {
#pragma unroll
    for (int j = 0; j < RVQ_PER; ++j) {
        const int idx = min(gt + 256 * j, RVQ_ROWS * c4n - 1);
        *reinterpret_cast<f32x4_t *>(st + (idx / c4n) * RVQ_LD + (idx % c4n) * 4) = r[j];
    }
}

__global__ __launch_bounds__(512) void rvq_mfma_kernel(RvqArgs a) {
    __shared__ __attribute__((aligned(16))) float lds[RVQ_G][2][RVQ_ROWS * RVQ_LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = wave >> 2, wm = (wave >> 1) & 1, wn = wave & 1;
    const int gt = tid & 255;  // thread index inside the group
    const int tiles_n = (a.out_dim + RVQ_BT - 1) / RVQ_BT;
    const int t0 = (blockIdx.x / tiles_n) * RVQ_BT, n0 = (blockIdx.x % tiles_n) * RVQ_BT;
    const int c4n = a.dim / 4;  // 16-byte chunks per row
    // the tile's codes, validated and clamped once, so that a codebook's fetch is a single
    // round of loads (the code no longer precedes the embedding row's address)
    __shared__ int codes_t[RVQ_MAXQ * RVQ_BT];
    for (int i = tid; i < a.n_q * RVQ_BT; i += 512) {
        const int k = i / RVQ_BT, t_row = t0 + i % RVQ_BT;
        int code = a.codes[(int64_t)k * a.n_frames + min(t_row, a.n_frames - 1)];
        if (code < 0 || code >= a.cb_size) {
            if (t_row < a.n_frames) raise_flag(a.flag, FLAG_CODE);
            code = code < 0 ? 0 : a.cb_size - 1;
        }
        codes_t[i] = code;
    }
    __syncthreads();

    // MFMA operands: lane l holds rows wm*32 + l%32 (frames) and 64 + wn*32 + l%32 (outputs);
    // the half-waves take the same offset in the two halves of the codebook's dimensions
    const int h = lane >> 5, hd = a.dim / 2, nv = hd / 4;
    const int ar = (wm * 32 + (lane & 31)) * RVQ_LD + h * hd;
    const int br = (RVQ_BT + wn * 32 + (lane & 31)) * RVQ_LD + h * hd;
    rvq_f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    f32x4_t rg[RVQ_PER];  // native vectors: arrays of HIP's float4 class stay in scratch
    const int iters = (a.n_q + RVQ_G - 1) / RVQ_G;
    if (g < a.n_q) rvq_fetch(a, codes_t, g, gt, n0, c4n, rg);
    for (int it = 0, k = g; it < iters; ++it, k += RVQ_G) {
        float *st = lds[g][it & 1];
        if (k < a.n_q) rvq_put(st, gt, c4n, rg);
        __syncthreads();  // the stage is written; the one written next was last read before it
        if (k + RVQ_G < a.n_q) rvq_fetch(a, codes_t, k + RVQ_G, gt, n0, c4n, rg);  // in flight during the products
        if (k < a.n_q) {
#pragma unroll
            for (int v = 0; v < RVQ_MAXD / 8; ++v) {
                if (v >= nv) break;
                const f32x4_t av = *reinterpret_cast<const f32x4_t *>(st + ar + 4 * v);
                const f32x4_t bv = *reinterpret_cast<const f32x4_t *>(st + br + 4 * v);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[e], acc, 0, 0, 0);
            }
        }
    }
    // group 1's tile onto group 0's (through the idle stages), then the biases
    __syncthreads();
    float *red = &lds[0][0][0] + (wave & 3) * 16 * 64;
    if (g == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[r * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (g != 0) return;
    const int col = n0 + wn * 32 + (lane & 31);
    if (col >= a.out_dim) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += red[r * 64 + lane];
    float bias = 0.f;
    for (int k = 0; k < a.n_q; ++k) bias += a.proj_b[(int64_t)k * a.out_dim + col];
    // lane holds column col for rows (r / 4) * 8 + (lane / 32) * 4 + r % 4 of its 32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = t0 + wm * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        if (row < a.n_frames) a.out[(int64_t)row * a.out_dim + col] = acc[r] + bias;
    }
}

void launch_rvq_decode(const RvqArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.n_frames <= 0 || a.out_dim <= 0) return;
    auto go = [&](auto kernel, dim3 grid) {
        if (ev0 || ev1) hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, s, ev0, ev1, 0, a);
        else hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, a);  // plain launch (graph capture)
    };
    const bool aligned = ((reinterpret_cast<uintptr_t>(a.embed) | reinterpret_cast<uintptr_t>(a.proj_w)) & 15) == 0;
    if (a.dim % 8 == 0 && a.dim <= RVQ_MAXD && a.n_q <= RVQ_MAXQ && aligned) {
        const dim3 grid(((a.n_frames + RVQ_BT - 1) / RVQ_BT) * ((a.out_dim + RVQ_BT - 1) / RVQ_BT));
        if (ev0 || ev1) hipExtLaunchKernelGGL(rvq_mfma_kernel, grid, dim3(512), 0, s, ev0, ev1, 0, a);
        else hipLaunchKernelGGL(rvq_mfma_kernel, grid, dim3(512), 0, s, a);
        return;
    }
    go(rvq_decode_kernel, dim3((a.n_frames + RVQ_TF - 1) / RVQ_TF, (a.out_dim + RVQ_TN - 1) / RVQ_TN));
}

}  // namespace ttsbb
