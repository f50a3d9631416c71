// K7: greedy choice per head group; K8: MaskGIT scoring; K9: top-n unmasking.
//
// K7 (ncnn Qwen3-TTS port, "文本前端与生成循环": greedy decoding for strict numerical
// alignment): argmax over each group of classes, ties to the lowest class id.
//
// K8 (OmniVoice ARCHITECTURE, "Qwen3 0.6B backbone with custom IO": logits of the
// (8200, 1024) audio head viewed per codebook; "MaskGIT decoder": log_softmax, the mask
// class set to -inf, argmax, score = max log-prob - layer index * layer penalty, scores
// of already unmasked positions set to -inf).  One wave per (codebook, frame): the
// 1025 logits of the group are contiguous; max and argmax over non-mask classes in one
// sweep, sum of exp in a second, all in fp32.
//
// K9 (same section: topk over the flattened scores, then tokens[idx] = pred[idx]).
// The rank of element i is the number of elements that order before it (greater
// score, or equal score and lower flat index); the n elements of rank < n are the
// selection and picked[rank] = i.  Ranks are independent, so the selection is exact
// and needs no sort.  The count is split over (block of elements) x (tile of 1024
// scores staged in LDS) and summed with integer atomics, whose result does not
// depend on their order; a second pass scatters picks and updates the codes.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ttsbb {

__global__ __launch_bounds__(256) void argmax_groups_kernel(const float *logits, int rows, int ld,
                                                            int n_groups, int V, int32_t *out) {
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= rows * n_groups) return;
    const int gi = item % n_groups, r = item / n_groups;
    const float *x = logits + (int64_t)r * ld + (int64_t)gi * V;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int v = lane; v < V; v += 64) argmax_merge(best, bi, x[v], v);
    wave_argmax(best, bi);
    if (lane == 0) out[item] = bi;
}

void launch_argmax_groups(const float *logits, int rows, int ld, int n_groups, int group_vocab,
                          int32_t *out, hipStream_t s) {
    const int items = rows * n_groups;
    if (items <= 0) return;
    hipLaunchKernelGGL(argmax_groups_kernel, dim3((items + 3) / 4), dim3(256), 0, s, logits, rows, ld,
                       n_groups, group_vocab, out);
}

__global__ __launch_bounds__(256) void maskgit_scores_kernel(const float *logits, const float *logits_u,
                                                             float cfg_scale, int T, int ld, int n_cb, int V,
                                                             int mask_id, float penalty, const int32_t *codes,
                                                             int codes_ld, int32_t *pred, float *conf) {
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);  // flat index k*T + t
    if (item >= n_cb * T) return;
    const int k = item / T, t = item % T;
    const float *x = logits + (int64_t)t * ld + (int64_t)k * V;
    const float *xu = logits_u ? logits_u + (int64_t)t * ld + (int64_t)k * V : nullptr;
    // the scored logit of class v (guided when an unconditional row is given)
    auto lg = [&](int v) {
        const float c = x[v];
        return xu ? c + cfg_scale * (c - xu[v]) : c;
    };
    float mx = -INFINITY, best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int v = lane; v < V; v += 64) {
        const float xv = lg(v);
        mx = fmaxf(mx, xv);
        if (v != mask_id) argmax_merge(best, bi, xv, v);
    }
    mx = wave_max(mx);
    wave_argmax(best, bi);
    const float LOG2E = 1.4426950408889634f;
    float se = 0.f;
    for (int v = lane; v < V; v += 64) se += exp2f((lg(v) - mx) * LOG2E);
    se = wave_sum(se);
    if (lane == 0) {
        const float lse = mx + logf(se);
        pred[item] = bi;
        conf[item] = (codes[(int64_t)k * codes_ld + t] == mask_id) ? (best - lse) - (float)k * penalty : -INFINITY;
    }
}

void launch_maskgit_scores(const float *logits, const float *logits_u, float cfg_scale, int T, int ld,
                           int n_cb, int V, int mask_id, float penalty, const int32_t *codes, int codes_ld,
                           int32_t *pred, float *conf, hipStream_t s) {
    const int items = n_cb * T;
    if (items <= 0) return;
    hipLaunchKernelGGL(maskgit_scores_kernel, dim3((items + 3) / 4), dim3(256), 0, s, logits, logits_u, cfg_scale,
                       T, ld, n_cb, V, mask_id, penalty, codes, codes_ld, pred, conf);
}

// ------------------------------------------------------------------------------------
// K8 with the sampler (same page, "MaskGIT decoder": keep_top_k_ratio(log_probs, 0.1),
// gumbel_sample(temp = class_temp), score += gumbel * pos_temp; the uniforms of the
// Gumbel noise are the caller's).  One wave per (codebook, frame); the group's V log-probs
// are kept in LDS (V <= SAMPLE_MAXV).  The top-k threshold is the k-th largest log-prob,
// found by a bisection on the order-preserving integer image of the floats (counts by
// wave reductions); ties at the threshold are kept in class order (ballot prefix counts).
// Then lp' = lp / class_temp + G(u) on the kept classes (-inf elsewhere), pred = argmax
// lp' (ties: lowest id), score = max lp' - k * penalty + pos_temp * G(u_pos), with
// G(u) = -log(-log u).
// ------------------------------------------------------------------------------------
constexpr int SAMPLE_MAXV = 2048;

// order-preserving map float -> int32 (signed comparison), -inf lowest
__device__ __forceinline__ int fkey(float f) {
    const int i = __float_as_int(f);
    return i >= 0 ? i : i ^ 0x7FFFFFFF;
}

__device__ __forceinline__ float gumbel_f(float u) { return -logf(-logf(u)); }

__global__ __launch_bounds__(256) void maskgit_sample_kernel(const float *logits, const float *logits_u,
                                                             float cfg_scale, int T, int ld, int n_cb, int V,
                                                             int mask_id, float penalty, const int32_t *codes,
                                                             int codes_ld, float class_temp, float pos_temp,
                                                             int k_keep, const float *u_class, const float *u_pos,
                                                             int32_t *pred, float *conf) {
    __shared__ float lps[4][SAMPLE_MAXV];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int item = blockIdx.x * 4 + wave;  // flat index k*T + t
    if (item >= n_cb * T) return;
    const int k = item / T, t = item % T;
    const float *x = logits + (int64_t)t * ld + (int64_t)k * V;
    const float *xu = logits_u ? logits_u + (int64_t)t * ld + (int64_t)k * V : nullptr;
    float *lp = lps[wave];
    float mx = -INFINITY;
    for (int v = lane; v < V; v += 64) {
        const float c = x[v];
        const float g = xu ? c + cfg_scale * (c - xu[v]) : c;
        lp[v] = g;
        mx = fmaxf(mx, g);
    }
    mx = wave_max(mx);
    float se = 0.f;
    for (int v = lane; v < V; v += 64) se += expf(lp[v] - mx);
    se = wave_sum(se);
    const float lse = mx + logf(se);
    for (int v = lane; v < V; v += 64) lp[v] = v == mask_id ? -INFINITY : lp[v] - lse;  // own entries only

    const float *u = u_class + (int64_t)item * V;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    if (class_temp > 0.f) {
        // largest key K with #{v : key(lp_v) >= K} >= k_keep (bisection on [lo, hi])
        int64_t lo = INT32_MIN, hi = INT32_MAX;
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo + 1) / 2;
            int cnt = 0;
            for (int v = lane; v < V; v += 64) cnt += (int64_t)fkey(lp[v]) >= mid;
            cnt = (int)wave_sum((float)cnt);
            if (cnt >= k_keep) lo = mid;
            else hi = mid - 1;
        }
        const int th = (int)lo;
        int gt = 0;
        for (int v = lane; v < V; v += 64) gt += fkey(lp[v]) > th;
        gt = (int)wave_sum((float)gt);
        const int need = k_keep - gt;  // ties at the threshold kept, lowest class ids first
        int carry = 0;
        for (int v0 = 0; v0 < V; v0 += 64) {
            const int v = v0 + lane;
            const bool in = v < V;
            const int key = in ? fkey(lp[v]) : INT32_MIN;
            const bool eq = in && key == th;
            const uint64_t bal = __ballot(eq);
            const int below = __popcll(bal & ((1ull << lane) - 1ull));
            const bool keep = in && (key > th || (eq && carry + below < need));
            carry += __popcll(bal);
            if (in) {
                const float val = keep ? lp[v] / class_temp + gumbel_f(u[v]) : -INFINITY;
                argmax_merge(best, bi, val, v);
            }
        }
    } else {
        for (int v = lane; v < V; v += 64) argmax_merge(best, bi, lp[v], v);
    }
    wave_argmax(best, bi);
    if (lane == 0) {
        float sc = best - (float)k * penalty;
        if (pos_temp > 0.f) sc += pos_temp * gumbel_f(u_pos[item]);
        pred[item] = bi;
        conf[item] = (codes[(int64_t)k * codes_ld + t] == mask_id) ? sc : -INFINITY;
    }
}

void launch_maskgit_sample(const float *logits, const float *logits_u, float cfg_scale, int T, int ld, int n_cb,
                           int V, int mask_id, float penalty, const int32_t *codes, int codes_ld, float class_temp,
                           float pos_temp, int k_keep, const float *u_class, const float *u_pos, int32_t *pred,
                           float *conf, hipStream_t s) {
    const int items = n_cb * T;
    if (items <= 0) return;
    hipLaunchKernelGGL(maskgit_sample_kernel, dim3((items + 3) / 4), dim3(256), 0, s, logits, logits_u, cfg_scale,
                       T, ld, n_cb, V, mask_id, penalty, codes, codes_ld, class_temp, pos_temp, k_keep, u_class,
                       u_pos, pred, conf);
}

constexpr int SEL_TILE = 1024;  // scores staged in LDS per block

__global__ void zero_i32_kernel(int32_t *v, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) v[i] = 0;
}

// rank[i] += #{j in this block's tile : conf[j] > conf[i] or (== and j < i)}
__global__ __launch_bounds__(256) void rank_count_kernel(const float *conf, int n, int32_t *rank) {
    __shared__ __attribute__((aligned(16))) float tile[SEL_TILE];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int j0 = blockIdx.y * SEL_TILE;
    const int cnt = min(SEL_TILE, n - j0);
    for (int j = threadIdx.x; j < SEL_TILE; j += 256) tile[j] = j < cnt ? conf[j0 + j] : -INFINITY;
    __syncthreads();
    if (i >= n) return;
    const float ci = conf[i];
    int r = 0;
    const int lim = i - j0;  // tile positions j < lim have a lower flat index than i
    for (int j = 0; j < cnt; j += 4) {
        const float4 c = *reinterpret_cast<const float4 *>(&tile[j]);
        r += (c.x > ci) || (c.x == ci && j < lim);
        r += (c.y > ci) || (c.y == ci && j + 1 < lim);
        r += (c.z > ci) || (c.z == ci && j + 2 < lim);
        r += (c.w > ci) || (c.w == ci && j + 3 < lim);
    }
    // positions past cnt hold -inf: they can only tie with a -inf score, and such a
    // position has a higher index than every real one, so they never count
    if (r) atomicAdd(&rank[i], r);
}

__global__ void select_scatter_kernel(const float *conf, const int32_t *pred, const int32_t *rank, int n, int T,
                                      int n_unmask, int32_t *codes, int codes_ld, int32_t *picked) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int r = rank[i];
    if (r >= n_unmask) return;
    if (conf[i] > -INFINITY) {
        picked[r] = i;
        codes[(int64_t)(i / T) * codes_ld + i % T] = pred[i];
    } else {
        picked[r] = -1;
    }
}

void launch_select_update(const float *conf, const int32_t *pred, int n_cb, int T, int n_unmask,
                          int32_t *rank, int32_t *codes, int codes_ld, int32_t *picked, hipStream_t s) {
    const int n = n_cb * T;
    if (n <= 0 || n_unmask <= 0) return;
    const int blocks = (n + 255) / 256;
    hipLaunchKernelGGL(zero_i32_kernel, dim3(blocks), dim3(256), 0, s, rank, n);
    hipLaunchKernelGGL(rank_count_kernel, dim3(blocks, (n + SEL_TILE - 1) / SEL_TILE), dim3(256), 0, s, conf,
                       n, rank);
    hipLaunchKernelGGL(select_scatter_kernel, dim3(blocks), dim3(256), 0, s, conf, pred, rank, n, T, n_unmask,
                       codes, codes_ld, picked);
}

}  // namespace ttsbb
