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

// A group holding a NaN (no order) has no defined maximum: the kernel raises
// FLAG_NONFINITE; the choice is the argmax of the group's other values, or class 0 when
// every value is NaN.
// One block per (row, group): each thread takes the classes tid, tid + 256, ... and
// requests up to 16 of them before comparing any, so a 3072-class group costs one round of
// loads rather than a chain of 48 per lane; the four waves merge through LDS in a fixed
// order (ties to the lowest class id either way).
__global__ __launch_bounds__(256) void argmax_groups_kernel(const float *logits, int rows, int ld,
                                                            int n_groups, int V, int32_t *out, int *flag) {
    constexpr int BATCH = 16;
    __shared__ float red_v[4];
    __shared__ int red_i[4], red_nan[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int item = blockIdx.x;
    const int gi = item % n_groups, r = item / n_groups;
    const float *x = logits + (int64_t)r * ld + (int64_t)gi * V;
    float best = -INFINITY;
    int bi = 0x7FFFFFFF;
    bool nan = false;
    for (int v0 = 0; v0 < V; v0 += 256 * BATCH) {
        float xs[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int v = v0 + j * 256 + tid;
            xs[j] = v < V ? x[v] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int v = v0 + j * 256 + tid;
            if (v < V) {
                nan |= xs[j] != xs[j];
                argmax_merge(best, bi, xs[j], v);
            }
        }
    }
    wave_argmax(best, bi);
    nan = __any(nan);
    if (lane == 0) {
        red_v[wave] = best;
        red_i[wave] = bi;
        red_nan[wave] = nan;
    }
    __syncthreads();
    if (tid == 0) {
        bool any_nan = red_nan[0];
        for (int w = 1; w < 4; ++w) {
            argmax_merge(best, bi, red_v[w], red_i[w]);
            any_nan |= red_nan[w] != 0;
        }
        if (any_nan) raise_flag(flag, FLAG_NONFINITE);
        out[item] = bi == 0x7FFFFFFF ? 0 : bi;
    }
}

void launch_argmax_groups(const float *logits, int rows, int ld, int n_groups, int group_vocab,
                          int32_t *out, int *flag, hipStream_t s) {
    const int items = rows * n_groups;
    if (items <= 0) return;
    hipLaunchKernelGGL(argmax_groups_kernel, dim3(items), dim3(256), 0, s, logits, rows, ld, n_groups,
                       group_vocab, out, flag);
}

// The choice of a group whose scores have no order (a NaN, or an infinite logit that
// makes the log-softmax undefined): the lowest class id that is not the mask.
__device__ __forceinline__ int invalid_group_class(int mask_id) { return mask_id == 0 ? 1 : 0; }

__global__ __launch_bounds__(256) void maskgit_scores_kernel(const float *logits, const float *logits_u,
                                                             float cfg_scale, int T, int ld, int n_cb, int V,
                                                             int mask_id, float penalty, const int32_t *codes,
                                                             int codes_ld, int32_t *pred, float *conf, int *flag) {
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
        // se >= 1 (the maximum's own term) unless a NaN or an infinite logit entered it:
        // such a group has no scores, is never unmasked and raises the flag
        const bool ok = se >= 1.f && se < INFINITY && bi != 0x7FFFFFFF;
        if (!ok) raise_flag(flag, FLAG_NONFINITE);
        const float lse = mx + logf(se);
        pred[item] = ok ? bi : invalid_group_class(mask_id);
        conf[item] = (ok && codes[(int64_t)k * codes_ld + t] == mask_id) ? (best - lse) - (float)k * penalty
                                                                          : -INFINITY;
    }
}

void launch_maskgit_scores(const float *logits, const float *logits_u, float cfg_scale, int T, int ld,
                           int n_cb, int V, int mask_id, float penalty, const int32_t *codes, int codes_ld,
                           int32_t *pred, float *conf, int *flag, hipStream_t s) {
    const int items = n_cb * T;
    if (items <= 0) return;
    hipLaunchKernelGGL(maskgit_scores_kernel, dim3((items + 3) / 4), dim3(256), 0, s, logits, logits_u, cfg_scale,
                       T, ld, n_cb, V, mask_id, penalty, codes, codes_ld, pred, conf, flag);
}

// K8 from the head's partial statistics (launch_head_scores): 16 lanes per (codebook,
// frame), lane l taking the statistics of tiles j0 + l, j0 + l + 16, ... of the 128-column
// tiles its group meets; they merge by lane exchanges (max, rescaled sum of exp, best
// class with ties to the lowest id), then the scores of maskgit_scores_kernel.
__global__ __launch_bounds__(256) void maskgit_merge_kernel(const float4 *spart, int T, int N, int n_cb, int V,
                                                            int mask_id, float penalty, const int32_t *codes,
                                                            int codes_ld, int32_t *pred, float *conf, int *flag) {
    const int item = blockIdx.x * 16 + (threadIdx.x >> 4);  // flat index k*T + t
    const int l = threadIdx.x & 15;
    if (item >= n_cb * T) return;  // whole 16-lane groups leave together
    const int k = item / T, t = item % T;
    const int tiles_n = (N + 127) / 128;
    const int j0 = (k * V) / 128, j1 = (k * V + V - 1) / 128;
    const float LOG2E = 1.4426950408889634f;
    float M = -INFINITY, S = 0.f, best = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int j = j0 + l; j <= j1; j += 16) {
        const int s = k - (j * 128) / V;  // this group's slot in tile j (0 or 1)
        const float4 p = spart[((int64_t)t * tiles_n + j) * 2 + s];
        const float M2 = fmaxf(M, p.x);
        const float f1 = M == -INFINITY ? 0.f : exp2f((M - M2) * LOG2E);
        const float f2 = p.x == -INFINITY ? 0.f : exp2f((p.x - M2) * LOG2E);
        S = S * f1 + p.y * f2;
        M = M2;
        argmax_merge(best, bi, p.z, __float_as_int(p.w));
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const float M2 = __shfl_xor(M, o, WAVE), S2 = __shfl_xor(S, o, WAVE);
        const float b2 = __shfl_xor(best, o, WAVE);
        const int i2 = __shfl_xor(bi, o, WAVE);
        const float Mx = fmaxf(M, M2);
        const float f1 = M == -INFINITY ? 0.f : exp2f((M - Mx) * LOG2E);
        const float f2 = M2 == -INFINITY ? 0.f : exp2f((M2 - Mx) * LOG2E);
        S = S * f1 + S2 * f2;
        M = Mx;
        argmax_merge(best, bi, b2, i2);
    }
    if (l != 0) return;
    const bool ok = S >= 1.f && S < INFINITY && bi != 0x7FFFFFFF;
    if (!ok) raise_flag(flag, FLAG_NONFINITE);
    const float lse = M + logf(S);
    pred[item] = ok ? bi : invalid_group_class(mask_id);
    conf[item] = (ok && codes[(int64_t)k * codes_ld + t] == mask_id) ? (best - lse) - (float)k * penalty : -INFINITY;
}

void launch_maskgit_merge(const float4 *spart, int T, int N, int n_cb, int V, int mask_id, float penalty,
                          const int32_t *codes, int codes_ld, int32_t *pred, float *conf, int *flag, hipStream_t s) {
    const int items = n_cb * T;
    if (items <= 0) return;
    hipLaunchKernelGGL(maskgit_merge_kernel, dim3((items + 15) / 16), dim3(256), 0, s, spart, T, N, n_cb, V, mask_id,
                       penalty, codes, codes_ld, pred, conf, flag);
}

// ------------------------------------------------------------------------------------
// The sampler's random stream (OmniVoice ARCHITECTURE, "MaskGIT decoder", Determinism: a
// seedable Philox4x32-10 generator whose counter is threaded across calls).
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2,
// 3", SC'11): ten rounds of the 4 x 32-bit Philox bijection, each multiplying words 0
// and 2 by 0xD2511F53 and 0xCD9E8D57 and mixing the high halves with the other words and
// the key, whose halves advance by the Weyl constants 0x9E3779B9 and 0xBB67AE85.
// A uniform is ((w >> 9) + 0.5) * 2^-23 of a 32-bit word w: exact in fp32, strictly
// inside (0, 1).
// ------------------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t philox4x32_10(u32x4_t c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
        c = u32x4_t{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

__device__ __forceinline__ float open01(uint32_t w) { return ((float)(w >> 9) + 0.5f) * 0x1p-23f; }

// Word e % 4 of block (base + e / 4) of the call's draws in domain `dom` (word 2 of the
// counter): counter (lo, hi of the 64-bit block, dom, 0), key (lo, hi of the seed).
__device__ __forceinline__ float rng_uniform(uint64_t seed, uint64_t base, uint32_t dom, uint64_t e) {
    const uint64_t b = base + (e >> 2);
    const u32x4_t w = philox4x32_10(u32x4_t{(uint32_t)b, (uint32_t)(b >> 32), dom, 0u}, (uint32_t)seed,
                                    (uint32_t)(seed >> 32));
    const int j = (int)(e & 3);
    return open01(j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w);
}

__global__ void rng_words_kernel(uint64_t seed, uint64_t block0, uint32_t w2, uint32_t w3, int n, uint32_t *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t b = block0 + (uint64_t)i;
    const u32x4_t w = philox4x32_10(u32x4_t{(uint32_t)b, (uint32_t)(b >> 32), w2, w3}, (uint32_t)seed,
                                    (uint32_t)(seed >> 32));
    out[4 * i] = w.x;
    out[4 * i + 1] = w.y;
    out[4 * i + 2] = w.z;
    out[4 * i + 3] = w.w;
}

void launch_rng_words(uint64_t seed, uint64_t block0, uint32_t w2, uint32_t w3, int n_blocks, uint32_t *out,
                      hipStream_t s) {
    if (n_blocks <= 0) return;
    hipLaunchKernelGGL(rng_words_kernel, dim3((n_blocks + 255) / 256), dim3(256), 0, s, seed, block0, w2, w3,
                       n_blocks, out);
}

__global__ void advance_counter_kernel(uint64_t *ctr, uint64_t n) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *ctr += n;
}

void launch_advance_counter(uint64_t *ctr, uint64_t n, hipStream_t s) {
    hipLaunchKernelGGL(advance_counter_kernel, dim3(1), dim3(64), 0, s, ctr, n);
}

// ------------------------------------------------------------------------------------
// K8 with the sampler (same page, "MaskGIT decoder": keep_top_k_ratio(log_probs, 0.1),
// gumbel_sample(temp = class_temp), score += gumbel * pos_temp).  The uniforms of the
// Gumbel noise are the caller's arrays, or, where an array is not given, the call's
// draws of the Philox stream (class noise of element (k, t, v) = flat e = (k T + t) V + v
// in domain RNG_CLASS, position noise of (k, t) in domain RNG_POS, both from the block
// *counter at the call).  One wave per (codebook, frame); the group's V log-probs
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
                                                             uint64_t seed, const uint64_t *counter,
                                                             int32_t *pred, float *conf, int *flag) {
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
    // a NaN or an infinite logit leaves the group without scores (see maskgit_scores_kernel)
    const bool ok = se >= 1.f && se < INFINITY;
    const uint64_t base = counter ? *counter : 0;
    const int64_t e0 = (int64_t)item * V;
    auto u_class_at = [&](int v) {
        return u_class ? u_class[e0 + v] : rng_uniform(seed, base, RNG_CLASS, (uint64_t)(e0 + v));
    };
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
                const float val = keep ? lp[v] / class_temp + gumbel_f(u_class_at(v)) : -INFINITY;
                argmax_merge(best, bi, val, v);
            }
        }
    } else {
        for (int v = lane; v < V; v += 64) argmax_merge(best, bi, lp[v], v);
    }
    wave_argmax(best, bi);
    if (lane == 0) {
        float sc = best - (float)k * penalty;
        if (pos_temp > 0.f)
            sc += pos_temp * gumbel_f(u_pos ? u_pos[item] : rng_uniform(seed, base, RNG_POS, (uint64_t)item));
        const bool valid = ok && bi != 0x7FFFFFFF;
        if (!valid) raise_flag(flag, FLAG_NONFINITE);
        pred[item] = valid ? bi : invalid_group_class(mask_id);
        conf[item] = (valid && codes[(int64_t)k * codes_ld + t] == mask_id) ? sc : -INFINITY;
    }
}

void launch_maskgit_sample(const float *logits, const float *logits_u, float cfg_scale, int T, int ld, int n_cb,
                           int V, int mask_id, float penalty, const int32_t *codes, int codes_ld, float class_temp,
                           float pos_temp, int k_keep, const float *u_class, const float *u_pos, uint64_t seed,
                           const uint64_t *counter, int32_t *pred, float *conf, int *flag, hipStream_t s) {
    const int items = n_cb * T;
    if (items <= 0) return;
    hipLaunchKernelGGL(maskgit_sample_kernel, dim3((items + 3) / 4), dim3(256), 0, s, logits, logits_u, cfg_scale,
                       T, ld, n_cb, V, mask_id, penalty, codes, codes_ld, class_temp, pos_temp, k_keep, u_class,
                       u_pos, seed, counter, pred, conf, flag);
}

constexpr int SEL_TILE = 256;  // scores staged in LDS per block

// Order key of score c at flat index i: larger key = earlier in the selection order
// (higher score; equal scores: lower index).  A score's bits are mapped to an unsigned
// value that orders like the float (sign bit set for >= 0, all bits flipped below 0),
// and the index fills the low word reversed.  Scores are never NaN; every key exceeds 0.
__device__ __forceinline__ uint64_t select_key(float c, int i) {
    const uint32_t b = __float_as_uint(c);
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// rank[i] += #{j in this block's tile of SEL_TILE scores : key(j) > key(i)}.  rank holds
// zeros on entry (the scatter of the previous call, or the context's creation, left it so).
__global__ __launch_bounds__(256) void rank_count_kernel(const float *conf, int n, int32_t *rank) {
    __shared__ __attribute__((aligned(16))) uint64_t tile[SEL_TILE];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int j0 = blockIdx.y * SEL_TILE;
    const int j = j0 + threadIdx.x;
    tile[threadIdx.x] = j < n ? select_key(conf[j], j) : 0;  // 0: below every key
    __syncthreads();
    if (i >= n) return;
    const uint64_t ki = select_key(conf[i], i);
    int r0 = 0, r1 = 0;
#pragma unroll 8
    for (int jj = 0; jj < SEL_TILE; jj += 2) {
        r0 += tile[jj] > ki;
        r1 += tile[jj + 1] > ki;
    }
    const int r = r0 + r1;
    if (r) atomicAdd(&rank[i], r);
}

// picked[rank] = i and the code update for the n_unmask best scores (-1 for a rank whose
// score is -inf); every rank entry is read once and set back to zero for the next call.
__global__ void select_scatter_kernel(const float *conf, const int32_t *pred, int32_t *rank, int n, int T,
                                      int n_unmask, int32_t *codes, int codes_ld, int32_t *picked) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int r = rank[i];
    rank[i] = 0;
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
    hipLaunchKernelGGL(rank_count_kernel, dim3(blocks, (n + SEL_TILE - 1) / SEL_TILE), dim3(256), 0, s, conf,
                       n, rank);
    hipLaunchKernelGGL(select_scatter_kernel, dim3(blocks), dim3(256), 0, s, conf, pred, rank, n, T, n_unmask,
                       codes, codes_ld, picked);
}

}  // namespace ttsbb
