// K4: per-head q/k RMSNorm + half-rotate RoPE + K/V write, and K5: q_len=1 decode
// attention over a paged KV cache.
//
// K4 (OmniVoice ARCHITECTURE, "Qwen3 0.6B backbone with custom IO": per-head RMSNorm
// on Q and K before RoPE, theta 1e6; ncnn Qwen3-TTS port, "单token SDPA问题与host
// attention" and "mRoPE结论": half-rotate RoPE, then the token's K/V are appended to
// the layer's cache).  One block per token; one wave per head; lane l holds dimensions
// l and l+64, which is exactly a RoPE pair, so the rotation is lane-local.  cos/sin
// come from a table computed on the host in double precision.
//
// K5 (same ncnn section: GQA attention of the q_len=1 step; the new token attends to
// positions 0..p).  HBM-bound.  Work item = (stream, KV head, piece of positions);
// one wave per item reads each 16-token page of K and V once with 16-byte non-temporal
// lane loads (a 4 KB bf16 page block is four fully coalesced wave loads) and serves all
// query heads of the GQA group from those registers.  Scores reduce over the lanes
// sharing a token with xor-shuffles; each lane keeps an online-softmax state (max, sum,
// 8 or 4 output dims) in base-2 units; lanes of a piece merge by shuffles; pieces merge
// in a fixed order in the combine kernel (deterministic, no atomics).  The items come
// from a work list built once per step on the device (decode_plan_kernel): for prefill
// rows equal page-aligned chunks of each stream; for q_len = 1 decode the streams' pages
// laid end to end and cut into one segment per wave and KV head (four waves per CU),
// weighted between the even and the odd XCDs, a wave taking its segment's pieces.  When
// every cache fits one chunk (direct mode), a wave covers its stream whole, reads the
// position and page ids itself and writes the output rows itself: no work list and no
// merge.
#include <hip/hip_ext.h>
#include <type_traits>
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ttsbb {

constexpr int COPY_GROUPS = 16;  // prefill: workgroups per KV head copying the cached prefix

// Prefill (dense_copy): the stream's cached positions before the prompt, [0, p0), from the
// paged pool into the dense K rows and V^T (bf16).  Workgroup bx takes KV head bx % Hkv
// and the 64-position groups bx / Hkv, + COPY_GROUPS, ...; K rows are copied in 16-byte
// chunks, V goes through LDS so that the transposed writes (64 positions = 128 bytes per
// dim row) are coalesced.  The prompt's own positions are written by the token blocks.
__device__ void copy_cached_prefix(const RopeKvArgs &a, int bx) {
    __shared__ uint16_t tile[64][128 + 8];
    const int h = bx % a.Hkv, x = bx / a.Hkv;
    const int p0 = min(max(a.pos[0], 0), a.s_pad - a.M);  // as the flash kernel's rows allow
    const uint16_t *pool = reinterpret_cast<const uint16_t *>(a.pool_layer);
    for (int t0 = x * 64; t0 < p0; t0 += COPY_GROUPS * 64) {
        // 64 rows x 16 chunks of 16 bytes: 4 per thread, for K and for V
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int idx = threadIdx.x + 256 * c, t = idx >> 4, ch = idx & 15, p = t0 + t;
            u32x4_t kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (p < p0) {
                const int pi = p / a.page;
                const int pg = pi < a.max_pages ? a.page_table[pi] : -1;
                if (pg >= 0 && pg < a.n_pages) {
                    const int64_t base = (((int64_t)pg * 2 * a.Hkv + h) * a.page + p % a.page) * 128 + ch * 8;
                    kv = *reinterpret_cast<const u32x4_t *>(pool + base);
                    vv = *reinterpret_cast<const u32x4_t *>(pool + base + (int64_t)a.Hkv * a.page * 128);
                }
                *reinterpret_cast<u32x4_t *>(a.kbuf + ((int64_t)h * a.s_pad + p) * 128 + ch * 8) = kv;
            }
            *reinterpret_cast<u32x4_t *>(&tile[t][ch * 8]) = vv;
        }
        __syncthreads();
        uint16_t *vt = a.vtbuf + (int64_t)h * 128 * a.s_pad;
        for (int i = threadIdx.x; i < 128 * 64; i += 256) {
            const int d = i >> 6, t = i & 63;
            if (t0 + t < p0) vt[(int64_t)d * a.s_pad + t0 + t] = tile[t][d];
        }
        __syncthreads();
    }
}

template <typename TKV, bool MULTI>
__global__ __launch_bounds__(256) void rope_kv_kernel(RopeKvArgs a) {
    constexpr int MAXJ = 8;  // heads per wave per pass (MULTI: more than 4 * MAXJ heads)
    if (a.dense_copy && (int)blockIdx.x >= a.M) {
        copy_cached_prefix(a, blockIdx.x - a.M);
        return;
    }
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int width = (a.H + 2 * a.Hkv) * 128;
    const float *row = a.qkv + (int64_t)m * width;
    // dense (bf16) mode leaves V to the transpose kernel below
    const int jobs = a.dense && !a.dense_f32 ? a.H + a.Hkv : a.H + 2 * a.Hkv;

    // Loads complete in order: the position goes first, then all of the first pass's
    // row values (they do not depend on it), and only then the position-dependent
    // page-table and RoPE-table loads, so no wait drains more than it needs.
    int p = a.dense ? (a.seg1 > 0 && m >= a.seg1 ? m - a.seg1 : m) : (a.shared ? a.pos[0] + m : a.pos[m]);
    float u[MAXJ], u2[MAXJ];
#pragma unroll
    for (int i = 0; i < MAXJ; ++i) {
        const int j = min(wave + 4 * i, jobs - 1);  // clamped: unconditional loads
        u[i] = row[j * 128 + lane];
        u2[i] = row[j * 128 + 64 + lane];
    }
    __builtin_amdgcn_sched_barrier(0);

    // position-dependent loads, all issued before any check (indices clamped in range)
    const int pc = min(max(p, 0), a.max_pos - 1);
    const int pi = a.dense ? 0 : min(pc / a.page, a.max_pages - 1);  // dense mode: no page table
    const int page_id = a.dense ? 0 : a.page_table[(int64_t)(a.shared ? 0 : m) * a.max_pages + pi];
    const float2 cs = a.rope[(int64_t)pc * 64 + lane];
    const float gq0 = a.q_gain[lane], gq1 = a.q_gain[lane + 64];
    const float gk0 = a.k_gain[lane], gk1 = a.k_gain[lane + 64];
    const int slot = a.dense ? 0 : pc % a.page;
    bool ok = true;
    if (p != pc) {
        if (threadIdx.x == 0) raise_flag(a.flag, FLAG_POSITION);
        ok = false;
    }
    if (!a.dense) {
        if (pc / a.page >= a.max_pages) {
            if (threadIdx.x == 0) raise_flag(a.flag, FLAG_POSITION);
            ok = false;
        } else if (page_id < 0 || page_id >= a.n_pages) {
            if (threadIdx.x == 0) raise_flag(a.flag, FLAG_PAGE);
            ok = false;
        }
    }

    // every operand of the first pass has been requested: one wait for all of them, so
    // that the stores below are never waited on
    __builtin_amdgcn_s_waitcnt(0);
    for (int j0 = wave; j0 < (MULTI ? jobs : wave + 1); j0 += 4 * MAXJ) {
        if (MULTI && j0 != wave) {  // further passes
#pragma unroll
            for (int i = 0; i < MAXJ; ++i) {
                const int j = min(j0 + 4 * i, jobs - 1);
                u[i] = row[j * 128 + lane];
                u2[i] = row[j * 128 + 64 + lane];
            }
        }
#pragma unroll
        for (int i = 0; i < MAXJ; ++i) {
            const int j = j0 + 4 * i;
            if (j >= jobs) continue;
            float x = u[i], x2 = u2[i];
            if (j < a.H + a.Hkv) {
                const float ss = wave_sum(x * x + x2 * x2);
                const float inv = 1.0f / sqrtf(ss / 128.0f + a.eps);
                const float x0 = x * inv * (j < a.H ? gq0 : gk0), x1 = x2 * inv * (j < a.H ? gq1 : gk1);
                x = x0 * cs.x - x1 * cs.y;
                x2 = x1 * cs.x + x0 * cs.y;
            }
            if (j < a.H) {
                if ((a.dense && !a.dense_f32) || a.q_bf16) {
                    bf16_t *q = reinterpret_cast<bf16_t *>(a.q_out) + (int64_t)m * a.H * 128 + j * 128;
                    q[lane] = f32_to_bf16(x);
                    q[lane + 64] = f32_to_bf16(x2);
                } else {
                    float *q = reinterpret_cast<float *>(a.q_out) + (int64_t)m * a.H * 128 + j * 128;
                    q[lane] = x;
                    q[lane + 64] = x2;
                }
                continue;
            }
            const int kv = j < a.H + a.Hkv ? 0 : 1;
            const int h = j - a.H - kv * a.Hkv;
            if (a.dense_f32) {
                float *dst = reinterpret_cast<float *>(kv ? a.vtbuf : a.kbuf) + ((int64_t)h * a.s_pad + m) * 128;
                dst[lane] = x;
                dst[lane + 64] = x2;
            } else if (a.dense) {
                bf16_t *k = a.kbuf + ((int64_t)h * a.s_pad + m) * 128;
                k[lane] = f32_to_bf16(x);
                k[lane + 64] = f32_to_bf16(x2);
            } else {
                if (ok) {
                    TKV *dst = reinterpret_cast<TKV *>(a.pool_layer) +
                               ((((int64_t)page_id * 2 + kv) * a.Hkv + h) * a.page + slot) * 128;
                    dst[lane] = from_f32<TKV>(x);
                    dst[lane + 64] = from_f32<TKV>(x2);
                }
                // prefill: the token's K row and V^T column of the dense buffers at its
                // position (any position below max_pos <= s_pad; the pool write above
                // also needs a valid page)
                if (a.dense_copy && p == pc) {
                    if (kv == 0) {
                        bf16_t *kd = a.kbuf + ((int64_t)h * a.s_pad + p) * 128;
                        kd[lane] = f32_to_bf16(x);
                        kd[lane + 64] = f32_to_bf16(x2);
                    } else {
                        bf16_t *vt = a.vtbuf + (int64_t)h * 128 * a.s_pad + p;
                        vt[(int64_t)lane * a.s_pad] = f32_to_bf16(x);
                        vt[(int64_t)(lane + 64) * a.s_pad] = f32_to_bf16(x2);
                    }
                }
            }
        }
    }
}

// Dense mode: V^T [Hkv][128][s_pad] (bf16) from the V part of qkv, 64 tokens x 128 dims
// per block through LDS, so that both the fp32 reads and the bf16 writes (64 tokens =
// 128 bytes per dim row) are coalesced.
__global__ __launch_bounds__(256) void dense_vt_kernel(RopeKvArgs a) {
    __shared__ float tile[64][129];
    const int t0 = blockIdx.x * 64, h = blockIdx.y;
    const int width = (a.H + 2 * a.Hkv) * 128;
    const int off = (a.H + a.Hkv + h) * 128;
    for (int i = threadIdx.x; i < 64 * 128; i += 256) {
        const int t = i >> 7, d = i & 127;
        tile[t][d] = (t0 + t < a.M) ? a.qkv[(int64_t)(t0 + t) * width + off + d] : 0.f;
    }
    __syncthreads();
    bf16_t *vt = a.vtbuf + (int64_t)h * 128 * a.s_pad;
    for (int i = threadIdx.x; i < 128 * 64; i += 256) {
        const int d = i >> 6, t = i & 63;
        if (t0 + t < a.M) vt[(int64_t)d * a.s_pad + t0 + t] = f32_to_bf16(tile[t][d]);
    }
}

void launch_rope_kv(const RopeKvArgs &a, DType kv_dt, hipStream_t s) {
    if (a.M <= 0) return;
    const bool multi = (a.dense && !a.dense_f32 ? a.H + a.Hkv : a.H + 2 * a.Hkv) > 32;
    const dim3 grid(a.M + (a.dense_copy ? a.Hkv * COPY_GROUPS : 0));
    if (kv_dt == DT_BF16 || a.dense) {
        if (multi) hipLaunchKernelGGL((rope_kv_kernel<bf16_t, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((rope_kv_kernel<bf16_t, false>), grid, dim3(256), 0, s, a);
    } else {
        if (multi) hipLaunchKernelGGL((rope_kv_kernel<float, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((rope_kv_kernel<float, false>), grid, dim3(256), 0, s, a);
    }
    if (a.dense && !a.dense_f32)
        hipLaunchKernelGGL(dense_vt_kernel, dim3((a.M + 63) / 64, a.Hkv), dim3(256), 0, s, a);
}

// ------------------------------------------------------------------------------------
// K5
// ------------------------------------------------------------------------------------
constexpr int PART_STRIDE = 132;

template <typename T> struct KVRaw {
    static constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte lane load
    __device__ static void unpack(const u32x4_t &t, float v[EPL]);
};
template <> __device__ inline void KVRaw<bf16_t>::unpack(const u32x4_t &t, float v[8]) {
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <> __device__ inline void KVRaw<float>::unpack(const u32x4_t &t, float v[4]) {
    v[0] = __uint_as_float(t.x); v[1] = __uint_as_float(t.y);
    v[2] = __uint_as_float(t.z); v[3] = __uint_as_float(t.w);
}

// Issue the 16-byte lane loads of the K and V blocks of page `pg` of a stream.
template <typename T, int NR, int RPL>
__device__ __forceinline__ bool load_page(const T *pool, int page_id, int n_pages, int Hkv, int hk,
                                          int64_t blk, int lane_off, u32x4_t (&kr)[NR], u32x4_t (&vr)[NR]) {
    // An invalid id (flagged by K4) reads page 0, which always exists, and is ignored.
    // Non-temporal loads: a launch reads each cached K / V byte once, and the streaming
    // policy keeps it from being allocated through L2 and the memory-side cache (64-stream
    // decode: 93.8 -> 85.8 us per launch).
    const bool ok = page_id >= 0 && page_id < n_pages;
    const T *kb = pool + (((int64_t)(ok ? page_id : 0) * 2 + 0) * Hkv + hk) * blk + lane_off;
    const T *vb = kb + (int64_t)Hkv * blk;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        kr[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(kb + r * RPL * 128));
        vr[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vb + r * RPL * 128));
    }
    return ok;
}

// Online-softmax update of one wave with one 16-token page: scores of the lane's tokens
// (reduced over the LPR lanes sharing a token), running max / sum, V accumulation.
template <typename T, int GROUP, int NR, int RPL>
__device__ __forceinline__ void process_page(const u32x4_t (&kr)[NR], const u32x4_t (&vr)[NR], int nvalid,
                                             int rsub, const float (&qv)[GROUP][KVRaw<T>::EPL],
                                             float (&m_run)[GROUP], float (&l_run)[GROUP],
                                             float (&acc)[GROUP][KVRaw<T>::EPL]) {
    constexpr int EPL = KVRaw<T>::EPL;
    constexpr int LPR = 128 / EPL;
    float s[NR][GROUP];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int tok = rsub + RPL * r;
        float kv[EPL];
        KVRaw<T>::unpack(kr[r], kv);
#pragma unroll
        for (int j = 0; j < GROUP; ++j) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(qv[j][e], kv[e], d);
            d = group_sum<LPR>(d);
            s[r][j] = tok < nvalid ? d : -INFINITY;
        }
    }
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
        float mx = m_run[j];
#pragma unroll
        for (int r = 0; r < NR; ++r) mx = fmaxf(mx, s[r][j]);
        if (mx == -INFINITY) {  // nothing valid for this lane yet
#pragma unroll
            for (int r = 0; r < NR; ++r) s[r][j] = 0.f;
            continue;
        }
        const float sc = exp2f(m_run[j] - mx);
        l_run[j] *= sc;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= sc;
        m_run[j] = mx;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            s[r][j] = exp2f(s[r][j] - mx);
            l_run[j] += s[r][j];
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int tok = rsub + RPL * r;
        if (tok >= nvalid) continue;  // slots past the length may hold anything
        float vv[EPL];
        KVRaw<T>::unpack(vr[r], vv);
#pragma unroll
        for (int j = 0; j < GROUP; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(s[r][j], vv[e], acc[j][e]);
    }
}

// Value of dimension d +- 64 of the same head (the RoPE partner), held by the lane LPR/2
// away inside the lane's row group.
template <int LPR>
__device__ __forceinline__ float rope_partner(float v) {
    if constexpr (LPR == 16) return dpp_f<DPP_ROR8>(v);
    else return __shfl_xor(v, LPR / 2, WAVE);
}

// Per-head RMSNorm + RoPE of one 128-dim head row of the step's projections, in the decode
// kernel's lane layout (lane holds dims d0 .. d0 + EPL - 1; the LPR lanes of a row group
// hold the whole head): y = x / sqrt(mean(x^2) + eps) * g, then dims d and d + 64 rotated
// by the angle of pair d mod 64.
template <int EPL, int LPR>
__device__ __forceinline__ void norm_rope_head(const float *x, const float *gain, int d0, const float (&c)[EPL],
                                               const float (&sn)[EPL], float eps, float (&out)[EPL]) {
    float y[EPL], ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss = fmaf(x[e], x[e], ss);
    ss = group_sum<LPR>(ss);
    const float inv = 1.0f / sqrtf(ss / 128.0f + eps);
#pragma unroll
    for (int e = 0; e < EPL; ++e) y[e] = x[e] * inv * gain[e];
    const bool first = d0 < 64;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const float pv = rope_partner<LPR>(y[e]);
        out[e] = first ? y[e] * c[e] - pv * sn[e] : y[e] * c[e] + pv * sn[e];
    }
}

// One work item of the decode attention on one wave: a piece of one stream's positions
// (a work-list entry) for one KV head, or in direct mode the stream's whole cache.  The
// K and V blocks of the next page are loaded into a second register set while the
// current page is processed, so the wave keeps one page (8 KB in bf16) of loads in
// flight behind its arithmetic.  Returns false when `pair` lies past the work list (or
// the batch) or names an empty entry.
template <typename T, int GROUP, bool FUSED, bool DIRECT>
__device__ __forceinline__ bool decode_attn_item(const DecodeAttnArgs &a, int pair, int hk, int limit) {
    constexpr int EPL = KVRaw<T>::EPL;
    constexpr int LPR = 128 / EPL;  // lanes per 128-dim row
    constexpr int RPL = 64 / LPR;   // rows (tokens) per wave load
    constexpr int NR = 16 / RPL;    // wave loads per 16-token page block
    const int lane = threadIdx.x & 63;
    // pair: an entry of the step's work list (entries at or past `limit` -- plan_n[0] when
    // limit < 0 -- and empty ones do nothing), or in direct mode the stream
    const int d0 = (lane % LPR) * EPL;
    const int rsub = lane / LPR;
    const int cap = a.max_pages * a.page;
    // The piece's page ids (one per lane) come with the pair, in the same round of loads,
    // and are read once: a page-id load inside the page loop would have to complete before
    // the next page's addresses exist, and loads complete in order, so that wait would also
    // drain the prefetch.
    int b, c, p_tok, p_begin, chunk, my_page;  // chunk: the piece's positions; p_tok: the step token's
    if (DIRECT) {
        // one item per (stream, KV head) over the whole cache: positions and page ids from
        // the stream's own entries, no work list
        if (pair >= a.B) return false;
        b = pair;
        c = 0;
        p_begin = 0;
        chunk = cap;
        p_tok = a.pos[b];
        my_page = a.page_table[(int64_t)b * a.max_pages + min(lane, a.max_pages - 1)];
        const bool bad = p_tok < 0 || p_tok >= a.max_pos || p_tok >= cap;
        if (bad && hk == 0 && lane == 0) raise_flag(a.flag, FLAG_POSITION);
        if (p_tok < 0) {  // no cached position: zero rows, as the merge writes for such a stream
#pragma unroll
            for (int j = 0; j < GROUP; ++j)
                if (lane < LPR) {
                    const int k = (hk * GROUP + j) * 128 + d0;
                    T *o = reinterpret_cast<T *>(a.out) +
                           (a.out_mt > 0 ? frag_index(b, k, a.out_mt) : (int64_t)b * a.H * 128 + k);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[e] = from_f32<T>(0.f);
                }
            return true;
        }
    } else {
        const int pc = min(pair, a.plan_cap - 1);
        const int n_pairs = limit >= 0 ? limit : *a.plan_n;
        const int4 w = a.plan[pc];
        my_page = a.plan_pages[(int64_t)pc * 64 + lane];
        b = w.x;
        c = w.y & 0xFFFF;
        chunk = (w.y >> 16) * a.page;  // the piece's pages
        p_tok = w.z;
        p_begin = w.w;
        if (pair >= n_pairs || chunk == 0 || b >= a.B || c >= a.part_stride) return false;
    }
    const int pg_first = p_begin / a.page;
    // FUSED: the raw q rows and the q gains do not depend on the position either; they
    // are requested in the same round as it
    const float *row = FUSED ? a.qkv + (int64_t)b * (a.H + 2 * a.Hkv) * 128 : nullptr;
    float x[GROUP][EPL], gq[EPL];
    if (FUSED) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) gq[e] = a.q_gain[d0 + e];
#pragma unroll
        for (int j = 0; j < GROUP; ++j)
#pragma unroll
            for (int e = 0; e < EPL; ++e) x[j][e] = row[(hk * GROUP + j) * 128 + d0 + e];
    }
    const int L = min(p_tok + 1, cap);  // the plan holds pieces below L only
    const int p_end = min(L, p_begin + chunk);
    // FUSED: the piece that holds the token's slot takes the token's K / V from registers
    // (rounded to the pool's type, as a read-back would give) and scans only the earlier
    // positions, so its page reads never wait for the slot's store
    const bool tok_here = FUSED && p_tok >= p_begin && p_tok < p_end;
    const int scan_end = tok_here ? p_tok : p_end;

    const T *pool = reinterpret_cast<const T *>(a.pool_layer);
    const int64_t blk = (int64_t)a.page * 128;  // elements of one (page, K|V, head) block
    const int lane_off = rsub * 128 + d0;
    const int pg_last = (scan_end - 1) / a.page;
    auto page_of = [&](int pg) { return __builtin_amdgcn_readlane(my_page, pg - pg_first); };
    u32x4_t ka[NR], va[NR], kb2[NR], vb2[NR];

    float qv[GROUP][EPL];
    float m_run[GROUP], l_run[GROUP], acc[GROUP][EPL];
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
    }
    bool ok_a;
    if (FUSED) {
        const int pc = min(max(p_tok, 0), a.max_pos - 1);
        float cr[EPL], sr[EPL], kx[EPL], vx[EPL], gk[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float2 t = a.rope[(int64_t)pc * 64 + ((d0 + e) & 63)];
            cr[e] = t.x;
            sr[e] = t.y;
        }
        if (tok_here) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                kx[e] = row[(a.H + hk) * 128 + d0 + e];
                vx[e] = row[(a.H + a.Hkv + hk) * 128 + d0 + e];
                gk[e] = a.k_gain[d0 + e];
            }
        }
        // the first page goes out behind the position-dependent loads: waiting for those
        // leaves it in flight while q is normalised and rotated
        ok_a = load_page<T, NR, RPL>(pool, page_of(pg_first), a.n_pages, a.Hkv, hk, blk, lane_off, ka, va);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < GROUP; ++j) {
            norm_rope_head<EPL, LPR>(x[j], gq, d0, cr, sr, a.eps, qv[j]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) qv[j][e] *= a.scale_log2;
        }
        if (tok_here) {
            float kn[EPL];
            norm_rope_head<EPL, LPR>(kx, gk, d0, cr, sr, a.eps, kn);
            T kt[EPL], vt[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                kt[e] = from_f32<T>(kn[e]);
                vt[e] = from_f32<T>(vx[e]);
            }
            const int page_id = __builtin_amdgcn_readlane(my_page, p_tok / a.page - pg_first);
            const bool ok = p_tok < a.max_pos && page_id >= 0 && page_id < a.n_pages;
            if (p_tok < a.max_pos && !ok && hk == 0 && lane == 0) raise_flag(a.flag, FLAG_PAGE);
            if (ok && rsub == 0) {
                T *dst = reinterpret_cast<T *>(a.pool_layer) +
                         ((((int64_t)page_id * 2) * a.Hkv + hk) * a.page + p_tok % a.page) * 128 + d0;
                T *dsv = dst + (int64_t)a.Hkv * a.page * 128;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    dst[e] = kt[e];
                    dsv[e] = vt[e];
                }
            }
            // the token as the first key of lane group 0 (every lane group holds the
            // whole row, so every lane gets the same score)
#pragma unroll
            for (int j = 0; j < GROUP; ++j) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d = fmaf(qv[j][e], to_f32<T>(kt[e]), d);
                d = group_sum<LPR>(d);
                if (rsub == 0) {
                    m_run[j] = d;
                    l_run[j] = 1.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[j][e] = to_f32<T>(vt[e]);
                }
            }
        }
        // the prologue's temporaries die here, before the page pipeline's registers are live
        __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
        for (int j = 0; j < GROUP; ++j) {
            const float *q = a.q + (int64_t)b * a.H * 128 + (hk * GROUP + j) * 128 + d0;
#pragma unroll
            for (int e = 0; e < EPL; ++e) qv[j][e] = q[e] * a.scale_log2;
        }
        ok_a = load_page<T, NR, RPL>(pool, page_of(pg_first), a.n_pages, a.Hkv, hk, blk, lane_off, ka, va);
    }

    // Ping-pong over the piece's pages.  Every load is issued unconditionally (the index
    // is clamped to the last page, whose re-read hits L2) and every page is processed
    // unconditionally (an invalid page counts no valid token), so no branch forces the
    // outstanding prefetch to drain.
    const int np = pg_last - pg_first + 1;
    bool ok_b;
    for (int i = 0; i < np; i += 2) {
        // ping: page i in (ka, va); pong: page i + 1 in (kb2, vb2)
        const int pg = pg_first + i;
        ok_b = load_page<T, NR, RPL>(pool, page_of(pg_first + min(i + 1, np - 1)), a.n_pages, a.Hkv, hk, blk,
                                     lane_off, kb2, vb2);
        process_page<T, GROUP, NR, RPL>(ka, va, ok_a ? scan_end - pg * a.page : 0, rsub, qv, m_run, l_run, acc);
        if (i + 1 >= np) break;
        ok_a = load_page<T, NR, RPL>(pool, page_of(pg_first + min(i + 2, np - 1)), a.n_pages, a.Hkv, hk, blk,
                                     lane_off, ka, va);
        process_page<T, GROUP, NR, RPL>(kb2, vb2, ok_b ? scan_end - (pg + 1) * a.page : 0, rsub, qv, m_run, l_run,
                                        acc);
    }

    // merge the RPL lane groups (same dims, different tokens)
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
        float mt = m_run[j];
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) mt = fmaxf(mt, __shfl_xor(mt, o, WAVE));
        const float sc = (m_run[j] == -INFINITY) ? 0.f : exp2f(m_run[j] - mt);
        float lt = l_run[j] * sc;
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) lt += __shfl_xor(lt, o, WAVE);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float v = acc[j][e] * sc;
#pragma unroll
            for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, WAVE);
            acc[j][e] = v;
        }
        if (DIRECT) {
            // the stream's only chunk: its normalised output, as the merge computes it from
            // one partial (weight 2^0 = 1, sum 1 * lt, then acc * (1 / sum))
            const float inv = 1.0f / lt;
            if (lane < LPR) {
                const int k = (hk * GROUP + j) * 128 + d0;  // EPL contiguous columns in both layouts
                T *o = reinterpret_cast<T *>(a.out) + (a.out_mt > 0 ? frag_index(b, k, a.out_mt) : (int64_t)b * a.H * 128 + k);
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = from_f32<T>(acc[j][e] * inv);
            }
            continue;
        }
        float *part = a.part + (((int64_t)b * a.H + hk * GROUP + j) * a.part_stride + c) * PART_STRIDE;
        if (lane < LPR) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) part[4 + d0 + e] = acc[j][e];
        }
        if (lane == 0) {
            part[0] = mt;
            part[1] = lt;
        }
    }
    return true;
}

// The grid: in segment mode (q_len = 1 decode) one wave per segment and KV head; for
// prefill rows as many waves as the chunks the caches could hold; in direct mode one per
// stream and KV head.  Outside segment mode each wave takes items wave, wave + (waves in
// the grid), ... until the list runs out.
// DIRECT: a.direct (a separate instantiation, so the work-list kernels keep their
// registers; short caches are latency-bound, so it takes the 3-wave register budget).
template <typename T, int GROUP, bool FUSED, bool DIRECT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? (FUSED || DIRECT ? 3 : 4) : 2)))
void decode_attn_kernel(DecodeAttnArgs a) {
    // wave-uniform by construction; readfirstlane lets the compiler keep the item's
    // indices in scalar registers (no per-lane page-id selection loops)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // segment mode: segment k on workgroups of parity k & 1 (Hkv / 4 of them, one KV head
    // per wave); KV heads vary fastest, so a block streams neighbouring 4 KB blocks of the
    // same pool pages (a page holds all heads' K and V contiguously)
    const bool seg = !DIRECT && a.target_items > 0;
    int k = 0, hk = 0;
    int2 more = make_int2(0, 0);
    if (seg) {
        if ((a.Hkv & 3) == 0) {
            const int bps = a.Hkv >> 2, t = blockIdx.x >> 1;
            k = 2 * (t / bps) + (blockIdx.x & 1);
            hk = (t % bps) * 4 + wave;
        } else {
            const int item = blockIdx.x * 4 + wave;
            k = item / a.Hkv;
            hk = item % a.Hkv;
        }
        if (k >= a.n_seg) return;
        more = a.seg_cont[k];  // requested with the first piece's entry
    }
    // one call site, so that the item's code is inlined once: segment mode takes the first
    // piece (entry k), then entries n_seg + more.x + j - 1 (`more` is read only after the
    // first piece, so its load is not waited for before that piece's loads); otherwise
    // items wave, wave + (waves in the grid), ...
    int pair, h, limit, item = 0;
    if (seg) {
        pair = k;
        h = hk;
        limit = a.n_seg;
    } else {
        item = blockIdx.x * 4 + wave;
        pair = item / a.Hkv;
        h = item % a.Hkv;
        limit = -1;
    }
    for (int j = 0;; ++j) {
        if (!decode_attn_item<T, GROUP, FUSED, DIRECT>(a, pair, h, limit)) break;
        if (seg) {
            if (j >= more.y) break;
            pair = a.n_seg + more.x + j;
            limit = a.plan_cap;
        } else {
            item += gridDim.x * 4;
            pair = item / a.Hkv;
            h = item % a.Hkv;
        }
    }
}

// The split of a stream's L cached positions for the step's chunk bound c (a multiple of
// the page): n = ceil(L / c) items would leave a short remainder item, so the positions
// are spread evenly instead -- every item holds `len` = ceil(L / n) positions rounded up
// to a page (at most c), the last one the rest -- and n is recounted from len so that no
// item is empty.  The work list and the merge both use it, so they agree on the items.
__device__ __forceinline__ void stream_split(int L, int c, int page, int &n, int &len) {
    if (L <= 0) {
        n = 0;
        len = c;
        return;
    }
    const int n0 = (L + c - 1) / c;
    len = ((L + n0 - 1) / n0 + page - 1) / page * page;
    n = (L + len - 1) / len;
}

// The decode attention's work list, built once per step (the positions are the same in
// every layer).  Streams with no valid position get no piece; with a.flag set such a
// token raises FLAG_POSITION.
//  * target_items == 0 (prefill rows): every stream is cut into ceil(L / chunk) equal
//    page-aligned pieces (stream_split), entries in stream order.
//  * target_items > 0 (q_len = 1 decode): the streams' pages laid end to end are cut into
//    w_eff <= n_seg segments; a piece is a stream's part of a segment, at most 64 pages.
//    When the segments average at least SEG_WEIGHTED_PAGES pages (bandwidth-bound waves)
//    their page counts are weighted SEG_WE : SEG_WO between even and odd segments (the
//    even ones run on the even XCDs, which stream faster), so all waves of the launch
//    finish at about the same time; shorter segments are equal (latency-bound waves: the
//    longest chain sets the time).  w_eff starts at min(n_seg, ceil(P / 2)) for P pages
//    (every segment then holds one or more pages) and drops until each stream's pieces fit its
//    part_stride partial slots (always true by w_eff = 2: at most ceil(pages / 64) + 1
//    pieces, and part_stride >= n_chunks + 2).
constexpr int SEG_WE = 9, SEG_WO = 8;
constexpr int SEG_WEIGHTED_PAGES = 8;  // least mean segment (pages) that takes the weights

// First page of segment k of w over P pages with weights we (even k) and wo (odd k); P
// for k >= w.  64-bit products: P can exceed 2^31 / (w * 9).
__device__ inline int seg_start(int k, int w, int P, int we, int wo) {
    if (k >= w) return P;
    auto before = [&](int j) { return (int64_t)(j >> 1) * (we + wo) + (j & 1) * we; };
    return (int)((int64_t)P * before(k) / before(w));
}

// The segment that holds page q: the last k < w with start[k] <= q (start[] in LDS,
// non-decreasing, start[0] = 0).
__device__ inline int seg_find(const int *start, int w, int q) {
    int lo = 0, hi = w - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= q) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Whether no segment exceeds 64 pages (one piece per segment and stream): a segment's
// size is at most ceil(P * max(we, wo) / before(w)).
__device__ inline bool seg_small(int w, int P, int we, int wo) {
    const int64_t bw = (int64_t)(w >> 1) * (we + wo) + (w & 1) * we;
    return (int64_t)P * max(we, wo) <= 64 * bw;
}

// Pieces of a stream whose np > 0 pages start at page `off` of the laid-out sequence (no
// segment is empty; `small`: seg_small holds, so the count is that of the segments its
// first and last pages span).
__device__ inline int seg_pieces(const int *start, int w, int off, int np, bool small) {
    if (small) return seg_find(start, w, off + np - 1) - seg_find(start, w, off) + 1;
    int n = 0;
    for (int q = off, k = seg_find(start, w, off); q < off + np && k < w; ++k) {
        const int se = min(off + np, start[k + 1]);
        n += (se - q + 63) / 64;
        q = max(q, se);
    }
    return n;
}

__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeAttnArgs a, int4 *plan, int *plan_n) {
    __shared__ int wsum[16];
    __shared__ int sstart[SEG_MAX + 1];  // q_len = 1 decode: first page of each segment
    __shared__ int sfirst[SEG_MAX];      // ... and the global index of its first piece
    // per stream (at most 1024; per-segment writing): first laid-out page, global index of
    // its first piece, segment of its first page, token position
    __shared__ int soff[1025], sg0[1024], skf[1024], stok[1024];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cap = a.max_pages * a.page;
    auto token = [&](int b) { return a.shared ? a.pos[0] + b : a.pos[b]; };
    // positions of stream b in the cache (0 for an invalid token)
    auto length = [&](int b) { return max(0, min(token(b) + 1, cap)); };
    auto block_sum = [&](int v) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, WAVE);
        __syncthreads();  // wsum's previous use is over
        if (lane == 0) wsum[wave] = v;
        __syncthreads();
        int t = 0;
        for (int k = 0; k < 16; ++k) t += wsum[k];
        return t;
    };
    auto block_max = [&](int v) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) v = max(v, __shfl_xor(v, o, WAVE));
        __syncthreads();
        if (lane == 0) wsum[wave] = v;
        __syncthreads();
        int t = 0;
        for (int k = 0; k < 16; ++k) t = max(t, wsum[k]);
        return t;
    };
    // exclusive scan over the block's threads; `total` = the sum over all of them
    auto block_scan = [&](int v, int &total) {
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, WAVE);
            if (lane >= o) incl += t;
        }
        __syncthreads();
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int off = incl - v;
        total = 0;
        for (int k = 0; k < 16; ++k) {
            if (k < wave) off += wsum[k];
            total += wsum[k];
        }
        return off;
    };
    auto check = [&](int b) {
        const int p_tok = token(b);
        if (a.flag && (p_tok < 0 || p_tok >= a.max_pos || p_tok >= cap)) raise_flag(a.flag, FLAG_POSITION);
        return p_tok;
    };

    int n_entries = 0, info = a.chunk;
    if (a.target_items == 0) {
        int base = 0;
        for (int b0 = 0; b0 < a.B; b0 += 1024) {
            const int b = b0 + tid;
            int nc = 0, p_tok = 0, len = a.chunk;
            if (b < a.B) {
                p_tok = check(b);
                stream_split(length(b), a.chunk, a.page, nc, len);  // nc <= n_chunks
                a.plan_nc[b] = nc;
            }
            int total;
            const int off = base + block_scan(nc, total);
            for (int c = 0; c < nc; ++c)
                if (off + c < a.plan_cap) plan[off + c] = make_int4(b, c | ((len / a.page) << 16), p_tok, c * len);
            base += total;
        }
        n_entries = min(base, a.plan_cap);
    } else {
        const int W = a.n_seg;  // <= SEG_MAX
        // streams 0 .. 1023: token and page count read once, kept in a register
        const int tok0 = tid < a.B ? check(tid) : 0;
        const int np0 = tid < a.B ? (max(0, min(tok0 + 1, cap)) + a.page - 1) / a.page : 0;
        auto pages_of = [&](int b0) {
            const int b = b0 + tid;
            return b0 == 0 ? np0 : (b < a.B ? (length(b) + a.page - 1) / a.page : 0);
        };
        int P = np0;
        for (int b = 1024 + tid; b < a.B; b += 1024) P += (length(b) + a.page - 1) / a.page;
        P = block_sum(P);
        int w = P == 0 ? 0 : min(W, (P + 1) / 2);
        bool small;
        while (true) {
            const bool weighted = w > 0 && P >= SEG_WEIGHTED_PAGES * w;
            const int we = weighted ? SEG_WE : 1, wo = weighted ? SEG_WO : 1;
            for (int k = tid; k <= w; k += 1024) sstart[k] = seg_start(k, w, P, we, wo);
            small = seg_small(w, P, we, wo);
            __syncthreads();
            if (w <= 1) break;
            int worst = 0, base = 0;
            for (int b0 = 0; b0 < a.B; b0 += 1024) {
                const int np = pages_of(b0);
                int total;
                const int off = base + block_scan(np, total);
                if (np > 0) worst = max(worst, seg_pieces(sstart, w, off, np, small));
                base += total;
            }
            if (block_max(worst) <= a.part_stride) break;  // (its barriers end the reads of sstart)
            w -= w > 2 ? 2 : 1;
        }
        // the pieces, in stream and position order; G counts them over all streams.  The
        // first piece of segment k goes to entry k, the others to n_seg + G - (k + 1) (every
        // segment below w holds pages, so k + 1 first pieces precede), which makes a
        // segment's further pieces consecutive entries; sfirst[k] = G of segment k's first
        // piece.
        // At most 1024 streams and no segment above 64 pages (one piece per stream and
        // segment): the pieces are written per segment, from the streams' offsets in LDS;
        // otherwise each stream's thread walks its segments.
        const bool by_seg = a.B <= 1024 && small;
        int base = 0, gbase = 0;
        for (int b0 = 0; b0 < a.B; b0 += 1024) {
            const int b = b0 + tid;
            const int np = pages_of(b0);
            const int p_tok = b0 == 0 ? tok0 : (b < a.B ? check(b) : 0);
            int t1, t2;
            const int off = base + block_scan(np, t1);
            const int nc = np > 0 ? seg_pieces(sstart, w, off, np, small) : 0;
            const int g0 = gbase + block_scan(nc, t2);
            if (b < a.B) a.plan_nc[b] = nc;
            if (by_seg) {
                if (b < a.B) {
                    soff[b] = off;
                    sg0[b] = g0;
                    skf[b] = np > 0 ? seg_find(sstart, w, off) : 0;
                    stok[b] = p_tok;
                }
                base += t1;
                gbase += t2;
                continue;
            }
            int c = 0;
            for (int q0 = off, k = np > 0 ? seg_find(sstart, w, off) : w; q0 < off + np && k < w; ++k) {
                const int ks = sstart[k], se = min(off + np, sstart[k + 1]);
                for (int q = q0; q < se; q += 64) {
                    const int n = min(64, se - q);
                    const bool first = q == ks;
                    const int slot = first ? k : W + g0 + c - (k + 1);
                    if (slot < a.plan_cap) plan[slot] = make_int4(b, c | (n << 16), p_tok, (q - off) * a.page);
                    if (first) sfirst[k] = g0 + c;
                    ++c;
                }
                q0 = max(q0, se);
            }
            base += t1;
            gbase += t2;
        }
        if (by_seg) {
            if (tid == 0) soff[a.B] = base;  // = P
            __syncthreads();
            for (int k = tid; k < w; k += 1024) {
                const int q_end = sstart[k + 1];
                int q = sstart[k];
                // the stream that holds page q: the last b with soff[b] <= q (its pages
                // reach past q)
                int lo = 0, hi = a.B - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (soff[mid] <= q) lo = mid; else hi = mid - 1;
                }
                for (int b = lo; q < q_end; ++b) {
                    if (soff[b + 1] <= q) continue;  // a stream without pages
                    const int se = min(q_end, soff[b + 1]);
                    const int c = k - skf[b];  // its pieces: one per segment from skf[b] on
                    const int g = sg0[b] + c;
                    const bool first = q == sstart[k];
                    const int slot = first ? k : W + g - (k + 1);
                    if (slot < a.plan_cap) plan[slot] = make_int4(b, c | ((se - q) << 16), stok[b], (q - soff[b]) * a.page);
                    if (first) sfirst[k] = g;
                    q = se;
                }
            }
        }
        __syncthreads();  // sfirst is complete
        for (int k = tid; k < W; k += 1024) {
            if (k < w) {
                const int gk = sfirst[k], gn = k + 1 < w ? sfirst[k + 1] : gbase;
                a.seg_cont[k] = make_int2(gk - k, gn - gk - 1);
            } else {
                a.seg_cont[k] = make_int2(0, 0);
                plan[k] = make_int4(0, 0, 0, 0);  // an empty segment: no pages
            }
        }
        n_entries = min(W + gbase - w, a.plan_cap);
        info = w;
    }
    // page ids of every entry's piece, one per lane of the attention wave (clamped into the
    // stream's page-table row); the entries written above are visible after the barrier.
    // Four entries per thread and round, every load requested before any store: a round
    // is two dependent loads (the entry, then its page id), not eight.
    __syncthreads();
    const int n_ids = n_entries * 64;
    for (int idx0 = tid; idx0 < n_ids; idx0 += 4 * 1024) {
        int row[4], pg[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = min(idx0 + u * 1024, n_ids - 1);
            const int4 e = plan[idx >> 6];
            row[u] = a.shared ? 0 : e.x;
            pg[u] = min(e.w / a.page + (idx & 63), a.max_pages - 1);
        }
        int id[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) id[u] = a.page_table[(int64_t)row[u] * a.max_pages + pg[u]];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (idx0 + u * 1024 < n_ids) a.plan_pages[idx0 + u * 1024] = id[u];
    }
    if (tid == 0) {
        plan_n[0] = n_entries;
        plan_n[1] = info;
    }
}

void launch_decode_plan(const DecodeAttnArgs &a, hipStream_t s) {
    if (a.B <= 0) return;
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, s, a, const_cast<int4 *>(a.plan),
                       const_cast<int *>(a.plan_n));
}

// One pass of the chunk merge over chunks c0 .. c0 + n - 1 (n <= CB): lane c loads
// (m_c, l_c), and the accumulators arrive as 16-byte loads -- lane l takes dims
// 4(l % 32) .. +3 of the chunks of parity l / 32 -- so a pass is one round of CB / 2 loads
// per lane; the maximum and the weights come from wave reductions, each half-wave adds
// its chunks in chunk order and rescales the running sums of earlier passes (the two
// halves are added at the end).
template <int CB>
__device__ __forceinline__ void combine_pass(const float *part, int c0, int n, int lane, float &M, float &lsum,
                                             float (&acc)[4]) {
    const int half = lane >> 5, d4 = (lane & 31) * 4;
    const int cl = c0 + min(lane, n - 1);  // clamped: unconditional loads
    const float ml = part[(int64_t)cl * PART_STRIDE], ll = part[(int64_t)cl * PART_STRIDE + 1];
    float4 x[CB / 2];
#pragma unroll
    for (int u = 0; u < CB / 2; ++u)
        x[u] = *reinterpret_cast<const float4 *>(part + (int64_t)(c0 + min(2 * u + half, n - 1)) * PART_STRIDE + 4 + d4);
    __builtin_amdgcn_sched_barrier(0);
    const float mn = fmaxf(M, wave_max(lane < n ? ml : -INFINITY));
    const float sc = exp2f(M - mn);  // 0 on the first pass (M = -inf)
    const float wl = lane < n ? exp2f(ml - mn) : 0.f;  // 0 past the pass's chunks
    lsum = lsum * sc + wave_sum(wl * ll);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < CB / 2; ++u) {
        if (2 * u >= n) break;
        const float w0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), 2 * u));
        const float w1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), 2 * u + 1));
        const float w = half ? w1 : w0;
        acc[0] += w * x[u].x;
        acc[1] += w * x[u].y;
        acc[2] += w * x[u].z;
        acc[3] += w * x[u].w;
    }
    M = mn;
}

// Merge of the piece partials of one (stream, head), in piece (position) order: one pass
// of up to 32 partials, or passes of 64 for streams split into more, so a stream of up to
// 64 pieces costs one round of loads.
template <typename TO>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeAttnArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int item = blockIdx.x * 4 + wave;
    if (item >= a.B * a.H) return;
    const int h = item % a.H, b = item / a.H;
    const int nc = a.plan_nc[b];  // the stream's pieces (partials), from the work list
    if (nc <= 0) {  // a token outside the cache (flagged by the plan) has no chunks: zeros
        if (lane < 32) {
            const int k = h * 128 + lane * 4;
            TO *out = reinterpret_cast<TO *>(a.out) + (a.out_mt > 0 ? frag_index(b, k, a.out_mt) : (int64_t)b * a.H * 128 + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = from_f32<TO>(0.f);
        }
        return;
    }
    const float *part = a.part + ((int64_t)b * a.H + h) * a.part_stride * PART_STRIDE;
    float M = -INFINITY, lsum = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (nc <= 32) {
        combine_pass<32>(part, 0, nc, lane, M, lsum, acc);
    } else {
        for (int c0 = 0; c0 < nc; c0 += 64) combine_pass<64>(part, c0, min(64, nc - c0), lane, M, lsum, acc);
    }
    // odd chunks (upper half-wave) onto even ones: chunk order within each parity, then
    // the two parities
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], 32, WAVE);
    const float inv = 1.0f / lsum;
    if (lane < 32) {
        const int k = h * 128 + lane * 4;  // fragment-major: 4 contiguous columns either way
        TO *out = reinterpret_cast<TO *>(a.out) + (a.out_mt > 0 ? frag_index(b, k, a.out_mt) : (int64_t)b * a.H * 128 + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = from_f32<TO>(acc[e] * inv);
    }
}

void launch_decode_attn(const DecodeAttnArgs &a, DType dt, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.B <= 0) return;
    const int group = a.H / a.Hkv;
    int items = a.B * a.Hkv * a.n_chunks;  // at most; the work list holds the real ones
    if (a.target_items > 0 && a.target_items < items) items = a.target_items;  // the list's budget
    if (a.target_items > 0 && !a.direct) items = a.n_seg * a.Hkv;  // one wave per segment and KV head
    const dim3 grid((items + 3) / 4), block(256);
    auto go = [&](auto kernel) {
        if (ev0 || ev1) hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev0, ev1, 0, a);
        else hipLaunchKernelGGL(kernel, grid, block, 0, s, a);  // plain launch (graph capture)
    };
    const bool fused = a.qkv != nullptr && !a.shared;
    auto pick = [&](auto t, auto g) {
        using T = decltype(t);
        constexpr int G = decltype(g)::value;
        if (a.direct) fused ? go(decode_attn_kernel<T, G, true, true>) : go(decode_attn_kernel<T, G, false, true>);
        else fused ? go(decode_attn_kernel<T, G, true, false>) : go(decode_attn_kernel<T, G, false, false>);
    };
    if (dt == DT_BF16) {
        if (group == 2) pick(bf16_t(), std::integral_constant<int, 2>());
        else pick(bf16_t(), std::integral_constant<int, 1>());
    } else {
        if (group == 2) pick(float(), std::integral_constant<int, 2>());
        else pick(float(), std::integral_constant<int, 1>());
    }
}

void launch_decode_combine(const DecodeAttnArgs &a, DType dt, hipStream_t s) {
    if (a.B <= 0) return;
    const dim3 grid((a.B * a.H + 3) / 4);
    if (dt == DT_BF16) hipLaunchKernelGGL(decode_combine_kernel<bf16_t>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(decode_combine_kernel<float>, grid, dim3(256), 0, s, a);
}

}  // namespace ttsbb
