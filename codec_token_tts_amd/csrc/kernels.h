// Launchers of the ttsbb kernels (host-callable, implemented in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttsbb {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// Device-side index check codes (OR-ed into the context flag).
enum : int { FLAG_CODE = 1, FLAG_TEXT_ID = 2, FLAG_PAGE = 4, FLAG_POSITION = 8, FLAG_NONFINITE = 16 };

// Domains (word 2 of the Philox counter) of the sampler's draws.
enum : uint32_t { RNG_CLASS = 1, RNG_POS = 2 };

// ---- K1: gather-sum codebook embedding ------------------------------------------
// Row r (< n_rows) is a text row if (is_text ? is_text[r] : r < text_prefix); text rows
// copy text_table[text_ids[r]].  Audio rows sum over k < n_cb the table row
// k*cb_vocab + codes[(r - audio_row0)*code_row_stride + k*code_cb_stride].
struct EmbedArgs {
    int n_rows, n_cb, hidden;
    const int32_t *codes;
    int code_row_stride, code_cb_stride, audio_row0;
    const void *tables;
    int cb_vocab;
    const uint8_t *is_text;
    int text_prefix;
    const int32_t *text_ids;
    const void *text_table;
    int text_vocab;
    float *out;
    int *flag;
};
void launch_embed(const EmbedArgs &a, DType dt, hipStream_t s);

// ---- K2: RMSNorm of fp32 rows into the operand dtype ------------------------------
// Optional deferred residual update first: with n_pend > 0, row r of x becomes
// x[r] + pend[0][r] + ... + pend[n_pend-1][r] (summed in that order; pend rows are
// pend_ld floats apart, splits pend_stride apart) and is written back.  gain == nullptr
// applies the update only (out unused).
// out_mt > 0: out (bf16) in the fragment-major layout with out_mt 16-row tiles
void launch_rmsnorm(float *x, int ldx, int rows, int hidden, const float *gain, float eps,
                    void *out, DType out_dt, hipStream_t s, const float *pend = nullptr, int n_pend = 0,
                    int64_t pend_ld = 0, int64_t pend_stride = 0, int out_mt = 0);

// ---- K3: projections  Y[M][N] = A[M][K] * W[N][K]^T with an epilogue --------------
enum Epi { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };
struct WSrc {
    // EPI_STORE / EPI_ADD: logical row n lives in p[i] for start[i] <= n < start[i+1]
    //   (start[0] = 0, nseg <= 3 segments, start[nseg] = N).
    // EPI_SWIGLU: p[0] = W_gate, p[1] = W_up, each [N/2][K]; logical rows interleave 16
    //   gate rows and 16 up rows; the output has N/2 columns silu(gate) * up.
    const void *p[3];
    int start[4];
    int nseg;
};
struct GemmArgs {
    const void *A;  // [M][lda] operand dtype
    int lda, M, K, N;
    WSrc w;
    void *C;        // EPI_STORE / EPI_ADD: fp32 [M][ldc]; EPI_SWIGLU: operand dtype [M][ldc]
    int ldc;
    int epi;
    // Fused RMSNorm (GEMV path only: M <= 8 rows in bf16 mode, any M in fp32 mode): when nx
    // is set, A is RMSNorm(nx rows, fp32 [M][K]) * ng (eps neps) instead of g.A
    const float *nx;
    const float *ng;
    float neps;
    // Skinny path only (8 < M <= 64, bf16): A (a_mt > 0) and, for EPI_SWIGLU, C (c_mt > 0)
    // are in the fragment-major layout of frag_index() with that many 16-row tiles (the
    // kernel's own: 1, 2 or 4) instead of row-major
    int a_mt, c_mt;
    // launch_head_scores only: groups of gv columns (a head of gv classes per group)
    int gv, gmask;
    float4 *spart;
};
// part: fp32 workspace of part_cap floats for split-K partial sums.  Returns the number
// of K splits whose partial sums are left in part[z][M][N] for the caller to add (an
// EPI_ADD product on the skinny path defers its residual update to the next RMSNorm,
// which sums them in split order); 0 when C holds the result.
int launch_gemm(const GemmArgs &g, DType dt, float *part, int64_t part_cap, hipStream_t s);
// 16-row tiles (1, 2 or 4) of the skinny kernel that a bf16 product of this shape runs on,
// or 0 when it runs elsewhere (the fragment-major layout is only for that kernel)
int skinny_tiles(const GemmArgs &g, int64_t part_cap);

// Head product + MaskGIT scoring statistics (bf16, M > 64, K % 64 == 0): the logits
// Y = A W^T are never stored; for every row m and every 128-column tile j, each group of
// g.gv columns that meets the tile gets its partial statistics over the tile's columns
//   spart[(m * ceil(N / 128) + j) * 2 + s] = (max over all classes, sum of exp(y - max),
//                                             best class value, its class id as int bits)
// with s = group - (first group of the tile), s in {0, 1} (a group of >= 128 columns
// meets a tile in at most two groups); the best excludes class g.gmask (ties: lowest id).
// Returns false (nothing launched) when the shape is not taken.
bool launch_head_scores(const GemmArgs &g, hipStream_t s);

// ---- K4: per-head RMSNorm + RoPE + K/V write --------------------------------------
// qkv fp32 [M][(H + 2 Hkv) * 128].  Decode mode (dense == 0): row m is stream m at
// position pos[m]; K/V go to pool slot (page_table[m][p / page], p % page); q goes to
// q_out fp32 [M][H*128].  Dense mode: row m is position m; q goes to q_out bf16
// [M][H*128], K to kbuf [Hkv][s_pad][128] and V transposed to vtbuf [Hkv][128][s_pad].
struct RopeKvArgs {
    const float *qkv;
    int M, H, Hkv;
    const float *q_gain, *k_gain;
    float eps;
    const float2 *rope;  // [max_pos][64] (cos, sin)
    int max_pos;
    void *q_out;
    int dense;
    const int32_t *pos;
    const int32_t *page_table;
    int max_pages, n_pages, page;
    void *pool_layer;    // [n_pages][2][Hkv][page][128]
    uint16_t *kbuf, *vtbuf;
    int s_pad;
    int *flag;
    int shared;          // decode mode, prefill of one stream: row m is at position pos[0] + m
                         // and every row uses page-table row 0
    int seg1;            // dense mode, two sequences: rows m >= seg1 > 0 are at position m - seg1
    int q_bf16;          // decode mode: q_out gets bf16 rows (as in dense mode) instead of fp32
    int dense_f32;       // dense mode in fp32: q_out fp32 [M][H*128], K and V rows fp32
                         // [Hkv][s_pad][128] in kbuf and vtbuf (V not transposed)
    int dense_copy;      // shared-row (prefill) mode, bf16: also the dense K rows [Hkv][s_pad][128]
                         // and V^T [Hkv][128][s_pad] of positions [0, pos[0] + M) -- the prompt's
                         // from its own rows, the cached prefix copied from the pool by extra
                         // workgroups of the same launch -- for the causal flash kernel
};
void launch_rope_kv(const RopeKvArgs &a, DType kv_dt, hipStream_t s);
// Dense mode fused into the q/k/v projection (g: EPI_STORE product of N = (H + 2 Hkv) *
// 128 columns): writes q_out / kbuf / vtbuf directly, qkv is not written.  Returns
// false (nothing launched) when the shape is not taken by the fused kernel (M <= 64).
bool launch_qkv_dense(const GemmArgs &g, const RopeKvArgs &rk, hipStream_t s);


// ---- K5: split-sequence decode attention over the paged pool -----------------------
constexpr int SEG_MAX = 2048;  // most work-list segments of a q_len = 1 decode step

struct DecodeAttnArgs {
    const float *q;  // [B][H*128] fp32
    void *pool_layer;     // [n_pages][2][Hkv][page][128] (written only by the fused step-token path)
    const int32_t *pos;
    const int32_t *page_table;
    int max_pages, n_pages, page;
    int B, H, Hkv;
    int chunk, n_chunks;  // least positions per chunk (multiple of page), most chunks per stream
    int part_stride;      // chunks per (stream, head) in part: >= n_chunks
    // The step's work list (launch_decode_plan).  An entry is one piece of a stream's
    // cached positions: (stream, piece index | pages << 16, token position, first
    // position); plan_pages [plan_cap][64] holds its page ids (one per lane).  A stream's
    // pieces are numbered 0 .. plan_nc[b] - 1 in position order (its partials).
    //  * target_items == 0 (prefill rows): each stream cut into equal page-aligned pieces
    //    of at most `chunk` positions, one wave each, entries 0 .. plan_n[0] - 1 in stream
    //    order; plan_cap >= B * n_chunks.
    //  * target_items > 0 (q_len = 1 decode): up to n_seg (even) segments of the streams'
    //    pages laid end to end; segments that average 8 pages or more are weighted 9 : 8
    //    between even and odd ones, shorter ones are equal.  Segment k runs on workgroups
    //    of parity k & 1, i.e. on the even or the odd XCDs (workgroup b runs on XCD b mod
    //    8, and the odd XCDs stream ~10% slower).  A piece
    //    is a stream's part of a segment (at most 64 pages): entry k < n_seg is segment
    //    k's first piece (0 pages: empty), its further pieces are entries n_seg +
    //    seg_cont[k].x + j, j < seg_cont[k].y.  part_stride >= n_chunks + 2 and
    //    plan_cap >= B * part_stride + n_seg.
    const int4 *plan;
    const int *plan_n;
    int *plan_pages;
    int plan_cap;
    int target_items;
    int n_seg;            // <= SEG_MAX
    int2 *seg_cont;       // [n_seg]
    int *plan_nc;         // [B]
    // Direct mode (q_len = 1 decode whose caches fit one chunk: max_pages * page <= chunk):
    // one item per (stream, KV head) over its whole cache, positions and page ids read from
    // pos / page_table (no work list), the output rows written by the attention kernel
    // itself (no partials, no merge; zero rows for a negative position), FLAG_POSITION
    // raised by it.
    int direct;
    float *part;          // [B][H][part_stride][132]: m, l, pad, pad, acc[128]
    void *out;            // [B][H*128] operand dtype (out_mt > 0: bf16, fragment-major)
    int out_mt;
    float scale_log2;     // log2(e) / sqrt(128)
    int shared;           // prefill of one stream: query b is at position pos[0] + b and
                          // every query reads page-table row 0 (causal by construction)
    // Fused step-token preparation (q_len = 1 decode, shared == 0): when qkv is set, q is
    // the per-head RMSNorm + RoPE of the raw projections qkv [B][(H + 2 Hkv) * 128] (the
    // q field is not read), and the wave owning each stream's last chunk writes the
    // token's normed + rotated K and its V to the pool slot of position pos[b] and uses
    // them from registers; it raises FLAG_PAGE as the separate kernel does (FLAG_POSITION
    // is raised by the plan kernel).
    const float *qkv;
    const float *q_gain, *k_gain;
    const float2 *rope;   // [max_pos][64] (cos, sin)
    float eps;
    int max_pos;
    int *flag;
};
// ev0 / ev1 (optional): events stamped with the kernel's own start and end
void launch_decode_attn(const DecodeAttnArgs &a, DType dt, hipStream_t s, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);
void launch_decode_combine(const DecodeAttnArgs &a, DType dt, hipStream_t s);
// Builds a.plan / a.plan_n from the positions (one launch per step, before the layers).
void launch_decode_plan(const DecodeAttnArgs &a, hipStream_t s);

// ---- K6: bidirectional flash attention (bf16 MFMA) ---------------------------------
struct FlashArgs {
    const uint16_t *q;   // [S][H*128] bf16
    const uint16_t *k;   // [Hkv][s_pad][128] bf16
    const uint16_t *vt;  // [Hkv][128][s_pad] bf16
    int S, s_pad, H, Hkv;
    float scale_log2;
    uint16_t *out;       // [S][H*128] bf16
    // Two independent sequences in one launch (seg1 > 0, a multiple of 32): rows [0, len0)
    // attend to keys [0, len0), rows [seg1, seg1 + len1) to keys [seg1, seg1 + len1); rows
    // between len0 and seg1 are padding.  seg1 == 0: one sequence, len0 = S.
    int seg1, len0, len1;
    // Causal (non-null, seg1 == 0): row i is at position p0 + i, p0 = causal_pos[0] read on
    // the device and clamped to [0, s_pad - S]; it attends to keys [0, p0 + i].
    const int32_t *causal_pos;
};
void launch_flash_attn(const FlashArgs &a, hipStream_t s);

// The same attention in fp32 (an fp32 context's MaskGIT pass): q [S][H*128], K and V rows
// [Hkv][s_pad][128] (V not transposed), out [S][H*128], all fp32; seg1 / len0 / len1 as
// above; scale = 1 / sqrt(128).
struct AttnF32Args {
    const float *q, *k, *v;
    int S, s_pad, H, Hkv;
    float scale;
    float *out;
    int seg1, len0, len1;
};
void launch_attn_f32(const AttnF32Args &a, hipStream_t s);

// ---- K7: greedy choice per group --------------------------------------------------
// A group holding a NaN raises FLAG_NONFINITE (its choice: the argmax of its other values,
// or 0 when all are NaN).
void launch_argmax_groups(const float *logits, int rows, int ld, int n_groups, int group_vocab,
                          int32_t *out, int *flag, hipStream_t s);

// ---- K8: MaskGIT scores: log-softmax, mask class excluded, argmax, confidence --------
// logits [T][ld] (flat k*V + v per row).  With logits_u (same layout) the scored logits
// are the guided c + cfg_scale * (c - u).  codes: element (k, t) at codes[k*codes_ld + t].
// A group whose log-softmax is undefined (a NaN or an infinite logit) raises
// FLAG_NONFINITE, predicts the lowest non-mask class and scores -inf.
void launch_maskgit_scores(const float *logits, const float *logits_u, float cfg_scale, int T, int ld,
                           int n_cb, int V, int mask_id, float penalty, const int32_t *codes, int codes_ld,
                           int32_t *pred, float *conf, int *flag, hipStream_t s);

// The same scores from the head's partial statistics (launch_head_scores, ld = the head
// width N): the group's tiles are merged in tile order into max, sum of exp, best class.
void launch_maskgit_merge(const float4 *spart, int T, int N, int n_cb, int V, int mask_id, float penalty,
                          const int32_t *codes, int codes_ld, int32_t *pred, float *conf, int *flag,
                          hipStream_t s);

// With the sampler: class_temp > 0 keeps the k_keep best log-probs of each group and
// adds Gumbel noise from u_class [n_cb][T][V]; pos_temp > 0 adds noise from u_pos
// [n_cb][T] to the score.  A NULL array draws its uniforms from Philox4x32-10 (key
// seed, blocks from *counter on, domains RNG_CLASS / RNG_POS).  V <= SAMPLE_MAXV (2048).
void launch_maskgit_sample(const float *logits, const float *logits_u, float cfg_scale, int T, int ld, int n_cb,
                           int V, int mask_id, float penalty, const int32_t *codes, int codes_ld, float class_temp,
                           float pos_temp, int k_keep, const float *u_class, const float *u_pos, uint64_t seed,
                           const uint64_t *counter, int32_t *pred, float *conf, int *flag, hipStream_t s);
// out[4 i + j] = word j of Philox4x32-10(counter (lo, hi of block0 + i, w2, w3), key (lo, hi
// of seed)), i < n_blocks.
void launch_rng_words(uint64_t seed, uint64_t block0, uint32_t w2, uint32_t w3, int n_blocks, uint32_t *out,
                      hipStream_t s);
// *ctr += n on the device (one thread).
void launch_advance_counter(uint64_t *ctr, uint64_t n, hipStream_t s);

// ---- K9: top-n selection by rank + code update -------------------------------------
// rank: int32 scratch [n], all zero on entry, left all zero (the context zeroes it once)
// Top-n over conf [n_cb][T] (flat k*T + t); picked codes go to codes[k*codes_ld + t].
void launch_select_update(const float *conf, const int32_t *pred, int n_cb, int T, int n_unmask,
                          int32_t *rank, int32_t *codes, int codes_ld, int32_t *picked, hipStream_t s);

// ---- codec RVQ decode (fp32) -----------------------------------------------------------
struct RvqArgs {
    int n_frames, n_q, cb_size, dim, out_dim;
    const int32_t *codes;  // [n_q][n_frames]
    const float *embed;    // [n_q][cb_size][dim]
    const float *proj_w;   // [n_q][out_dim][dim]
    const float *proj_b;   // [n_q][out_dim]
    float *out;            // [n_frames][out_dim]
    int *flag;
};
// ev0 / ev1 (optional): events stamped with the kernel's own start and end
void launch_rvq_decode(const RvqArgs &a, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// ---- misc ---------------------------------------------------------------------------
void launch_increment(int32_t *v, int n, hipStream_t s, int delta = 1);  // v[i] += delta, i < n
// dst[i0][i1][i2] (fp32, dense) = src[i0*s0 + i1*s1 + i2*s2] (element strides)
void launch_tap_copy(const void *src, DType dt, int64_t s0, int64_t s1, int64_t s2, int d0,
                     int d1, int d2, float *dst, hipStream_t s);

}  // namespace ttsbb
