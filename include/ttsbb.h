/* ttsbb — forward pass of a Qwen3-0.6B-shaped TTS backbone on AMD MI355X (gfx950).
 *
 * Plain C99 interface (extern "C"), opaque context, integer status codes with 0 = OK
 * and negative values for errors.  Every tensor argument of a compute call is a
 * DEVICE pointer owned by the caller; the library never frees it.  Calls enqueue work
 * on the stream given at creation and return without synchronising, so a sequence
 * of calls can be captured into a HIP graph.  Argument errors are found on the host
 * before anything is enqueued; out-of-range indices met on the device (a code, a
 * page id, a position) are clamped away from memory and raise a device flag that
 * ttsbb_sync() reports.
 *
 * The model (OmniVoice ARCHITECTURE, "Qwen3 0.6B backbone with custom IO" and "GGUF
 * layout"; ncnn Qwen3-TTS port, "模型结构拆解"): pre-norm decoder layers
 *   h  = RMSNorm(x; g_attn)                      input_layernorm
 *   q,k,v = Wq h, Wk h, Wv h                     no biases
 *   q,k = per-head RMSNorm(g_q / g_k), then half-rotate RoPE at the token position
 *   o  = softmax(q k^T / sqrt(head_dim)) v       GQA: query head h reads KV head h / (H/H_kv)
 *   x1 = x + Wo o
 *   x2 = x1 + Wd (silu(Wg h2) * Wu h2),  h2 = RMSNorm(x1; g_ffn)   SwiGLU, no biases
 * with RMSNorm(x; g) = x / sqrt(mean(x^2) + eps) * g and RoPE pairing dimension j with
 * j + head_dim/2 at angle pos * theta^(-2j/head_dim) (ncnn port, "mRoPE结论").
 * Supported shapes: head_dim 128, hidden and ffn multiples of 128 (hidden at most 4096),
 * n_heads a multiple of n_kv_heads with group size 1 or 2.
 *
 * Precision: in TTSBB_BF16 mode the weights, embedding tables, heads, KV cache and the
 * operands of every matrix product are bf16; the residual stream, all accumulations,
 * norms and softmax statistics are fp32.  In TTSBB_F32 mode everything is fp32.
 */
#ifndef TTSBB_H
#define TTSBB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ttsbb_ctx ttsbb_ctx;

typedef enum {
    TTSBB_OK = 0,
    TTSBB_INVALID_ARG = -1,   /* NULL where a pointer is required, a size out of range */
    TTSBB_UNSUPPORTED = -2,   /* a shape or mode these kernels do not implement */
    TTSBB_OOM = -3,           /* device memory could not be allocated (create only) */
    TTSBB_DEVICE_ERROR = -4   /* a HIP call failed, or a device-side index check fired */
} ttsbb_status;

typedef enum { TTSBB_F32 = 0, TTSBB_BF16 = 1 } ttsbb_dtype;

/* Model shape and workspace limits.  Fill with ttsbb_default_config() first. */
typedef struct {
    int32_t n_layers;      /* decoder layers (0 is allowed: embedding -> final norm -> head) */
    int32_t hidden;        /* 1024 */
    int32_t n_heads;       /* 16 query heads */
    int32_t n_kv_heads;    /* 8 KV heads */
    int32_t head_dim;      /* 128 */
    int32_t ffn;           /* 3072 */
    float rms_eps;         /* 1e-6, all norms */
    double rope_theta;     /* 1e6 */
    int32_t dtype;         /* ttsbb_dtype of weights, tables, heads, KV cache */
    int32_t kv_page;       /* tokens per KV page: 16 */
    int32_t max_rows;      /* most tokens in one call (decode batch, MaskGIT sequence) */
    int32_t max_pos;       /* RoPE positions 0..max_pos-1 are usable */
    int32_t max_head_cols; /* widest head (n_groups * group_vocab) any call will use */
} ttsbb_config;

/* Borrowed device pointers of one layer; they must outlive the context.
 * Gains are fp32 vectors; linear weights are [out][in] row-major in cfg.dtype:
 * wq [H*d][hidden], wk and wv [Hkv*d][hidden], wo [hidden][H*d],
 * w_gate and w_up [ffn][hidden], w_down [hidden][ffn]. */
typedef struct {
    const float *attn_norm; /* [hidden] */
    const float *q_norm;    /* [head_dim] */
    const float *k_norm;    /* [head_dim] */
    const float *ffn_norm;  /* [hidden] */
    const void *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
} ttsbb_layer;

/* Qwen3-0.6B backbone defaults (OmniVoice ARCHITECTURE, "GGUF layout"): 28 layers,
 * hidden 1024, 16/8 heads of 128, ffn 3072, eps 1e-6, theta 1e6, bf16, 16-token pages. */
void ttsbb_default_config(ttsbb_config *cfg);

/* Create a context on the current HIP device (OmniVoice ARCHITECTURE, "Public API": one
 * opaque handle per pipeline, one init and one free; "ABI guarantee": plain C99,
 * extern "C", only the prefixed symbols exported).  `layers` holds cfg->n_layers entries
 * (copied; the pointers inside are borrowed).  `final_norm` is the fp32 [hidden] gain
 * of the last RMSNorm (llm.norm); it may be NULL only if no call uses a head.
 * `hip_stream` is a hipStream_t (NULL = the null stream).  Allocates the workspace
 * (sized by max_rows, max_pos, max_head_cols) and the fp32 RoPE cos/sin table, which
 * is computed on the host in double precision.  Returns TTSBB_OOM if that fails. */
ttsbb_status ttsbb_create(const ttsbb_config *cfg, const ttsbb_layer *layers,
                          const float *final_norm, void *hip_stream, ttsbb_ctx **out);

/* Free a context (OmniVoice ARCHITECTURE, "Public API": the one free of the handle):
 * waits for its stream, then releases the workspace.  NULL is a no-op; the weights and
 * every caller buffer stay the caller's. */
void ttsbb_destroy(ttsbb_ctx *ctx);

/* Static text of a status code (OmniVoice ARCHITECTURE, "Public API": status codes, 0
 * for success and negative values for failures). */
const char *ttsbb_status_str(ttsbb_status s);

/* Wait for the context's stream; report (and clear) the device-side flag: an index out
 * of range (a code, a text id, a page id, a position) or a head output without an order
 * (a NaN, or an infinite logit in a MaskGIT group).  Returns TTSBB_DEVICE_ERROR for a
 * failed wait or a raised flag (OmniVoice ARCHITECTURE, "Public API": a failed generate
 * is reported by status). */
ttsbb_status ttsbb_sync(ttsbb_ctx *ctx);

/* Summed codebook embedding (OmniVoice ARCHITECTURE, "Qwen3 0.6B backbone with custom
 * IO": rows k*cb_vocab + code of a flattened [n_cb*cb_vocab][hidden] table, summed over
 * the n_cb codebooks; ncnn port, "模型结构拆解": the frame's codebook embeddings are
 * summed into the next input).
 *   out[r] = sum_{k<n_cb} tables[k*cb_vocab + codes[r*n_cb + k]]      (audio rows)
 *   out[r] = text_table[text_ids[r]]               (rows with is_text[r] != 0)
 * codes int32 [n_rows][n_cb]; tables cfg.dtype; is_text uint8 [n_rows] or NULL (all
 * audio); text_ids int32 [n_rows] and text_table [text_vocab][hidden] needed only if
 * is_text is given; out fp32 [n_rows][hidden].  The sum is formed in double precision
 * in codebook order and rounded once to fp32.  n_rows may be 0 (no work). */
ttsbb_status ttsbb_codebook_embed(ttsbb_ctx *ctx, int32_t n_rows, int32_t n_cb,
                                  const int32_t *codes, const void *tables, int32_t cb_vocab,
                                  const uint8_t *is_text, const int32_t *text_ids,
                                  const void *text_table, int32_t text_vocab, float *out);

/* One q_len=1 decode step of every layer for `batch` independent streams (ncnn port,
 * "单token SDPA问题与host attention": RoPE + KV append + GQA attention per layer).
 *   x          fp32 [batch][hidden], in: the embedded token; out: the residual stream
 *              after the last layer (before the final norm).
 *   positions  int32 [batch], in: the position of this token = tokens already cached;
 *              incremented by one on the device at the end of the call.
 *   page_table int32 [batch][max_pages]: pool page of each kv_page-token block.
 *   kv_pool    cfg.dtype [n_layers][n_pages][2 (K, V)][n_kv_heads][kv_page][head_dim];
 *              K is stored normalised and rotated.  The token's K and V are written at
 *              (page_table[b][p / kv_page], p % kv_page) before it attends to 0..p.
 *   head       optional [n_groups*group_vocab][hidden] (cfg.dtype): if not NULL the
 *              final RMSNorm and the head are applied and argmax int32 [batch][n_groups]
 *              receives the greedy class of each group (ties: lowest id).
 *   logits     optional fp32 [batch][n_groups*group_vocab] copy of the head output.
 *              A group holding a NaN raises the device flag; its choice is the argmax
 *              of its other values, or class 0 if all are NaN.
 * Positions outside [0, max_pages*kv_page) or page ids outside [0, n_pages) raise the
 * device flag and skip the write; a stream whose position is negative attends to
 * nothing (its attention output is zero). */
ttsbb_status ttsbb_decode_step(ttsbb_ctx *ctx, int32_t batch, float *x, int32_t *positions,
                               const int32_t *page_table, int32_t max_pages, void *kv_pool,
                               int32_t n_pages, const void *head, int32_t n_groups,
                               int32_t group_vocab, int32_t *argmax, float *logits);

/* ttsbb_decode_step for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): same arguments,
 * kernels and results, but every per-call scratch buffer of the step (normalised and
 * projected rows, attention work list and partial sums, split products' partial sums,
 * the head logits when `logits` is NULL) lives in one static device array of the
 * library, 32 MiB on each GPU it runs on, held until the process ends, instead of the
 * context's workspace.  It allocates nothing.  Limits: batch <= 64 streams and
 * n_groups * group_vocab <= 8200 (TTSBB_UNSUPPORTED beyond; also if the context's shape
 * needs more scratch than the array holds); when batch * (ceil(max_pages * kv_page /
 * 128) + 2) > 2048 its attention may split the caches differently from
 * ttsbb_decode_step (the same result up to fp32 rounding order).  Every call of this entry point on one GPU shares
 * that GPU's array and leaves its contents behind: calls that overlap on one GPU (other
 * streams, contexts or threads) race. */
ttsbb_status ttsbb_decode_step_noalloc(ttsbb_ctx *ctx, int32_t batch, float *x, int32_t *positions,
                                       const int32_t *page_table, int32_t max_pages, void *kv_pool,
                                       int32_t n_pages, const void *head, int32_t n_groups,
                                       int32_t group_vocab, int32_t *argmax, float *logits);

/* Causal multi-token prefill of one stream (ncnn Qwen3-TTS port, "单token SDPA问题与host
 * attention": RoPE + KV append + GQA attention per layer; the Talker prompt and the code
 * predictor's two-token start are prefills): n_tokens embedded tokens at positions
 * cache_len[0] .. cache_len[0] + n_tokens - 1 run through every layer; each token's
 * rotated K and raw V are written to the stream's pages (page_table row, as in
 * ttsbb_decode_step) and token i attends to positions 0 .. cache_len[0] + i (the cached
 * prefix and the tokens before it).  x [n_tokens][hidden] fp32 is the embedded input and
 * the final residual stream on return; cache_len int32 [1] is advanced by n_tokens on the
 * device.  With head != NULL the final norm + head + argmax run on the last token only
 * (argmax [n_groups], logits [n_groups*group_vocab] if not NULL).  n_tokens <= max_rows.
 * bf16 contexts run a prefill of more than 64 tokens (no layer tapped) with the causal
 * form of the MaskGIT attention kernel over the stream's positions 0 .. cache_len[0] +
 * n_tokens - 1 read back from the pool (bf16 q and attention weights, as that kernel
 * keeps them); shorter ones attend token by token with the decode attention. */
ttsbb_status ttsbb_prefill(ttsbb_ctx *ctx, int32_t n_tokens, float *x, int32_t *cache_len,
                           const int32_t *page_table, int32_t max_pages, void *kv_pool, int32_t n_pages,
                           const void *head, int32_t n_groups, int32_t group_vocab, int32_t *argmax,
                           float *logits);

/* One MaskGIT step (OmniVoice ARCHITECTURE, "MaskGIT decoder" and "Inner-loop
 * optimisations"): embed n_text text tokens then n_frames audio frames (sum of n_cb
 * codebook rows, mask_id included as a code), run every layer with bidirectional
 * attention over all S = n_text + n_frames positions (RoPE positions 0..S-1, no cache),
 * apply the final RMSNorm and the per-codebook heads on the audio window only, then
 *   lp   = logits - logsumexp over the cb_vocab classes of codebook k
 *   pred = argmax over classes != mask_id (ties: lowest id)
 *   conf = lp[pred] - k * layer_penalty, or -inf where codes[k][t] != mask_id
 * and unmask the n_unmask highest conf over the flat index f = k*n_frames + t (ties:
 * lowest f): codes[f] = pred[f].  picked[r] is the flat index of rank r, or -1 where
 * fewer than r+1 positions were still masked.
 *   text_ids int32 [n_text]; text_table [text_vocab][hidden]; audio_tables and
 *   audio_heads [n_cb*cb_vocab][hidden] (cfg.dtype); codes int32 [n_cb][n_frames]
 *   in/out; pred int32 and conf fp32 [n_cb][n_frames]; picked int32 [n_unmask].
 * A bf16 context runs the MFMA kernels (bf16 storage, fp32 accumulation); an fp32 context
 * computes every step in fp32 (weight-streaming products and a plain fp32 attention
 * kernel: a reference mode for checking, not a fast path). */
ttsbb_status ttsbb_maskgit_pass(ttsbb_ctx *ctx, int32_t n_text, const int32_t *text_ids,
                                const void *text_table, int32_t text_vocab, int32_t n_frames,
                                int32_t n_cb, int32_t cb_vocab, int32_t mask_id,
                                const void *audio_tables, const void *audio_heads,
                                int32_t *codes, int32_t n_unmask, float layer_penalty,
                                int32_t *pred, float *conf, int32_t *picked);

/* One MaskGIT step with classifier-free guidance (OmniVoice ARCHITECTURE, "MaskGIT
 * decoder": the unconditional prompt is the trailing target tokens alone; the step
 * scores log_softmax(c + cfg_scale * (c - u))).  The last n_target of the n_frames audio
 * frames are the target window (the frames before it are reference audio, conditioning
 * only).  Two passes of every layer:
 *   conditional:   n_text text tokens + all n_frames frames, positions 0..S-1, logits c
 *                  on the window (the last n_target positions);
 *   unconditional: the window's n_target frames alone, positions 0..n_target-1, logits u;
 * then, with g = c + cfg_scale * (c - u), the scoring of ttsbb_maskgit_pass on g over the
 * window, and the update of the n_unmask best window positions.
 *   codes int32 [n_cb][n_frames] in/out (only the window changes); pred int32 and conf
 *   fp32 [n_cb][n_target]; picked int32 [n_unmask] holds flat window indices
 *   f = k*n_target + t (or -1); other arguments as in ttsbb_maskgit_pass.
 * When S rounded up to 64 plus n_target fits cfg.max_rows, the two prompts run as one
 * batch of two independent sequences (same results up to rounding order; fewer, larger
 * launches), else as two passes.
 * Requires 0 < n_target <= n_frames (bf16 or fp32 as ttsbb_maskgit_pass).  With taps on, the
 * per-layer taps and TTSBB_TAP_LOGITS come from the conditional pass (its rows lead the
 * batch), TTSBB_TAP_LOGITS_U holds u. */
ttsbb_status ttsbb_maskgit_pass_cfg(ttsbb_ctx *ctx, int32_t n_text, const int32_t *text_ids,
                                    const void *text_table, int32_t text_vocab, int32_t n_frames,
                                    int32_t n_target, int32_t n_cb, int32_t cb_vocab, int32_t mask_id,
                                    const void *audio_tables, const void *audio_heads, int32_t *codes,
                                    int32_t n_unmask, float layer_penalty, float cfg_scale, int32_t *pred,
                                    float *conf, int32_t *picked);

/* Arguments of the general MaskGIT step: those of ttsbb_maskgit_pass_cfg plus the
 * sampler (OmniVoice ARCHITECTURE, "MaskGIT decoder": keep_top_k_ratio, gumbel_sample with
 * the class temperature, Gumbel noise on the scores with the position temperature;
 * Determinism: a seedable Philox4x32-10 stream whose counter is threaded across calls).
 * The uniforms of the Gumbel noise come from the caller's arrays when given, else from
 * the library's Philox4x32-10 stream: uniform e of a call is
 *   ((w >> 9) + 0.5) * 2^-23,  w = word e % 4 of Philox4x32-10(counter = (lo, hi of
 *   *rng_counter + e / 4, domain, 0), key = (lo, hi of rng_seed))
 * with domain 1 and e = (k * n_target + t) * cb_vocab + v for the class noise, domain 2
 * and e = k * n_target + t for the position noise; ttsbb_philox_words exposes the
 * words.  The counter lives on the device and the call advances it there, so a captured
 * step replays with fresh draws. */
typedef struct {
    int32_t n_text;
    const int32_t *text_ids;     /* int32 [n_text] */
    const void *text_table;      /* [text_vocab][hidden] */
    int32_t text_vocab;
    int32_t n_frames, n_target;  /* audio frames; the last n_target are the target window */
    int32_t n_cb, cb_vocab, mask_id;
    const void *audio_tables, *audio_heads; /* [n_cb*cb_vocab][hidden] */
    int32_t *codes;              /* int32 [n_cb][n_frames], in/out (window only changes) */
    int32_t n_unmask;
    float layer_penalty;
    float cfg_scale;             /* 0: no unconditional pass */
    float class_temp;            /* > 0: top-k ratio filter + Gumbel noise on the classes */
    float pos_temp;              /* > 0: Gumbel noise on the scores */
    float top_k_ratio;           /* keeps max(1, floor(top_k_ratio * cb_vocab)) classes */
    const float *u_class;        /* fp32 [n_cb][n_target][cb_vocab] in (0,1), or NULL: drawn */
    const float *u_pos;          /* fp32 [n_cb][n_target] in (0,1), or NULL: drawn */
    int32_t *pred;               /* int32 [n_cb][n_target] */
    float *conf;                 /* fp32 [n_cb][n_target] */
    int32_t *picked;             /* int32 [n_unmask], flat window indices or -1 */
    uint64_t rng_seed;           /* Philox4x32-10 key of the drawn uniforms */
    uint64_t *rng_counter;       /* device uint64 [1], in/out: the first counter block of
                                    this call's draws; advanced on the device by
                                    ceil(n_cb * n_target * cb_vocab / 4) when the call
                                    draws anything.  Required if a needed array is NULL. */
} ttsbb_maskgit_step_args;

/* One MaskGIT step in general form: the passes of ttsbb_maskgit_pass_cfg (one pass when
 * cfg_scale == 0), g = c + cfg_scale * (c - u), then on the window
 *   lp   = g - logsumexp(g) over the cb_vocab classes; lp[mask_id] = -inf
 *   if class_temp > 0: keep the max(1, floor(top_k_ratio * cb_vocab)) largest lp (ties:
 *                      lowest id; the others -inf), lp = lp / class_temp + G(u_class)
 *   pred = argmax lp (ties: lowest id); conf = max lp - k * layer_penalty
 *   if pos_temp > 0:   conf += pos_temp * G(u_pos)
 *   conf = -inf where the code is already set
 * with G(u) = -log(-log(u)), and the top-n update of ttsbb_maskgit_pass_cfg.  All
 * pointers are device memory; cb_vocab <= 2048 when class_temp > 0. */
ttsbb_status ttsbb_maskgit_step(ttsbb_ctx *ctx, const ttsbb_maskgit_step_args *args);

/* The sampler's counter-based generator (OmniVoice ARCHITECTURE, "MaskGIT decoder",
 * Determinism: Philox4x32-10; Salmon, Moraes, Dror, Shaw, SC'11): out [n_blocks][4]
 * (device uint32) receives, for block i, the four words of Philox4x32-10 with counter
 * (lo, hi of block0 + i, word2, word3) and key (lo, hi of seed).  n_blocks may be 0. */
ttsbb_status ttsbb_philox_words(ttsbb_ctx *ctx, uint64_t seed, uint64_t block0, uint32_t word2, uint32_t word3,
                                int32_t n_blocks, uint32_t *out);

/* Codec RVQ decode (OmniVoice ARCHITECTURE, "Audio tokenizer pipeline", decode path; ncnn
 * Qwen3-TTS port, "Codec Decoder的切分"): for every frame t the sum over codebooks k of
 * the code's embedding projected by that codebook's project_out Linear,
 *   out[t][n] = sum_k ( sum_d embed[k][codes[k][t]][d] * proj_w[k][n][d] + proj_b[k][n] ),
 * in fp32 (the codec's quantizer precision).  The page then views out as [out_dim][T] for
 * the codec body (not part of this library).
 *   codes int32 [n_q][n_frames]; embed fp32 [n_q][codebook_size][codebook_dim];
 *   proj_w fp32 [n_q][out_dim][codebook_dim]; proj_b fp32 [n_q][out_dim];
 *   out fp32 [n_frames][out_dim].  All device pointers; a code outside
 *   [0, codebook_size) is clamped and raises the device flag (ttsbb_sync).  The sums run
 *   on the fp32 matrix cores when codebook_dim is a multiple of 8 and at most 64, n_q <= 32
 *   and embed and proj_w are 16-byte aligned; otherwise on the vector units (same result
 *   within fp32 rounding; the summation order differs from the formula's). */
ttsbb_status ttsbb_rvq_decode(ttsbb_ctx *ctx, int32_t n_frames, int32_t n_q, int32_t codebook_size,
                              int32_t codebook_dim, int32_t out_dim, const int32_t *codes, const float *embed,
                              const float *proj_w, const float *proj_b, float *out);

/* Host helper: how many positions each of n_steps MaskGIT steps unmasks (OmniVoice
 * ARCHITECTURE, "MaskGIT decoder": ceil(N * (t[i+1] - t[i])) over a time grid), on the
 * cosine grid t_i = 1 - cos(pi/2 * i/n_steps); each count is capped at what is left and
 * the last step takes the remainder.  out int32 [n_steps] is HOST memory. */
ttsbb_status ttsbb_unmask_schedule(int32_t n_total, int32_t n_steps, int32_t *out);

/* Debug taps: fp32 copies of one layer's intermediates from the next calls. */
typedef enum {
    TTSBB_TAP_X_IN = 0,    /* residual stream entering the layer   [rows][hidden] */
    TTSBB_TAP_H_ATTN = 1,  /* input_layernorm output (GEMM operand) [rows][hidden] */
    TTSBB_TAP_QKV = 2,     /* q|k|v projections before the head norms [rows][(H+2Hkv)*d] */
    TTSBB_TAP_Q = 3,       /* q after head norm + RoPE, as attention reads it [rows][H*d] */
    TTSBB_TAP_K = 4,       /* MaskGIT only: K after head norm + RoPE [rows][Hkv*d] */
    TTSBB_TAP_V = 5,       /* MaskGIT only: V [rows][Hkv*d] */
    TTSBB_TAP_ATTN = 6,    /* attention output (GEMM operand) [rows][H*d] */
    TTSBB_TAP_X_MID = 7,   /* x + Wo o                             [rows][hidden] */
    TTSBB_TAP_H_FFN = 8,   /* post_attention_layernorm output      [rows][hidden] */
    TTSBB_TAP_MLP = 9,     /* silu(gate) * up (GEMM operand)       [rows][ffn] */
    TTSBB_TAP_X_OUT = 10,  /* layer output                         [rows][hidden] */
    TTSBB_TAP_HEAD_IN = 11,/* final-normed head operand (not per layer) [rows][hidden] */
    TTSBB_TAP_LOGITS = 12, /* head output (not per layer) [rows][head cols] */
    TTSBB_TAP_LOGITS_U = 13, /* guided MaskGIT step: unconditional logits [rows][head cols] */
    TTSBB_TAP_COUNT = 14
} ttsbb_tap;

/* Record taps of `layer` (0-based) in the following calls; -1 turns taps off.
 * Allocates the tap buffers (not for use under graph capture). */
ttsbb_status ttsbb_set_tap_layer(ttsbb_ctx *ctx, int32_t layer);

/* Copy tap `tap` of the last call into dst (device fp32, n_floats elements); the rows
 * and width of the tap are written to *rows and *cols (host, may be NULL). */
ttsbb_status ttsbb_read_tap(ttsbb_ctx *ctx, int32_t tap, float *dst, int64_t n_floats,
                            int32_t *rows, int32_t *cols);


/* Instrumentation: HIP events recorded on the context's stream around every launch of
 * the kernel classes below, so a caller can measure per-kernel durations live.  Event
 * creation happens in ttsbb_profile_start (not for use under graph capture). */
typedef enum {
    TTSBB_K_EMBED = 0,         /* gather-sum embedding */
    TTSBB_K_RMSNORM = 1,       /* all RMSNorms */
    TTSBB_K_GEMM_QKV = 2,      /* q|k|v projection */
    TTSBB_K_ROPE_KV = 3,       /* head norms + RoPE + K/V write */
    TTSBB_K_DECODE_ATTN = 4,   /* split-sequence decode attention (main pass) */
    TTSBB_K_DECODE_COMBINE = 5,/* merge of the decode attention partials */
    TTSBB_K_FLASH_ATTN = 6,    /* bidirectional attention */
    TTSBB_K_GEMM_O = 7,        /* o_proj + residual */
    TTSBB_K_GEMM_GATE_UP = 8,  /* gate|up projection + SwiGLU */
    TTSBB_K_GEMM_DOWN = 9,     /* down_proj + residual */
    TTSBB_K_GEMM_HEAD = 10,    /* output heads */
    TTSBB_K_ARGMAX = 11,       /* greedy choice per group */
    TTSBB_K_SCORES = 12,       /* MaskGIT log-softmax / argmax / confidence */
    TTSBB_K_SELECT = 13,       /* MaskGIT top-n + code update */
    TTSBB_K_RVQ = 14,          /* codec RVQ decode */
    TTSBB_K_COUNT = 15
} ttsbb_kernel_class;

/* Start recording events for the classes whose bit (1 << class) is set in `mask`;
 * `max_launches` bounds the launches recorded before ttsbb_profile_stop. */
ttsbb_status ttsbb_profile_start(ttsbb_ctx *ctx, uint32_t mask, int32_t max_launches);

/* Synchronise, stop recording and return per class the summed milliseconds and launch
 * count (host arrays of TTSBB_K_COUNT entries; either may be NULL). */
ttsbb_status ttsbb_profile_stop(ttsbb_ctx *ctx, float *ms, int32_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* TTSBB_H */
