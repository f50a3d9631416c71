// ttsbb C ABI: context, argument checks, and the order of kernels of each call.
//
// Decode step (ncnn Qwen3-TTS port, "单token SDPA问题与host attention": per layer the
// pre-attention half, then RoPE + KV append + GQA attention, then output projection,
// MLP and residuals):
//   K2 norm -> K3 q|k|v -> K4 head norms + RoPE + KV write -> K5 attention -> K3 o_proj
//   (+x) -> K2 norm -> K3 gate|up with SwiGLU -> K3 down_proj (+x); after the layers
//   K2 final norm -> K3 head -> K7 argmax; positions += 1.
// MaskGIT step (OmniVoice ARCHITECTURE, "MaskGIT decoder" and "Inner-loop
// optimisations"): K1 hybrid embedding -> layers with K6 bidirectional attention ->
// K2 final norm on the audio window only -> K3 heads -> K8 scores -> K9 top-n update.
// Every call only enqueues on the context's stream.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <new>
#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/ttsbb.h"
#include "kernels.h"

using namespace ttsbb;

#define TTSBB_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int MAX_CHUNKS = 32;   // decode attention partials per (stream, head)
constexpr int SEG_PER_CU = 4;    // q_len = 1 decode attention waves per CU (work-list segments)
constexpr int PART_STRIDE = 132; // floats per partial (m, l, 2 pad, 128 dims)

// The decode step without allocation (ttsbb_decode_step_noalloc): its per-call scratch
// lives in one file-scope device array; every GPU the library runs on holds its own copy
// until the process ends.  Sized for the limits below at the default backbone shape.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)32 << 20;
constexpr int STATIC_MAX_BATCH = 64;
constexpr int STATIC_MAX_HEAD_COLS = 8200;
constexpr int STATIC_GPART_SPLITS = 8;  // the skinny products' largest K split
constexpr int MAX_DEVICES = 64;

struct Tap {
    float *buf = nullptr;
    int rows = 0, cols = 0;
};

struct Prof {
    uint32_t mask = 0;
    int cap = 0, used = 0;
    std::vector<hipEvent_t> ev;  // 2 per recorded launch
    std::vector<int> cls;
};

}  // namespace

struct ttsbb_ctx {
    ttsbb_config cfg;
    std::vector<ttsbb_layer> layers;
    const float *final_norm = nullptr;
    hipStream_t stream = nullptr;
    DType dt = DT_BF16;
    size_t esz = 2;  // bytes per operand element
    int qkv_w = 0;   // (H + 2 Hkv) * head_dim
    int n_cu = 256;  // compute units of the context's device
    // workspace
    void *h = nullptr;
    float *qkv = nullptr;
    void *q = nullptr;
    void *attn = nullptr;
    void *mlp = nullptr;
    float *x = nullptr;
    uint16_t *kbuf = nullptr, *vtbuf = nullptr;
    int s_pad_cap = 0;
    float *part = nullptr;
    float *logits = nullptr;
    float *logits_u = nullptr;  // unconditional logits of a guided MaskGIT step
    float4 *spart = nullptr;    // head-product scoring statistics [rows][128-column tiles][2]
    int32_t *rank = nullptr;
    int rank_cap = 0;
    float *gpart = nullptr;   // split-K partial sums
    int64_t gpart_cap = 0;    // floats
    int pend_splits = 0;      // K splits of a residual update still held in gpart
    int pend_rows = 0;
    float2 *rope = nullptr;
    int *flag = nullptr;
    int4 *plan = nullptr;     // decode attention work list (plan_entries(work_rows) entries)
    int *plan_n = nullptr;
    int *plan_pages = nullptr;  // [plan_entries][64]
    int2 *seg_cont = nullptr;   // [SEG_PER_CU * n_cu]
    int *plan_nc = nullptr;     // [work_rows]
    int work_rows = 0;          // rows the attention work list and partials are sized for
    void *static_scratch = nullptr;  // this device's copy of the static scratch array
    std::vector<void *> allocs;
    // taps
    int tap_layer = -1;
    Tap taps[TTSBB_TAP_COUNT];
    Prof prof;
};

// Entries of the decode attention's work list for `rows` streams: MAX_CHUNKS pieces per
// stream plus one first-piece entry per segment.
static size_t plan_entries(const ttsbb_ctx *c, size_t rows) { return rows * MAX_CHUNKS + (size_t)SEG_PER_CU * c->n_cu; }

// The static scratch of ttsbb_decode_step_noalloc.  Host code never uses this name as an
// address (it is a host-side stand-in): the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current (ttsbb_create).
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch array (nullptr if it cannot be had).
void *static_scratch_of(int dev) {
    if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p) g_scratch_ptr[dev] = p;
        else hipGetLastError();
    }
    return g_scratch_ptr[dev];
}

bool dev_alloc(ttsbb_ctx *c, void **p, size_t bytes) {
    if (bytes == 0) bytes = 256;
    if (hipMalloc(p, bytes) != hipSuccess) {
        *p = nullptr;
        return false;
    }
    c->allocs.push_back(*p);
    return true;
}

void free_all(ttsbb_ctx *c) {
    for (void *p : c->allocs) hipFree(p);
    c->allocs.clear();
    for (auto &t : c->taps) {
        if (t.buf) hipFree(t.buf);
        t.buf = nullptr;
    }
}

int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Event pair around one launch of a profiled kernel class.  With `attach` the scope
// records nothing itself: the single launch inside it takes start() / stop() and has
// the runtime stamp them from its own dispatch (hipExtLaunchKernel), so the pair times
// the kernel alone, without two extra packets in the stream.
struct KScope {
    ttsbb_ctx *c;
    int idx = -1;
    bool attach;
    KScope(ttsbb_ctx *ctx, int k, bool attach_to_launch = false) : c(ctx), attach(attach_to_launch) {
        Prof &p = c->prof;
        if (((p.mask >> k) & 1u) && p.used < p.cap) {
            idx = p.used++;
            p.cls[idx] = k;
            if (!attach) hipEventRecord(p.ev[2 * idx], c->stream);
        }
    }
    hipEvent_t start() const { return idx >= 0 ? c->prof.ev[2 * idx] : nullptr; }
    hipEvent_t stop() const { return idx >= 0 ? c->prof.ev[2 * idx + 1] : nullptr; }
    ~KScope() {
        if (idx >= 0 && !attach) hipEventRecord(c->prof.ev[2 * idx + 1], c->stream);
    }
};

void prof_release(Prof &p) {
    for (hipEvent_t e : p.ev) hipEventDestroy(e);
    p.ev.clear();
    p.cls.clear();
    p.cap = p.used = 0;
    p.mask = 0;
}

bool launch_failed() { return hipPeekAtLastError() != hipSuccess; }

int tap_width(const ttsbb_ctx *c, int tap) {
    const ttsbb_config &g = c->cfg;
    switch (tap) {
        case TTSBB_TAP_QKV: return c->qkv_w;
        case TTSBB_TAP_Q:
        case TTSBB_TAP_ATTN: return g.n_heads * g.head_dim;
        case TTSBB_TAP_K:
        case TTSBB_TAP_V: return g.n_kv_heads * g.head_dim;
        case TTSBB_TAP_MLP: return g.ffn;
        case TTSBB_TAP_LOGITS:
        case TTSBB_TAP_LOGITS_U: return g.max_head_cols > 0 ? g.max_head_cols : 1;
        default: return g.hidden;
    }
}

// Record a tap as a dense fp32 [rows][cols] copy of a strided source.
void tap(ttsbb_ctx *c, int which, const void *src, DType dt, int rows, int cols, int64_t s_row,
         int64_t s_col_hi, int64_t s_col_lo, int cols_lo) {
    Tap &t = c->taps[which];
    if (!t.buf) return;
    t.rows = rows;
    t.cols = cols;
    // view cols as [cols / cols_lo][cols_lo]
    launch_tap_copy(src, dt, s_row, s_col_hi, s_col_lo, rows, cols / cols_lo, cols_lo, t.buf, c->stream);
}

void tap_dense(ttsbb_ctx *c, int which, const void *src, DType dt, int rows, int cols, int ld) {
    tap(c, which, src, dt, rows, cols, ld, cols, 1, cols);
}

}  // namespace

// ------------------------------------------------------------------------------------

TTSBB_API void ttsbb_default_config(ttsbb_config *cfg) {
    if (!cfg) return;
    memset(cfg, 0, sizeof(*cfg));
    cfg->n_layers = 28;
    cfg->hidden = 1024;
    cfg->n_heads = 16;
    cfg->n_kv_heads = 8;
    cfg->head_dim = 128;
    cfg->ffn = 3072;
    cfg->rms_eps = 1e-6f;
    cfg->rope_theta = 1e6;
    cfg->dtype = TTSBB_BF16;
    cfg->kv_page = 16;
    cfg->max_rows = 1024;
    cfg->max_pos = 8192;
    cfg->max_head_cols = 8200;
}

TTSBB_API const char *ttsbb_status_str(ttsbb_status s) {
    switch (s) {
        case TTSBB_OK: return "ok";
        case TTSBB_INVALID_ARG: return "invalid argument";
        case TTSBB_UNSUPPORTED: return "unsupported shape or mode";
        case TTSBB_OOM: return "out of device memory";
        case TTSBB_DEVICE_ERROR: return "device error";
        default: return "unknown status";
    }
}

TTSBB_API ttsbb_status ttsbb_create(const ttsbb_config *cfg, const ttsbb_layer *layers,
                                    const float *final_norm, void *hip_stream, ttsbb_ctx **out) {
    if (!cfg || !out) return TTSBB_INVALID_ARG;
    *out = nullptr;
    const ttsbb_config &g = *cfg;
    if (g.n_layers < 0 || g.hidden <= 0 || g.n_heads <= 0 || g.n_kv_heads <= 0 || g.head_dim <= 0 ||
        g.ffn <= 0 || !(g.rms_eps >= 0.f) || !(g.rope_theta > 0.0) || g.kv_page <= 0 ||
        g.max_rows <= 0 || g.max_pos <= 0 || g.max_head_cols < 0 ||
        (g.dtype != TTSBB_F32 && g.dtype != TTSBB_BF16))
        return TTSBB_INVALID_ARG;
    if (g.n_layers > 0 && !layers) return TTSBB_INVALID_ARG;
    for (int l = 0; l < g.n_layers; ++l) {
        const ttsbb_layer &L = layers[l];
        if (!L.attn_norm || !L.q_norm || !L.k_norm || !L.ffn_norm || !L.wq || !L.wk || !L.wv ||
            !L.wo || !L.w_gate || !L.w_up || !L.w_down)
            return TTSBB_INVALID_ARG;
    }
    if (g.head_dim != 128 || g.hidden % 128 != 0 || g.hidden > 4096 || g.ffn % 128 != 0 ||
        g.n_heads % g.n_kv_heads != 0 || (g.n_heads / g.n_kv_heads > 2) || g.kv_page != 16)
        return TTSBB_UNSUPPORTED;

    ttsbb_ctx *c = new (std::nothrow) ttsbb_ctx();
    if (!c) return TTSBB_OOM;
    c->cfg = g;
    c->layers.assign(layers, layers + g.n_layers);
    c->final_norm = final_norm;
    c->stream = reinterpret_cast<hipStream_t>(hip_stream);
    c->dt = g.dtype == TTSBB_BF16 ? DT_BF16 : DT_F32;
    c->esz = g.dtype == TTSBB_BF16 ? 2 : 4;
    c->qkv_w = (g.n_heads + 2 * g.n_kv_heads) * g.head_dim;
    {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess) {
            if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                c->n_cu = n;
            c->static_scratch = static_scratch_of(dev);
        }
    }
    c->work_rows = g.max_rows;

    const size_t R = (size_t)g.max_rows;
    const size_t hd_all = (size_t)g.n_heads * g.head_dim;
    // dense K / V^T rows: a MaskGIT pass (max_rows) or a prefilled stream (max_pos)
    c->s_pad_cap = round_up(g.max_rows > g.max_pos ? g.max_rows : g.max_pos, 64);
    c->rank_cap = g.max_rows * (g.max_head_cols / 2 + 1);
    c->gpart_cap = (int64_t)16 << 20;  // 64 MB of split-K partials
    const size_t RA = R < 64 ? 64 : R;  // activation rows: a fragment-major layout spans 4 x 16
    bool ok = dev_alloc(c, &c->h, RA * g.hidden * c->esz) &&
              dev_alloc(c, (void **)&c->qkv, R * c->qkv_w * 4) &&
              dev_alloc(c, &c->q, R * hd_all * 4) &&
              dev_alloc(c, &c->attn, RA * hd_all * c->esz) &&
              dev_alloc(c, &c->mlp, RA * g.ffn * c->esz) &&
              dev_alloc(c, (void **)&c->x, R * g.hidden * 4) &&
              dev_alloc(c, (void **)&c->kbuf, (size_t)g.n_kv_heads * c->s_pad_cap * g.head_dim * c->esz) &&
              dev_alloc(c, (void **)&c->vtbuf, (size_t)g.n_kv_heads * c->s_pad_cap * g.head_dim * c->esz) &&
              dev_alloc(c, (void **)&c->part, R * g.n_heads * MAX_CHUNKS * PART_STRIDE * 4) &&
              dev_alloc(c, (void **)&c->logits, R * (size_t)(g.max_head_cols > 0 ? g.max_head_cols : 1) * 4) &&
              dev_alloc(c, (void **)&c->logits_u, R * (size_t)(g.max_head_cols > 0 ? g.max_head_cols : 1) * 4) &&
              dev_alloc(c, (void **)&c->spart, R * (size_t)((g.max_head_cols + 127) / 128 + 1) * 2 * sizeof(float4)) &&
              dev_alloc(c, (void **)&c->rank, (size_t)R * (g.max_head_cols / 2 + 1) * 4) &&
              dev_alloc(c, (void **)&c->gpart, (size_t)c->gpart_cap * 4) &&
              dev_alloc(c, (void **)&c->rope, (size_t)g.max_pos * 64 * sizeof(float2)) &&
              dev_alloc(c, (void **)&c->flag, 256) &&
              dev_alloc(c, (void **)&c->plan, plan_entries(c, R) * sizeof(int4)) &&
              dev_alloc(c, (void **)&c->plan_n, 256) &&
              dev_alloc(c, (void **)&c->plan_pages, plan_entries(c, R) * 64 * sizeof(int)) &&
              dev_alloc(c, (void **)&c->seg_cont, (size_t)SEG_PER_CU * c->n_cu * sizeof(int2)) &&
              dev_alloc(c, (void **)&c->plan_nc, R * sizeof(int));
    if (!ok) {
        free_all(c);
        delete c;
        hipGetLastError();
        return TTSBB_OOM;
    }
    // Padding keys of the MaskGIT K/V buffers must hold finite values (they meet a zero
    // probability), and the selection's rank counters must start from zero (every
    // selection leaves them zero again): zero them once here.
    ok = hipMemset(c->kbuf, 0, (size_t)g.n_kv_heads * c->s_pad_cap * g.head_dim * c->esz) == hipSuccess &&
         hipMemset(c->vtbuf, 0, (size_t)g.n_kv_heads * c->s_pad_cap * g.head_dim * c->esz) == hipSuccess &&
         hipMemset(c->flag, 0, 256) == hipSuccess &&
         hipMemset(c->rank, 0, (size_t)R * (g.max_head_cols / 2 + 1) * 4) == hipSuccess;
    // RoPE table: angle p * theta^(-2j/d) in double precision, rounded to fp32.
    std::vector<float2> tab((size_t)g.max_pos * 64);
    for (int p = 0; p < g.max_pos; ++p)
        for (int j = 0; j < 64; ++j) {
            const double w = pow(g.rope_theta, -2.0 * j / (double)g.head_dim);
            const double a = (double)p * w;
            tab[(size_t)p * 64 + j] = make_float2((float)cos(a), (float)sin(a));
        }
    ok = ok && hipMemcpy(c->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice) == hipSuccess;
    if (!ok) {
        free_all(c);
        delete c;
        hipGetLastError();
        return TTSBB_DEVICE_ERROR;
    }
    *out = c;
    return TTSBB_OK;
}

TTSBB_API void ttsbb_destroy(ttsbb_ctx *ctx) {
    if (!ctx) return;
    hipStreamSynchronize(ctx->stream);
    prof_release(ctx->prof);
    free_all(ctx);
    delete ctx;
}

TTSBB_API ttsbb_status ttsbb_sync(ttsbb_ctx *ctx) {
    if (!ctx) return TTSBB_INVALID_ARG;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess) return TTSBB_DEVICE_ERROR;
    int f = 0;
    if (hipMemcpy(&f, ctx->flag, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return TTSBB_DEVICE_ERROR;
    if (f) {
        hipMemset(ctx->flag, 0, sizeof(int));
        return TTSBB_DEVICE_ERROR;
    }
    return TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_codebook_embed(ttsbb_ctx *ctx, int32_t n_rows, int32_t n_cb,
                                            const int32_t *codes, const void *tables,
                                            int32_t cb_vocab, const uint8_t *is_text,
                                            const int32_t *text_ids, const void *text_table,
                                            int32_t text_vocab, float *out) {
    if (!ctx || n_rows < 0 || n_cb < 0 || cb_vocab <= 0) return TTSBB_INVALID_ARG;
    if (n_rows == 0) return TTSBB_OK;
    if (!out || (n_cb > 0 && (!codes || !tables))) return TTSBB_INVALID_ARG;
    if (is_text && (!text_ids || !text_table || text_vocab <= 0)) return TTSBB_INVALID_ARG;
    EmbedArgs a;
    a.n_rows = n_rows;
    a.n_cb = n_cb;
    a.hidden = ctx->cfg.hidden;
    a.codes = codes;
    a.code_row_stride = n_cb;
    a.code_cb_stride = 1;
    a.audio_row0 = 0;
    a.tables = tables;
    a.cb_vocab = cb_vocab;
    a.is_text = is_text;
    a.text_prefix = 0;
    a.text_ids = text_ids;
    a.text_table = text_table;
    a.text_vocab = text_vocab;
    a.out = out;
    a.flag = ctx->flag;
    {
        KScope k(ctx, TTSBB_K_EMBED);
        launch_embed(a, ctx->dt, ctx->stream);
    }
    return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
}

namespace {

// The post-attention half of a layer and the pre-attention projection; shared by both
// modes.  x is the fp32 residual stream [M][hidden].
// RMSNorm of rows [0, M) of the residual stream x into c->h, first applying a residual
// update that a split projection left in gpart (gain == nullptr: the update only).
// out_mt > 0: c->h in the fragment-major layout of the skinny products (out_mt tiles).
void norm_rows(ttsbb_ctx *c, float *x, int M, const float *gain, int out_mt = 0) {
    const ttsbb_config &g = c->cfg;
    const int np = c->pend_rows == M ? c->pend_splits : 0;  // rows always match by construction
    if (gain || np > 0) {
        KScope k(c, TTSBB_K_RMSNORM);
        launch_rmsnorm(x, g.hidden, M, g.hidden, gain, g.rms_eps, c->h, c->dt, c->stream, c->gpart, np, g.hidden,
                       (int64_t)M * g.hidden, out_mt);
    }
    c->pend_splits = 0;
}

// Activation layout of a decode layer's four products over M rows: the skinny kernel's
// fragment-major layout (its 16-row tiles; every operand fragment one contiguous 1 KB
// load) when all four run on that kernel and nothing taps the operands, else 0
// (row-major).  The producers (RMSNorm, chunk merge, SwiGLU epilogue) write it.
int layer_pack_mt(const ttsbb_ctx *c, int M, bool tapit) {
    const ttsbb_config &g = c->cfg;
    if (tapit || c->dt != DT_BF16) return 0;
    const int shapes[4][3] = {{g.hidden, c->qkv_w, EPI_STORE},
                              {g.n_heads * g.head_dim, g.hidden, EPI_ADD},
                              {g.hidden, 2 * g.ffn, EPI_SWIGLU},
                              {g.ffn, g.hidden, EPI_ADD}};
    int mt = -1;
    for (const auto &sh : shapes) {
        GemmArgs a = {};
        a.M = M;
        a.K = sh[0];
        a.N = sh[1];
        a.epi = sh[2];
        const int t = skinny_tiles(a, c->gpart_cap);
        if (t == 0 || (mt >= 0 && t != mt)) return 0;
        mt = t;
    }
    return mt;
}

// The same for the head product (K = hidden, N columns).
int head_pack_mt(const ttsbb_ctx *c, int M, int N, bool tapped) {
    if (tapped || c->dt != DT_BF16) return 0;
    GemmArgs a = {};
    a.M = M;
    a.K = c->cfg.hidden;
    a.N = N;
    a.epi = EPI_STORE;
    return skinny_tiles(a, c->gpart_cap);
}

void flush_residual(ttsbb_ctx *c, float *x, int M) {
    if (c->pend_splits > 0) norm_rows(c, x, M, nullptr);
}

// A product of at most 8 rows (any rows in fp32 mode) runs on the GEMV kernel, which can
// compute the RMSNorm of its operand rows itself: the separate RMSNorm launch is skipped
// when no split partials are pending and the normalized rows are not tapped.
// (The GEMV builds the normalized rows of one launch, at most 8, in 64 KB of LDS.)
bool gemv_rows_fold(const ttsbb_ctx *c, int M) {
    const int rows = M < 8 ? M : 8;
    return (c->dt == DT_F32 || M <= 8) && (int64_t)rows * c->cfg.hidden * (int64_t)c->esz <= 65536;
}

bool norm_folds(const ttsbb_ctx *c, int M, bool tapit) {
    const int np = c->pend_rows == M ? c->pend_splits : 0;
    return !tapit && np == 0 && gemv_rows_fold(c, M);
}

void fold_norm(const ttsbb_ctx *c, GemmArgs &a, const float *x, const float *gain) {
    a.nx = x;
    a.ng = gain;
    a.neps = c->cfg.rms_eps;
}

// Residual-add projection: the product may leave its update pending in gpart.
void add_projection(ttsbb_ctx *c, const GemmArgs &a) {
    c->pend_splits = launch_gemm(a, c->dt, c->gpart, c->gpart_cap, c->stream);
    c->pend_rows = a.M;
}

// RMSNorm + q/k/v projection.  With `dense` (the MaskGIT pass), the per-head norm, RoPE
// and the dense q / K / V^T layout are fused into the product when the shape allows;
// returns true when that happened (qkv is then not written).
bool qkv_projection(ttsbb_ctx *c, const ttsbb_layer &L, float *x, int M, bool tapit,
                    const RopeKvArgs *dense = nullptr, int pack_mt = 0) {
    const ttsbb_config &g = c->cfg;
    if (tapit) {
        flush_residual(c, x, M);
        tap_dense(c, TTSBB_TAP_X_IN, x, DT_F32, M, g.hidden, g.hidden);
    }
    const bool fold = !dense && norm_folds(c, M, tapit);
    if (!fold) norm_rows(c, x, M, L.attn_norm, pack_mt);
    GemmArgs a = {};
    if (fold) fold_norm(c, a, x, L.attn_norm);
    a.A = c->h;
    a.a_mt = pack_mt;
    a.lda = g.hidden;
    a.M = M;
    a.K = g.hidden;
    a.N = c->qkv_w;
    a.w.p[0] = L.wq;
    a.w.p[1] = L.wk;
    a.w.p[2] = L.wv;
    a.w.start[0] = 0;
    a.w.start[1] = g.n_heads * g.head_dim;
    a.w.start[2] = (g.n_heads + g.n_kv_heads) * g.head_dim;
    a.w.start[3] = c->qkv_w;
    a.w.nseg = 3;
    a.C = c->qkv;
    a.ldc = c->qkv_w;
    a.epi = EPI_STORE;
    bool fused = false;
    {
        KScope k(c, TTSBB_K_GEMM_QKV);
        if (dense) fused = launch_qkv_dense(a, *dense, c->stream);
        if (!fused) launch_gemm(a, c->dt, c->gpart, c->gpart_cap, c->stream);
    }
    if (tapit) {
        tap_dense(c, TTSBB_TAP_H_ATTN, c->h, c->dt, M, g.hidden, g.hidden);
        if (!fused) tap_dense(c, TTSBB_TAP_QKV, c->qkv, DT_F32, M, c->qkv_w, c->qkv_w);
    }
    return fused;
}

// attn_mt / pack_mt: layouts of the attention output and of the layer's other
// activations (0: row-major; see layer_pack_mt).
void post_attention(ttsbb_ctx *c, const ttsbb_layer &L, float *x, int M, bool tapit, int attn_mt = 0,
                    int pack_mt = 0) {
    const ttsbb_config &g = c->cfg;
    const int hd_all = g.n_heads * g.head_dim;
    if (tapit) tap_dense(c, TTSBB_TAP_ATTN, c->attn, c->dt, M, hd_all, hd_all);
    GemmArgs a = {};
    a.A = c->attn;
    a.a_mt = attn_mt;
    a.lda = hd_all;
    a.M = M;
    a.K = hd_all;
    a.N = g.hidden;
    a.w.p[0] = L.wo;
    a.w.start[0] = 0;
    a.w.start[1] = g.hidden;
    a.w.nseg = 1;
    a.C = x;
    a.ldc = g.hidden;
    a.epi = EPI_ADD;
    {
        KScope k(c, TTSBB_K_GEMM_O);
        add_projection(c, a);
    }
    if (tapit) {
        flush_residual(c, x, M);
        tap_dense(c, TTSBB_TAP_X_MID, x, DT_F32, M, g.hidden, g.hidden);
    }
    const bool fold = norm_folds(c, M, tapit);
    if (!fold) norm_rows(c, x, M, L.ffn_norm, pack_mt);
    if (tapit) tap_dense(c, TTSBB_TAP_H_FFN, c->h, c->dt, M, g.hidden, g.hidden);
    GemmArgs u = {};
    if (fold) fold_norm(c, u, x, L.ffn_norm);
    u.A = c->h;
    u.a_mt = pack_mt;
    u.c_mt = pack_mt;
    u.lda = g.hidden;
    u.M = M;
    u.K = g.hidden;
    u.N = 2 * g.ffn;
    u.w.p[0] = L.w_gate;
    u.w.p[1] = L.w_up;
    u.w.nseg = 2;
    u.C = c->mlp;
    u.ldc = g.ffn;
    u.epi = EPI_SWIGLU;
    {
        KScope k(c, TTSBB_K_GEMM_GATE_UP);
        launch_gemm(u, c->dt, c->gpart, c->gpart_cap, c->stream);
    }
    if (tapit) tap_dense(c, TTSBB_TAP_MLP, c->mlp, c->dt, M, g.ffn, g.ffn);

    GemmArgs d = {};
    d.A = c->mlp;
    d.a_mt = pack_mt;
    d.lda = g.ffn;
    d.M = M;
    d.K = g.ffn;
    d.N = g.hidden;
    d.w.p[0] = L.w_down;
    d.w.start[0] = 0;
    d.w.start[1] = g.hidden;
    d.w.nseg = 1;
    d.C = x;
    d.ldc = g.hidden;
    d.epi = EPI_ADD;
    {
        KScope k(c, TTSBB_K_GEMM_DOWN);
        add_projection(c, d);
    }
    if (tapit) {
        flush_residual(c, x, M);
        tap_dense(c, TTSBB_TAP_X_OUT, x, DT_F32, M, g.hidden, g.hidden);
    }
}

// Head product of rows [row0, row0 + M); with norm_x the final RMSNorm is folded into it
// (norm_x = the residual rows, which must hold no pending split partials).
void head_gemm(ttsbb_ctx *c, const void *head, int M, int N, float *out, int ldc, int row0 = 0,
               const float *norm_x = nullptr, int a_mt = 0) {
    const ttsbb_config &g = c->cfg;
    GemmArgs a = {};
    if (norm_x) fold_norm(c, a, norm_x + (size_t)row0 * g.hidden, c->final_norm);
    a.A = reinterpret_cast<const char *>(c->h) + (size_t)row0 * g.hidden * c->esz;
    a.a_mt = a_mt;  // fragment-major only with row0 == 0
    a.lda = g.hidden;
    a.M = M;
    a.K = g.hidden;
    a.N = N;
    a.w.p[0] = head;
    a.w.start[0] = 0;
    a.w.start[1] = N;
    a.w.nseg = 1;
    a.C = out;
    a.ldc = ldc;
    a.epi = EPI_STORE;
    KScope k(c, TTSBB_K_GEMM_HEAD);
    launch_gemm(a, c->dt, c->gpart, c->gpart_cap, c->stream);
}

// MaskGIT input rows [0, S) of ctx->x: n_text text rows, then audio frames whose code
// (k, t) is codes[k * codes_ld + t].
void maskgit_embed(ttsbb_ctx *ctx, int S, int n_text, const int32_t *text_ids, const void *text_table,
                   int text_vocab, int n_cb, int cb_vocab, const void *audio_tables, const int32_t *codes,
                   int codes_ld, int out_row0 = 0) {
    EmbedArgs e;
    e.n_rows = S;
    e.n_cb = n_cb;
    e.hidden = ctx->cfg.hidden;
    e.codes = codes;
    e.code_row_stride = 1;
    e.code_cb_stride = codes_ld;
    e.audio_row0 = n_text;
    e.tables = audio_tables;
    e.cb_vocab = cb_vocab;
    e.is_text = nullptr;
    e.text_prefix = n_text;
    e.text_ids = text_ids;
    e.text_table = text_table;
    e.text_vocab = text_vocab;
    e.out = ctx->x + (size_t)out_row0 * ctx->cfg.hidden;
    e.flag = ctx->flag;
    KScope k(ctx, TTSBB_K_EMBED);
    launch_embed(e, ctx->dt, ctx->stream);
}

// Every layer over rows [0, M) of ctx->x with bidirectional attention and no cache: one
// sequence (seg1 == 0, len0 == M, RoPE positions 0..M-1), or two independent ones in the
// same launches (rows [0, len0) and [seg1, seg1 + len1), each at positions from 0, seg1 a
// multiple of 64; the rows in between are padding).  Per-layer taps (all M rows: the
// first sequence leads) only when `taps`.  Leaves no split partials pending.
void maskgit_layers(ttsbb_ctx *ctx, int M, int seg1, int len0, int len1, bool taps) {
    const ttsbb_config &g = ctx->cfg;
    const int s_pad = round_up(M, 64);
    const int H = g.n_heads, Hkv = g.n_kv_heads, hd = g.head_dim;
    const int hd_all = H * hd;
    for (int l = 0; l < g.n_layers; ++l) {
        const ttsbb_layer &L = ctx->layers[l];
        const bool tapit = taps && (l == ctx->tap_layer);
        RopeKvArgs r = {};
        r.qkv = ctx->qkv;
        r.M = M;
        r.H = H;
        r.Hkv = Hkv;
        r.q_gain = L.q_norm;
        r.k_gain = L.k_norm;
        r.eps = g.rms_eps;
        r.rope = ctx->rope;
        r.max_pos = g.max_pos;
        r.q_out = ctx->q;
        r.dense = 1;
        r.kbuf = ctx->kbuf;
        r.vtbuf = ctx->vtbuf;
        r.s_pad = s_pad;
        r.flag = ctx->flag;
        r.seg1 = seg1;
        if (ctx->dt == DT_F32) {
            // fp32: the projection, then norms + RoPE into fp32 q / K / V rows, then the fp32
            // attention kernel
            r.dense_f32 = 1;
            qkv_projection(ctx, L, ctx->x, M, tapit);
            {
                KScope k(ctx, TTSBB_K_ROPE_KV);
                launch_rope_kv(r, DT_F32, ctx->stream);
            }
            if (tapit) {
                tap_dense(ctx, TTSBB_TAP_Q, ctx->q, DT_F32, M, hd_all, hd_all);
                // K, V [Hkv][s_pad][hd] -> [M][Hkv][hd]
                tap(ctx, TTSBB_TAP_K, ctx->kbuf, DT_F32, M, Hkv * hd, hd, (int64_t)s_pad * hd, 1, hd);
                tap(ctx, TTSBB_TAP_V, ctx->vtbuf, DT_F32, M, Hkv * hd, hd, (int64_t)s_pad * hd, 1, hd);
            }
            AttnF32Args f = {};
            f.q = reinterpret_cast<const float *>(ctx->q);
            f.k = reinterpret_cast<const float *>(ctx->kbuf);
            f.v = reinterpret_cast<const float *>(ctx->vtbuf);
            f.S = M;
            f.s_pad = s_pad;
            f.H = H;
            f.Hkv = Hkv;
            f.scale = (float)(1.0 / sqrt((double)hd));
            f.out = reinterpret_cast<float *>(ctx->attn);
            f.seg1 = seg1;
            f.len0 = len0;
            f.len1 = len1;
            {
                KScope k(ctx, TTSBB_K_FLASH_ATTN);
                launch_attn_f32(f, ctx->stream);
            }
            post_attention(ctx, L, ctx->x, M, tapit);
            continue;
        }
        if (!qkv_projection(ctx, L, ctx->x, M, tapit, &r)) {
            KScope k(ctx, TTSBB_K_ROPE_KV);
            launch_rope_kv(r, DT_BF16, ctx->stream);
        }
        if (tapit) {
            tap_dense(ctx, TTSBB_TAP_Q, ctx->q, DT_BF16, M, hd_all, hd_all);
            // K [Hkv][s_pad][hd] -> [M][Hkv][hd];  V^T [Hkv][hd][s_pad] -> [M][Hkv][hd]
            tap(ctx, TTSBB_TAP_K, ctx->kbuf, DT_BF16, M, Hkv * hd, hd, (int64_t)s_pad * hd, 1, hd);
            tap(ctx, TTSBB_TAP_V, ctx->vtbuf, DT_BF16, M, Hkv * hd, 1, (int64_t)hd * s_pad, s_pad, hd);
        }

        FlashArgs f = {};
        f.q = reinterpret_cast<const uint16_t *>(ctx->q);
        f.k = ctx->kbuf;
        f.vt = ctx->vtbuf;
        f.S = M;
        f.s_pad = s_pad;
        f.H = H;
        f.Hkv = Hkv;
        f.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
        f.out = reinterpret_cast<uint16_t *>(ctx->attn);
        f.seg1 = seg1;
        f.len0 = len0;
        f.len1 = len1;
        {
            KScope k(ctx, TTSBB_K_FLASH_ATTN);
            launch_flash_attn(f, ctx->stream);
        }
        post_attention(ctx, L, ctx->x, M, tapit);
    }
    flush_residual(ctx, ctx->x, M);
}

// Final RMSNorm of rows [row0, row0 + n_out) of ctx->x and the heads into logits
// [n_out][N].
void maskgit_head(ttsbb_ctx *ctx, int row0, int n_out, const void *heads, int N, float *logits, bool taps) {
    const ttsbb_config &g = ctx->cfg;
    {
        KScope k(ctx, TTSBB_K_RMSNORM);
        launch_rmsnorm(ctx->x + (size_t)row0 * g.hidden, g.hidden, n_out, g.hidden, ctx->final_norm, g.rms_eps,
                       ctx->h, ctx->dt, ctx->stream);
    }
    if (taps && ctx->tap_layer >= 0) tap_dense(ctx, TTSBB_TAP_HEAD_IN, ctx->h, ctx->dt, n_out, g.hidden, g.hidden);
    head_gemm(ctx, heads, n_out, N, logits, N);
}

// Unguided MaskGIT scores of rows [row0, row0 + n_out) (frames of the window, codes
// window[k * codes_ld + t]) straight from the head product: the final RMSNorm, the head
// GEMM with the scoring epilogue (logits never stored) and the merge into pred, conf.
// With taps on, the logits are also materialized by the plain head product for the
// logits tap.  Returns false (nothing launched) for a shape the fused head does not take
// (n_out <= 64, a codebook narrower than one 128-column tile).
bool maskgit_head_scores(ttsbb_ctx *ctx, int row0, int n_out, const void *heads, int n_cb, int V, int mask_id,
                         float penalty, const int32_t *window, int codes_ld, int32_t *pred, float *conf) {
    const ttsbb_config &g = ctx->cfg;
    const int N = n_cb * V;
    if (ctx->dt != DT_BF16 || n_out <= 64 || V < 128 || g.hidden % 64 != 0) return false;
    {
        KScope k(ctx, TTSBB_K_RMSNORM);
        launch_rmsnorm(ctx->x + (size_t)row0 * g.hidden, g.hidden, n_out, g.hidden, ctx->final_norm, g.rms_eps,
                       ctx->h, DT_BF16, ctx->stream);
    }
    if (ctx->tap_layer >= 0) {
        tap_dense(ctx, TTSBB_TAP_HEAD_IN, ctx->h, DT_BF16, n_out, g.hidden, g.hidden);
        head_gemm(ctx, heads, n_out, N, ctx->logits, N);
        tap_dense(ctx, TTSBB_TAP_LOGITS, ctx->logits, DT_F32, n_out, N, N);
    }
    GemmArgs a = {};
    a.A = ctx->h;
    a.lda = g.hidden;
    a.M = n_out;
    a.K = g.hidden;
    a.N = N;
    a.w.p[0] = heads;
    a.w.start[0] = 0;
    a.w.start[1] = N;
    a.w.nseg = 1;
    a.epi = EPI_STORE;
    a.gv = V;
    a.gmask = mask_id;
    a.spart = ctx->spart;
    {
        KScope k(ctx, TTSBB_K_GEMM_HEAD);
        if (!launch_head_scores(a, ctx->stream)) return false;  // excluded above: never taken
    }
    KScope k(ctx, TTSBB_K_SCORES);
    launch_maskgit_merge(ctx->spart, n_out, N, n_cb, V, mask_id, penalty, window, codes_ld, pred, conf, ctx->flag,
                         ctx->stream);
    return true;
}

// One sequence of S rows: layers, then the heads of rows [row0, row0 + n_out).
void maskgit_backbone(ttsbb_ctx *ctx, int S, int row0, int n_out, const void *heads, int N, float *logits,
                      bool taps) {
    maskgit_layers(ctx, S, 0, S, 0, taps);
    maskgit_head(ctx, row0, n_out, heads, N, logits, taps);
}

// The two passes of a guided step: the conditional sequence (the whole prompt, S rows,
// logits of its window rows [n_text + w0, n_text + w0 + n_target) into ctx->logits) and
// the unconditional one (the window's frames alone, into ctx->logits_u).  When both fit
// the workspace they run as one batch of two sequences (rows [0, S) and [seg1, seg1 +
// n_target), seg1 = S rounded up to 64): the products see one M = seg1 + n_target, and the
// attention keeps the sequences apart.  Otherwise two passes.
void maskgit_guided(ttsbb_ctx *ctx, int n_text, const int32_t *text_ids, const void *text_table, int text_vocab,
                    int n_frames, int n_target, int n_cb, int cb_vocab, const void *audio_tables,
                    const void *audio_heads, const int32_t *codes) {
    const ttsbb_config &g = ctx->cfg;
    const int S = n_text + n_frames, w0 = n_frames - n_target;
    const int N = n_cb * cb_vocab;
    const int32_t *window = codes + w0;
    const int seg1 = round_up(S, 64), M = seg1 + n_target;
    if (M <= g.max_rows) {
        maskgit_embed(ctx, S, n_text, text_ids, text_table, text_vocab, n_cb, cb_vocab, audio_tables, codes, n_frames);
        if (seg1 > S)  // padding rows: zero (no text, no codebook)
            maskgit_embed(ctx, seg1 - S, 0, nullptr, nullptr, 0, 0, cb_vocab, audio_tables, nullptr, n_frames, S);
        maskgit_embed(ctx, n_target, 0, nullptr, nullptr, 0, n_cb, cb_vocab, audio_tables, window, n_frames, seg1);
        maskgit_layers(ctx, M, seg1, S, n_target, true);
        maskgit_head(ctx, n_text + w0, n_target, audio_heads, N, ctx->logits, true);
        if (ctx->tap_layer >= 0) tap_dense(ctx, TTSBB_TAP_LOGITS, ctx->logits, DT_F32, n_target, N, N);
        maskgit_head(ctx, seg1, n_target, audio_heads, N, ctx->logits_u, false);
    } else {
        maskgit_embed(ctx, S, n_text, text_ids, text_table, text_vocab, n_cb, cb_vocab, audio_tables, codes, n_frames);
        maskgit_backbone(ctx, S, n_text + w0, n_target, audio_heads, N, ctx->logits, true);
        if (ctx->tap_layer >= 0) tap_dense(ctx, TTSBB_TAP_LOGITS, ctx->logits, DT_F32, n_target, N, N);
        maskgit_embed(ctx, n_target, 0, nullptr, nullptr, 0, n_cb, cb_vocab, audio_tables, window, n_frames);
        maskgit_backbone(ctx, n_target, 0, n_target, audio_heads, N, ctx->logits_u, false);
    }
    if (ctx->tap_layer >= 0) tap_dense(ctx, TTSBB_TAP_LOGITS_U, ctx->logits_u, DT_F32, n_target, N, N);
}

}  // namespace

// The paged forward shared by the decode step (batch streams, one token each, row b at
// position positions[b], page-table row b) and the prefill (batch tokens of one stream,
// row b at position positions[0] + b, page-table row 0, causal by construction since
// row b attends to positions 0..positions[0] + b).  The prefill's head reads the last
// row only.
static ttsbb_status paged_forward(ttsbb_ctx *ctx, int32_t batch, float *x, int32_t *positions, const int32_t *page_table,
                           int32_t max_pages, void *kv_pool, int32_t n_pages, const void *head, int32_t n_groups,
                           int32_t group_vocab, int32_t *argmax, float *logits, bool prefill) {
    if (!ctx || batch < 0) return TTSBB_INVALID_ARG;
    const ttsbb_config &g = ctx->cfg;
    ctx->pend_splits = 0;
    if (batch > g.max_rows) return TTSBB_INVALID_ARG;
    if (batch == 0) return TTSBB_OK;
    if (!x || !positions) return TTSBB_INVALID_ARG;
    if (g.n_layers > 0 && (!page_table || max_pages <= 0 || !kv_pool || n_pages <= 0))
        return TTSBB_INVALID_ARG;
    if (head) {
        if (n_groups <= 0 || group_vocab <= 0 || !argmax || !ctx->final_norm) return TTSBB_INVALID_ARG;
        if ((int64_t)n_groups * group_vocab > g.max_head_cols) return TTSBB_INVALID_ARG;
    }
    const int H = g.n_heads, Hkv = g.n_kv_heads, hd = g.head_dim;
    const int hd_all = H * hd;
    const size_t layer_elems = (size_t)n_pages * 2 * Hkv * g.kv_page * hd;

    // A prefill of more than 64 tokens (bf16, untapped) runs its attention as the causal
    // flash kernel over the stream's whole sequence, read from the pool into the dense
    // K / V^T buffers (sized for max_pos positions); shorter ones, and tapped runs, go
    // through the decode attention, each token over its prefix.
    if (prefill && batch > 64 && ctx->dt == DT_BF16 && ctx->tap_layer < 0 && g.n_layers > 0 &&
        batch <= ctx->s_pad_cap) {
        for (int l = 0; l < g.n_layers; ++l) {
            const ttsbb_layer &L = ctx->layers[l];
            qkv_projection(ctx, L, x, batch, false);
            void *pool_l = reinterpret_cast<char *>(kv_pool) + (size_t)l * layer_elems * ctx->esz;
            RopeKvArgs r = {};
            r.qkv = ctx->qkv;
            r.M = batch;
            r.H = H;
            r.Hkv = Hkv;
            r.q_gain = L.q_norm;
            r.k_gain = L.k_norm;
            r.eps = g.rms_eps;
            r.rope = ctx->rope;
            r.max_pos = g.max_pos;
            r.q_out = ctx->q;
            r.q_bf16 = 1;
            r.pos = positions;
            r.page_table = page_table;
            r.max_pages = max_pages;
            r.n_pages = n_pages;
            r.page = g.kv_page;
            r.pool_layer = pool_l;
            r.flag = ctx->flag;
            r.shared = 1;
            // the dense K / V^T rows of positions [0, p0 + batch) for the flash kernel: the
            // prompt's from its own rows, the cached prefix copied from the pool, in the
            // same launch (batch <= s_pad_cap, bf16: checked above)
            r.dense_copy = 1;
            r.kbuf = ctx->kbuf;
            r.vtbuf = ctx->vtbuf;
            r.s_pad = ctx->s_pad_cap;
            {
                KScope k(ctx, TTSBB_K_ROPE_KV);
                launch_rope_kv(r, ctx->dt, ctx->stream);
            }
            FlashArgs f = {};
            f.q = reinterpret_cast<const uint16_t *>(ctx->q);
            f.k = ctx->kbuf;
            f.vt = ctx->vtbuf;
            f.S = batch;
            f.s_pad = ctx->s_pad_cap;
            f.H = H;
            f.Hkv = Hkv;
            f.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
            f.out = reinterpret_cast<uint16_t *>(ctx->attn);
            f.len0 = batch;
            f.causal_pos = positions;
            {
                KScope k(ctx, TTSBB_K_FLASH_ATTN);
                launch_flash_attn(f, ctx->stream);
            }
            post_attention(ctx, L, x, batch, false);
        }
        if (!head) flush_residual(ctx, x, batch);
        if (head) {
            const int N = n_groups * group_vocab;
            const bool fold = gemv_rows_fold(ctx, 1);
            if (fold) flush_residual(ctx, x, batch);
            else norm_rows(ctx, x, batch, ctx->final_norm);
            float *lg = logits ? logits : ctx->logits;
            head_gemm(ctx, head, 1, N, lg, N, batch - 1, fold ? x : nullptr);
            KScope k(ctx, TTSBB_K_ARGMAX);
            launch_argmax_groups(lg, 1, N, n_groups, group_vocab, argmax, ctx->flag, ctx->stream);
        }
        launch_increment(positions, 1, ctx->stream, batch);
        return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
    }

    // The attention's chunk bound: 128 positions, halved while there are fewer than 256
    // (stream, KV head, chunk) items (batch 1, KV ~1000: 32-position chunks).  Prefill rows
    // take pieces of at most one chunk; in q_len = 1 decode the chunk count bounds the
    // number of segments and sizes each stream's partial slots, and caches within one
    // chunk take the direct mode.  The partial buffer holds max_rows * MAX_CHUNKS slots
    // per head, and a piece spans at most 64 pages (one page id per lane).
    const int cap = max_pages * g.kv_page;
    int chunk = 128;
    while (chunk > g.kv_page && (int64_t)batch * Hkv * ((cap + chunk - 1) / chunk) < 256) chunk /= 2;
    chunk = round_up(chunk, g.kv_page);
    int n_chunks = (cap + chunk - 1) / chunk;
    // q_len = 1 decode: a stream's weighted-segment pieces may number two more than its
    // chunks (the plan kernel's guarantee), so its partial slots hold n_chunks + 2
    const int extra = prefill ? 0 : 2;
    while ((int64_t)batch * (n_chunks + extra) > (int64_t)ctx->work_rows * MAX_CHUNKS) {
        chunk *= 2;
        n_chunks = (cap + chunk - 1) / chunk;
    }
    if (chunk > 64 * g.kv_page) return TTSBB_UNSUPPORTED;

    // the fields of the attention's arguments that every layer shares, and the step's work
    // list built from them
    DecodeAttnArgs da = {};
    da.pos = positions;
    da.page_table = page_table;
    da.max_pages = max_pages;
    da.n_pages = n_pages;
    da.page = g.kv_page;
    da.B = batch;
    da.H = H;
    da.Hkv = Hkv;
    da.chunk = chunk;
    da.n_chunks = n_chunks;
    da.part_stride = n_chunks + extra;
    da.plan = ctx->plan;
    da.plan_n = ctx->plan_n;
    da.plan_pages = ctx->plan_pages;
    da.plan_cap = (int)plan_entries(ctx, ctx->work_rows);
    da.seg_cont = ctx->seg_cont;
    da.plan_nc = ctx->plan_nc;
    // q_len = 1 decode: the streams' pages cut into weighted segments, one wave per segment
    // and KV head, one workgroup of four waves per CU (64-stream workload, µs per launch:
    // 85.3 against 86.1 with two workgroups per CU, 87.5 with three, 126 with half a
    // workgroup); an even number of segments, so that both XCD parities get their share
    da.target_items = prefill ? 0 : SEG_PER_CU * ctx->n_cu;
    da.n_seg = (int)std::min<int64_t>({da.target_items / Hkv, (int64_t)batch * n_chunks, SEG_MAX}) & ~1;
    if (da.n_seg < 2) da.n_seg = 2;
    da.part = ctx->part;
    da.out = ctx->attn;
    da.scale_log2 = (float)(1.4426950408889634 / sqrt((double)hd));
    da.shared = prefill ? 1 : 0;
    da.max_pos = g.max_pos;
    // caches that fit one chunk: the attention covers each stream whole and writes the
    // output rows itself (no work list, no merge launch)
    da.direct = !prefill && n_chunks == 1 ? 1 : 0;
    if (!da.direct) {
        if (!prefill) da.flag = ctx->flag;  // the prefill's positions are checked by the rope kernel
        launch_decode_plan(da, ctx->stream);
        da.flag = nullptr;
    }

    for (int l = 0; l < g.n_layers; ++l) {
        const ttsbb_layer &L = ctx->layers[l];
        const bool tapit = (l == ctx->tap_layer);
        const int pack_mt = layer_pack_mt(ctx, batch, tapit);
        qkv_projection(ctx, L, x, batch, tapit, nullptr, pack_mt);
        void *pool_l = reinterpret_cast<char *>(kv_pool) + (size_t)l * layer_elems * ctx->esz;

        RopeKvArgs r = {};
        r.qkv = ctx->qkv;
        r.M = batch;
        r.H = H;
        r.Hkv = Hkv;
        r.q_gain = L.q_norm;
        r.k_gain = L.k_norm;
        r.eps = g.rms_eps;
        r.rope = ctx->rope;
        r.max_pos = g.max_pos;
        r.q_out = ctx->q;
        r.dense = 0;
        r.pos = positions;
        r.page_table = page_table;
        r.max_pages = max_pages;
        r.n_pages = n_pages;
        r.page = g.kv_page;
        r.pool_layer = pool_l;
        r.flag = ctx->flag;
        r.shared = prefill ? 1 : 0;
        // a q_len = 1 step folds the token's head norms, RoPE and K/V append into the
        // attention kernel (below); the separate kernel runs for the prefill and when q is
        // tapped
        const bool fused = !prefill && !tapit;
        if (!fused) {
            KScope k(ctx, TTSBB_K_ROPE_KV);
            launch_rope_kv(r, ctx->dt, ctx->stream);
        }
        if (tapit) tap_dense(ctx, TTSBB_TAP_Q, ctx->q, DT_F32, batch, hd_all, hd_all);

        DecodeAttnArgs d = da;
        d.q = reinterpret_cast<const float *>(ctx->q);
        d.pool_layer = pool_l;
        d.out_mt = pack_mt;  // the merge writes the o-projection's operand
        if (fused) {
            d.qkv = ctx->qkv;
            d.q_gain = L.q_norm;
            d.k_gain = L.k_norm;
            d.rope = ctx->rope;
            d.eps = g.rms_eps;
            d.max_pos = g.max_pos;
            d.flag = ctx->flag;
        }
        {
            KScope k(ctx, TTSBB_K_DECODE_ATTN, true);
            launch_decode_attn(d, ctx->dt, ctx->stream, k.start(), k.stop());
        }
        if (!d.direct) {
            KScope k(ctx, TTSBB_K_DECODE_COMBINE);
            launch_decode_combine(d, ctx->dt, ctx->stream);
        }

        post_attention(ctx, L, x, batch, tapit, pack_mt, pack_mt);
    }
    if (!head) flush_residual(ctx, x, batch);
    if (head) {
        const int N = n_groups * group_vocab;
        const int r0 = prefill ? batch - 1 : 0, rows = prefill ? 1 : batch;  // rows read out
        const bool tap_head = ctx->tap_layer >= 0;
        const bool fold = !tap_head && gemv_rows_fold(ctx, rows);
        const int hmt = prefill ? 0 : head_pack_mt(ctx, rows, N, tap_head);
        if (fold) flush_residual(ctx, x, batch);
        else norm_rows(ctx, x, batch, ctx->final_norm, hmt);
        if (tap_head) tap_dense(ctx, TTSBB_TAP_HEAD_IN, ctx->h, ctx->dt, batch, g.hidden, g.hidden);
        float *lg = logits ? logits : ctx->logits;
        head_gemm(ctx, head, rows, N, lg, N, r0, fold ? x : nullptr, hmt);
        if (ctx->tap_layer >= 0) tap_dense(ctx, TTSBB_TAP_LOGITS, lg, DT_F32, rows, N, N);
        {
            KScope k(ctx, TTSBB_K_ARGMAX);
            launch_argmax_groups(lg, rows, N, n_groups, group_vocab, argmax, ctx->flag, ctx->stream);
        }
    }
    if (prefill) launch_increment(positions, 1, ctx->stream, batch);
    else launch_increment(positions, batch, ctx->stream);
    return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_decode_step(ttsbb_ctx *ctx, int32_t batch, float *x, int32_t *positions,
                                         const int32_t *page_table, int32_t max_pages, void *kv_pool,
                                         int32_t n_pages, const void *head, int32_t n_groups,
                                         int32_t group_vocab, int32_t *argmax, float *logits) {
    return paged_forward(ctx, batch, x, positions, page_table, max_pages, kv_pool, n_pages, head, n_groups,
                         group_vocab, argmax, logits, false);
}

namespace {

// The per-call scratch of a decode step, pointed at the context's workspace or at the
// static scratch array.
struct Work {
    void *h, *q, *attn, *mlp;
    float *qkv, *part, *logits, *gpart;
    int64_t gpart_cap;
    int4 *plan;
    int *plan_n, *plan_pages;
    int2 *seg_cont;
    int *plan_nc;
    int work_rows;
};

Work work_of(const ttsbb_ctx *c) {
    return Work{c->h, c->q, c->attn, c->mlp, c->qkv, c->part, c->logits, c->gpart, c->gpart_cap,
                c->plan, c->plan_n, c->plan_pages, c->seg_cont, c->plan_nc, c->work_rows};
}

void set_work(ttsbb_ctx *c, const Work &w) {
    c->h = w.h; c->q = w.q; c->attn = w.attn; c->mlp = w.mlp;
    c->qkv = w.qkv; c->part = w.part; c->logits = w.logits; c->gpart = w.gpart; c->gpart_cap = w.gpart_cap;
    c->plan = w.plan; c->plan_n = w.plan_n; c->plan_pages = w.plan_pages; c->work_rows = w.work_rows;
    c->seg_cont = w.seg_cont; c->plan_nc = w.plan_nc;
}

// Carve the static scratch into a decode step's buffers for STATIC_MAX_BATCH rows of this
// context's shape; false when they do not fit.
bool static_work(const ttsbb_ctx *c, Work &w) {
    const ttsbb_config &g = c->cfg;
    const size_t R = STATIC_MAX_BATCH, hd_all = (size_t)g.n_heads * g.head_dim;
    unsigned char *base = reinterpret_cast<unsigned char *>(c->static_scratch);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        void *p = base + off;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    w.h = take(R * g.hidden * c->esz);
    w.q = take(R * hd_all * 4);
    w.attn = take(R * hd_all * c->esz);
    w.mlp = take(R * g.ffn * c->esz);
    w.qkv = reinterpret_cast<float *>(take(R * c->qkv_w * 4));
    w.part = reinterpret_cast<float *>(take(R * g.n_heads * MAX_CHUNKS * PART_STRIDE * 4));
    w.logits = reinterpret_cast<float *>(take(R * STATIC_MAX_HEAD_COLS * 4));
    // only the residual-add products (N = hidden) are split over K on these rows
    w.gpart_cap = (int64_t)STATIC_GPART_SPLITS * R * g.hidden;
    w.gpart = reinterpret_cast<float *>(take((size_t)w.gpart_cap * 4));
    w.plan = reinterpret_cast<int4 *>(take(plan_entries(c, R) * sizeof(int4)));
    w.plan_n = reinterpret_cast<int *>(take(256));
    w.plan_pages = reinterpret_cast<int *>(take(plan_entries(c, R) * 64 * sizeof(int)));
    w.seg_cont = reinterpret_cast<int2 *>(take((size_t)SEG_PER_CU * c->n_cu * sizeof(int2)));
    w.plan_nc = reinterpret_cast<int *>(take(R * sizeof(int)));
    w.work_rows = (int)R;
    return base != nullptr && off <= STATIC_SCRATCH_BYTES;
}

}  // namespace

TTSBB_API ttsbb_status ttsbb_decode_step_noalloc(ttsbb_ctx *ctx, int32_t batch, float *x, int32_t *positions,
                                                 const int32_t *page_table, int32_t max_pages, void *kv_pool,
                                                 int32_t n_pages, const void *head, int32_t n_groups,
                                                 int32_t group_vocab, int32_t *argmax, float *logits) {
    if (!ctx) return TTSBB_INVALID_ARG;
    if (batch > STATIC_MAX_BATCH) return TTSBB_UNSUPPORTED;
    if (head && (int64_t)n_groups * group_vocab > STATIC_MAX_HEAD_COLS) return TTSBB_UNSUPPORTED;
    if (!ctx->static_scratch) return TTSBB_DEVICE_ERROR;
    Work w;
    if (!static_work(ctx, w)) return TTSBB_UNSUPPORTED;  // this context's shape needs more than the array
    const Work own = work_of(ctx);
    set_work(ctx, w);
    const ttsbb_status st = paged_forward(ctx, batch, x, positions, page_table, max_pages, kv_pool, n_pages, head,
                                          n_groups, group_vocab, argmax, logits, false);
    set_work(ctx, own);
    return st;
}

TTSBB_API ttsbb_status ttsbb_prefill(ttsbb_ctx *ctx, int32_t n_tokens, float *x, int32_t *cache_len,
                                     const int32_t *page_table, int32_t max_pages, void *kv_pool, int32_t n_pages,
                                     const void *head, int32_t n_groups, int32_t group_vocab, int32_t *argmax,
                                     float *logits) {
    return paged_forward(ctx, n_tokens, x, cache_len, page_table, max_pages, kv_pool, n_pages, head, n_groups,
                         group_vocab, argmax, logits, true);
}

TTSBB_API ttsbb_status ttsbb_maskgit_pass(ttsbb_ctx *ctx, int32_t n_text, const int32_t *text_ids,
                                          const void *text_table, int32_t text_vocab,
                                          int32_t n_frames, int32_t n_cb, int32_t cb_vocab,
                                          int32_t mask_id, const void *audio_tables,
                                          const void *audio_heads, int32_t *codes,
                                          int32_t n_unmask, float layer_penalty, int32_t *pred,
                                          float *conf, int32_t *picked) {
    if (!ctx) return TTSBB_INVALID_ARG;
    const ttsbb_config &g = ctx->cfg;
    ctx->pend_splits = 0;
    if (n_text < 0 || n_frames <= 0 || n_cb <= 0 || cb_vocab <= 0 || mask_id < 0 ||
        mask_id >= cb_vocab || n_unmask < 0 || (int64_t)n_unmask > (int64_t)n_cb * n_frames)
        return TTSBB_INVALID_ARG;
    if ((int64_t)n_text + n_frames > g.max_rows || (int64_t)n_text + n_frames > g.max_pos) return TTSBB_INVALID_ARG;
    if ((int64_t)n_cb * cb_vocab > g.max_head_cols) return TTSBB_INVALID_ARG;
    if ((int64_t)n_cb * n_frames > ctx->rank_cap) return TTSBB_INVALID_ARG;
    if (n_text > 0 && (!text_ids || !text_table || text_vocab <= 0)) return TTSBB_INVALID_ARG;
    if (!audio_tables || !audio_heads || !codes || !pred || !conf || (n_unmask > 0 && !picked) ||
        !ctx->final_norm)
        return TTSBB_INVALID_ARG;
    if (!(layer_penalty == layer_penalty)) return TTSBB_INVALID_ARG;

    const int S = n_text + n_frames;
    const int N = n_cb * cb_vocab;
    maskgit_embed(ctx, S, n_text, text_ids, text_table, text_vocab, n_cb, cb_vocab, audio_tables, codes, n_frames);
    maskgit_layers(ctx, S, 0, S, 0, true);
    if (!maskgit_head_scores(ctx, n_text, n_frames, audio_heads, n_cb, cb_vocab, mask_id, layer_penalty, codes,
                             n_frames, pred, conf)) {
        maskgit_head(ctx, n_text, n_frames, audio_heads, N, ctx->logits, true);
        if (ctx->tap_layer >= 0) tap_dense(ctx, TTSBB_TAP_LOGITS, ctx->logits, DT_F32, n_frames, N, N);
        KScope k(ctx, TTSBB_K_SCORES);
        launch_maskgit_scores(ctx->logits, nullptr, 0.f, n_frames, N, n_cb, cb_vocab, mask_id, layer_penalty, codes,
                              n_frames, pred, conf, ctx->flag, ctx->stream);
    }
    {
        KScope k(ctx, TTSBB_K_SELECT);
        launch_select_update(conf, pred, n_cb, n_frames, n_unmask, ctx->rank, codes, n_frames, picked, ctx->stream);
    }
    return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_maskgit_pass_cfg(ttsbb_ctx *ctx, int32_t n_text, const int32_t *text_ids,
                                              const void *text_table, int32_t text_vocab, int32_t n_frames,
                                              int32_t n_target, int32_t n_cb, int32_t cb_vocab, int32_t mask_id,
                                              const void *audio_tables, const void *audio_heads, int32_t *codes,
                                              int32_t n_unmask, float layer_penalty, float cfg_scale, int32_t *pred,
                                              float *conf, int32_t *picked) {
    if (!ctx) return TTSBB_INVALID_ARG;
    const ttsbb_config &g = ctx->cfg;
    ctx->pend_splits = 0;
    if (n_text < 0 || n_frames <= 0 || n_target <= 0 || n_target > n_frames || n_cb <= 0 || cb_vocab <= 0 ||
        mask_id < 0 || mask_id >= cb_vocab || n_unmask < 0 || (int64_t)n_unmask > (int64_t)n_cb * n_target)
        return TTSBB_INVALID_ARG;
    if ((int64_t)n_text + n_frames > g.max_rows || (int64_t)n_text + n_frames > g.max_pos) return TTSBB_INVALID_ARG;
    if ((int64_t)n_cb * cb_vocab > g.max_head_cols) return TTSBB_INVALID_ARG;
    if ((int64_t)n_cb * n_target > ctx->rank_cap) return TTSBB_INVALID_ARG;
    if (n_text > 0 && (!text_ids || !text_table || text_vocab <= 0)) return TTSBB_INVALID_ARG;
    if (!audio_tables || !audio_heads || !codes || !pred || !conf || (n_unmask > 0 && !picked) ||
        !ctx->final_norm)
        return TTSBB_INVALID_ARG;
    if (!(layer_penalty == layer_penalty) || !(cfg_scale == cfg_scale)) return TTSBB_INVALID_ARG;

    const int w0 = n_frames - n_target;
    const int N = n_cb * cb_vocab;
    int32_t *window = codes + w0;  // element (k, t) of the window at window[k * n_frames + t]
    // conditional pass (the whole prompt, logits on the window's rows) and unconditional
    // pass (the window's frames alone, positions 0..n_target-1)
    maskgit_guided(ctx, n_text, text_ids, text_table, text_vocab, n_frames, n_target, n_cb, cb_vocab, audio_tables,
                   audio_heads, codes);
    {
        KScope k(ctx, TTSBB_K_SCORES);
        launch_maskgit_scores(ctx->logits, ctx->logits_u, cfg_scale, n_target, N, n_cb, cb_vocab, mask_id,
                              layer_penalty, window, n_frames, pred, conf, ctx->flag, ctx->stream);
    }
    {
        KScope k(ctx, TTSBB_K_SELECT);
        launch_select_update(conf, pred, n_cb, n_target, n_unmask, ctx->rank, window, n_frames, picked, ctx->stream);
    }
    return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_maskgit_step(ttsbb_ctx *ctx, const ttsbb_maskgit_step_args *a) {
    if (!ctx || !a) return TTSBB_INVALID_ARG;
    const ttsbb_config &g = ctx->cfg;
    ctx->pend_splits = 0;
    const int n_text = a->n_text, n_frames = a->n_frames, n_target = a->n_target, n_cb = a->n_cb;
    const int cb_vocab = a->cb_vocab, mask_id = a->mask_id, n_unmask = a->n_unmask;
    if (n_text < 0 || n_frames <= 0 || n_target <= 0 || n_target > n_frames || n_cb <= 0 || cb_vocab <= 0 ||
        mask_id < 0 || mask_id >= cb_vocab || n_unmask < 0 || (int64_t)n_unmask > (int64_t)n_cb * n_target)
        return TTSBB_INVALID_ARG;
    if ((int64_t)n_text + n_frames > g.max_rows || (int64_t)n_text + n_frames > g.max_pos) return TTSBB_INVALID_ARG;
    if ((int64_t)n_cb * cb_vocab > g.max_head_cols) return TTSBB_INVALID_ARG;
    if ((int64_t)n_cb * n_target > ctx->rank_cap) return TTSBB_INVALID_ARG;
    if (n_text > 0 && (!a->text_ids || !a->text_table || a->text_vocab <= 0)) return TTSBB_INVALID_ARG;
    if (!a->audio_tables || !a->audio_heads || !a->codes || !a->pred || !a->conf || (n_unmask > 0 && !a->picked) ||
        !ctx->final_norm)
        return TTSBB_INVALID_ARG;
    const float temps[5] = {a->layer_penalty, a->cfg_scale, a->class_temp, a->pos_temp, a->top_k_ratio};
    for (float v : temps)
        if (!(v == v)) return TTSBB_INVALID_ARG;
    if (a->class_temp < 0.f || a->pos_temp < 0.f) return TTSBB_INVALID_ARG;
    const bool draw_class = a->class_temp > 0.f && !a->u_class, draw_pos = a->pos_temp > 0.f && !a->u_pos;
    if (a->class_temp > 0.f && (!(a->top_k_ratio > 0.f) || cb_vocab > 2048)) return TTSBB_INVALID_ARG;
    if ((draw_class || draw_pos) && !a->rng_counter) return TTSBB_INVALID_ARG;

    const int S = n_text + n_frames, w0 = n_frames - n_target;
    const int N = n_cb * cb_vocab;
    int32_t *window = a->codes + w0;
    const float *lu = nullptr;
    const bool sampled = a->class_temp > 0.f || a->pos_temp > 0.f;
    bool scored = false;  // pred and conf already written by the fused head
    if (a->cfg_scale != 0.f) {
        maskgit_guided(ctx, n_text, a->text_ids, a->text_table, a->text_vocab, n_frames, n_target, n_cb, cb_vocab,
                       a->audio_tables, a->audio_heads, a->codes);
        lu = ctx->logits_u;
    } else {
        maskgit_embed(ctx, S, n_text, a->text_ids, a->text_table, a->text_vocab, n_cb, cb_vocab, a->audio_tables,
                      a->codes, n_frames);
        maskgit_layers(ctx, S, 0, S, 0, true);
        scored = !sampled && maskgit_head_scores(ctx, n_text + w0, n_target, a->audio_heads, n_cb, cb_vocab, mask_id,
                                                 a->layer_penalty, window, n_frames, a->pred, a->conf);
        if (!scored) {
            maskgit_head(ctx, n_text + w0, n_target, a->audio_heads, N, ctx->logits, true);
            if (ctx->tap_layer >= 0) tap_dense(ctx, TTSBB_TAP_LOGITS, ctx->logits, DT_F32, n_target, N, N);
        }
    }
    if (!scored) {
        KScope k(ctx, TTSBB_K_SCORES);
        if (sampled) {
            const int k_keep = std::max(1, (int)floor((double)a->top_k_ratio * cb_vocab));
            launch_maskgit_sample(ctx->logits, lu, a->cfg_scale, n_target, N, n_cb, cb_vocab, mask_id,
                                  a->layer_penalty, window, n_frames, a->class_temp, a->pos_temp, k_keep, a->u_class,
                                  a->u_pos, a->rng_seed, a->rng_counter, a->pred, a->conf, ctx->flag, ctx->stream);
        } else {
            launch_maskgit_scores(ctx->logits, lu, a->cfg_scale, n_target, N, n_cb, cb_vocab, mask_id,
                                  a->layer_penalty, window, n_frames, a->pred, a->conf, ctx->flag, ctx->stream);
        }
    }
    if (draw_class || draw_pos)  // the call's draws span ceil(n_cb n_target cb_vocab / 4) counter blocks
        launch_advance_counter(a->rng_counter, ((uint64_t)n_cb * n_target * cb_vocab + 3) / 4, ctx->stream);
    {
        KScope k(ctx, TTSBB_K_SELECT);
        launch_select_update(a->conf, a->pred, n_cb, n_target, n_unmask, ctx->rank, window, n_frames, a->picked,
                             ctx->stream);
    }
    return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_rvq_decode(ttsbb_ctx *ctx, int32_t n_frames, int32_t n_q, int32_t codebook_size,
                                        int32_t codebook_dim, int32_t out_dim, const int32_t *codes,
                                        const float *embed, const float *proj_w, const float *proj_b, float *out) {
    if (!ctx || n_frames < 0 || n_q <= 0 || codebook_size <= 0 || codebook_dim <= 0 || out_dim <= 0)
        return TTSBB_INVALID_ARG;
    if (n_frames == 0) return TTSBB_OK;
    if (!codes || !embed || !proj_w || !proj_b || !out) return TTSBB_INVALID_ARG;
    RvqArgs r;
    r.n_frames = n_frames;
    r.n_q = n_q;
    r.cb_size = codebook_size;
    r.dim = codebook_dim;
    r.out_dim = out_dim;
    r.codes = codes;
    r.embed = embed;
    r.proj_w = proj_w;
    r.proj_b = proj_b;
    r.out = out;
    r.flag = ctx->flag;
    {
        KScope k(ctx, TTSBB_K_RVQ, true);
        launch_rvq_decode(r, ctx->stream, k.start(), k.stop());
    }
    return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_philox_words(ttsbb_ctx *ctx, uint64_t seed, uint64_t block0, uint32_t word2,
                                          uint32_t word3, int32_t n_blocks, uint32_t *out) {
    if (!ctx || n_blocks < 0) return TTSBB_INVALID_ARG;
    if (n_blocks == 0) return TTSBB_OK;
    if (!out) return TTSBB_INVALID_ARG;
    launch_rng_words(seed, block0, word2, word3, n_blocks, out, ctx->stream);
    return launch_failed() ? TTSBB_DEVICE_ERROR : TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_unmask_schedule(int32_t n_total, int32_t n_steps, int32_t *out) {
    if (n_total < 0 || n_steps <= 0 || !out) return TTSBB_INVALID_ARG;
    const double PI = 3.14159265358979323846;
    int left = n_total;
    for (int i = 0; i < n_steps; ++i) {
        int n;
        if (i == n_steps - 1) {
            n = left;
        } else {
            const double t0 = 1.0 - cos(0.5 * PI * i / n_steps);
            const double t1 = 1.0 - cos(0.5 * PI * (i + 1) / n_steps);
            n = (int)ceil((double)n_total * (t1 - t0));
            if (n > left) n = left;
        }
        out[i] = n;
        left -= n;
    }
    return TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_set_tap_layer(ttsbb_ctx *ctx, int32_t layer) {
    if (!ctx || layer < -1 || layer >= (ctx->cfg.n_layers > 0 ? ctx->cfg.n_layers : 1))
        return TTSBB_INVALID_ARG;
    ctx->tap_layer = layer;
    if (layer < 0) return TTSBB_OK;
    for (int t = 0; t < TTSBB_TAP_COUNT; ++t) {
        if (ctx->taps[t].buf) continue;
        const size_t bytes = (size_t)ctx->cfg.max_rows * tap_width(ctx, t) * sizeof(float);
        if (hipMalloc((void **)&ctx->taps[t].buf, bytes) != hipSuccess) {
            ctx->taps[t].buf = nullptr;
            hipGetLastError();
            return TTSBB_OOM;
        }
    }
    return TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_read_tap(ttsbb_ctx *ctx, int32_t tap, float *dst, int64_t n_floats,
                                      int32_t *rows, int32_t *cols) {
    if (!ctx || tap < 0 || tap >= TTSBB_TAP_COUNT || !dst) return TTSBB_INVALID_ARG;
    const Tap &t = ctx->taps[tap];
    if (!t.buf) return TTSBB_INVALID_ARG;
    const int64_t n = (int64_t)t.rows * t.cols;
    if (n_floats < n) return TTSBB_INVALID_ARG;
    if (rows) *rows = t.rows;
    if (cols) *cols = t.cols;
    if (n == 0) return TTSBB_OK;
    if (hipMemcpyAsync(dst, t.buf, (size_t)n * sizeof(float), hipMemcpyDeviceToDevice, ctx->stream) != hipSuccess)
        return TTSBB_DEVICE_ERROR;
    return TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_profile_start(ttsbb_ctx *ctx, uint32_t mask, int32_t max_launches) {
    if (!ctx || max_launches < 0) return TTSBB_INVALID_ARG;
    Prof &p = ctx->prof;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess) return TTSBB_DEVICE_ERROR;
    if (p.cap < max_launches) {
        prof_release(p);
        p.ev.resize(2 * (size_t)max_launches);
        // timing-only events: no system-scope fence (cache write-back / invalidate) at
        // record time, so they perturb the timed kernels less; profile_stop synchronizes
        // the stream before reading them
        for (auto &e : p.ev)
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
                e = nullptr;
                prof_release(p);
                return TTSBB_DEVICE_ERROR;
            }
        p.cls.assign(max_launches, 0);
        p.cap = max_launches;
    }
    p.used = 0;
    p.mask = mask;
    return TTSBB_OK;
}

TTSBB_API ttsbb_status ttsbb_profile_stop(ttsbb_ctx *ctx, float *ms, int32_t *launches) {
    if (!ctx) return TTSBB_INVALID_ARG;
    Prof &p = ctx->prof;
    p.mask = 0;
    if (ms)
        for (int k = 0; k < TTSBB_K_COUNT; ++k) ms[k] = 0.f;
    if (launches)
        for (int k = 0; k < TTSBB_K_COUNT; ++k) launches[k] = 0;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess) return TTSBB_DEVICE_ERROR;
    for (int i = 0; i < p.used; ++i) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) return TTSBB_DEVICE_ERROR;
        if (ms) ms[p.cls[i]] += t;
        if (launches) launches[p.cls[i]] += 1;
    }
    p.used = 0;
    return TTSBB_OK;
}
