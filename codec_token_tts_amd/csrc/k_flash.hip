// K6: bidirectional attention of the MaskGIT pass (OmniVoice ARCHITECTURE, "MaskGIT
// decoder": every step is a full prefill with fully bidirectional attention, no KV
// cache across steps).  Flash-style: keys stream through LDS in blocks of 32 with an
// online softmax, so the S x S score matrix never exists.
//
// Both products run on v_mfma_f32_32x32x16_bf16 (on gfx950 about 1.75x the flop rate of
// the 16x16x32 form) in transposed form, so that a lane's accumulators always belong to
// one query (column lane % 32):
//   S^T (32 keys x 32 queries) = K (32 x 128) * Q^T (128 x 32)        8 products
//   O^T (32 dims x 32 queries) = V^T (32 x 32) * P^T (32 x 32)         2 products / tile
// Lane l holds S^T rows 8j + 4(l/32) + i (j, i < 4) of query l%32, so the softmax
// statistics of a query live in lanes l and l^32.  The K tile's LDS row r holds key
// pi(r), pi swapping bits 2 and 3 of the row index, so that the keys of accumulator
// entries 8kk .. 8kk + 7 of lane l are the 8 consecutive keys 16kk + 8(l/32) ..: P^T
// feeds the second product straight from registers, and its V^T operand (V stored
// transposed, [Hkv][128][s_pad]) is one 16-byte LDS read per lane (the 80-byte row
// stride keeps 8 consecutive rows on distinct banks).
//
// Block = 8 waves = 4 key quarters x 2 waves.  The two waves of a quarter are the two
// query heads of a GQA group over the same 32 queries (or, without GQA, two query
// tiles of one head): they share the quarter's double-buffered K / V^T tiles in LDS.
// Every quarter runs the same number of iterations (a quarter past its last block
// processes masked copies) so that the block barriers match; at the end quarters 1-3
// hand their (max, sum, O^T) to quarter 0 through LDS, which merges the four
// online-softmax states in quarter order and stores.  The causal form (the prefill:
// query row i at position p0 + i sees keys 0..p0 + i, over the stream's whole sequence
// gathered from the paged pool) is the same loop over the keys below the tile's last
// query, with the keys past each query masked.  Scores are scaled by
// log2(e)/sqrt(128) inside the exponent (one FMA) and exponentiated with v_exp_f32;
// the running reference max is raised lazily (see the loop).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ttsbb {

constexpr int FB = 32;         // keys per block
constexpr int LDKF = 128 + 8;  // K tile row stride (elements)
constexpr int LDVF = FB + 8;   // V^T tile row stride (elements)
constexpr int KTILE = FB * LDKF, VTILE = 128 * LDVF;

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// Global -> register staging of one 32-key block of K (8 KB) and V^T (8 KB) by the 128
// threads of a quarter: copy c takes K row 8c + qtid / 16 (16-byte chunk qtid % 16) and
// V^T row 32c + qtid / 4 (keys 8 (qtid % 4) .. +7).  klane / vlane hold the thread's part
// of the addresses, so a copy adds only the block's first key and a constant (K) or a
// scalar stride (V^T) -- no per-copy index arithmetic on the VALU.
__device__ __forceinline__ void flash_gload(const bf16_t *klane, const bf16_t *vlane, int s_pad, int kb0,
                                            u32x4_t (&rk)[4], u32x4_t (&rv)[4]) {
    const bf16_t *kl = klane + (int64_t)kb0 * 128;
    const bf16_t *vl = vlane + kb0;
    const int64_t vstride = (int64_t)32 * s_pad;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        rk[c] = *reinterpret_cast<const u32x4_t *>(kl + c * 1024);
        rv[c] = *reinterpret_cast<const u32x4_t *>(vl + c * vstride);
    }
}

__device__ __forceinline__ void flash_sstore(bf16_t *sk, bf16_t *sv, int qtid, const u32x4_t (&rk)[4],
                                             const u32x4_t (&rv)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int ch = qtid + 128 * c;
        const int key = ch >> 4;  // stored at row pi(key): bits 2 and 3 swapped
        const int row = (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
        *reinterpret_cast<u32x4_t *>(&sk[row * LDKF + (ch & 15) * 8]) = rk[c];
        *reinterpret_cast<u32x4_t *>(&sv[(ch >> 2) * LDVF + (ch & 3) * 8]) = rv[c];
    }
}

template <int GROUP>
__global__ __launch_bounds__(512) void flash_kernel(FlashArgs a) {
    // [quarter][buffer] K tiles, then V^T tiles; reused at the end for the hand-over of
    // quarters 1-3 (one array, so the hand-over may span both parts)
    __shared__ __attribute__((aligned(16))) bf16_t smem[8 * (KTILE + VTILE)];
    bf16_t(*sK)[2][KTILE] = reinterpret_cast<bf16_t(*)[2][KTILE]>(smem);
    bf16_t(*sV)[2][VTILE] = reinterpret_cast<bf16_t(*)[2][VTILE]>(smem + 8 * KTILE);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qq = wave >> 1, u = wave & 1, qtid = tid & 127;
    // blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8): taking the
    // KV head from b % Hkv keeps each head's K / V^T (486 KB at S = 950) in one XCD's L2
    const int hk = blockIdx.x % a.Hkv, qtile = blockIdx.x / a.Hkv;
    const int head = GROUP == 2 ? hk * 2 + u : hk;
    const int q0 = (GROUP == 2 ? qtile : qtile * 2 + u) * 32;
    const int fq = lane & 31, h = lane >> 5;
    const int ldq = a.H * 128;

    // Q^T operand: lane -> query q0 + fq, dims ks*16 + 8h .. +7
    bf16x8_t qf[8];
    {
        const int qi = min(q0 + fq, a.S - 1);  // queries past S compute unused columns
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8_t *>(a.q + (int64_t)qi * ldq + head * 128 + ks * 16 + h * 8);
    }

    const bf16_t *kg = a.k + (int64_t)hk * a.s_pad * 128;
    const bf16_t *vg = a.vt + (int64_t)hk * 128 * a.s_pad;
    // the keys of the tile's sequence: [kb, ke) (a tile never straddles two sequences)
    const bool second = a.seg1 > 0 && q0 >= a.seg1;
    // causal: query row i is at position p0 + i and sees keys [0, p0 + i]; the tile needs
    // keys below p0 + q0 + 32, and every query of it sees the keys below p0 + q0 + 1
    const bool causal = a.causal_pos != nullptr;
    const int p0 = causal ? min(max(a.causal_pos[0], 0), a.s_pad - a.S) : 0;
    const int kb = second ? a.seg1 : 0;
    const int ke = causal ? min(p0 + a.S, p0 + q0 + 32) : kb + (second ? a.len1 : a.len0);
    const int k_all = causal ? min(ke, p0 + q0 + 1) : ke;  // keys below: unmasked for the whole tile
    const int q_pos = p0 + q0 + fq;                           // this lane's query position (causal)
    const int NB = (ke - kb + FB - 1) / FB, NBQ = (NB + 3) / 4;
    const int kb_first = qq * NBQ, nb_mine = max(0, min(NBQ, NB - kb_first));
    // iteration i works on block blk(i); past this quarter's blocks it re-reads a valid
    // block and masks every key
    auto blk = [&](int i) { return min(kb_first + max(0, min(i, nb_mine - 1)), NB - 1); };
    bf16_t *sk0 = sK[qq][0], *sk1 = sK[qq][1], *sv0 = sV[qq][0], *sv1 = sV[qq][1];

    f32x16_t o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    u32x4_t rk[4], rv[4];
    const bf16_t *klane = kg + (qtid >> 4) * 128 + (qtid & 15) * 8;
    const bf16_t *vlane = vg + (int64_t)(qtid >> 2) * a.s_pad + (qtid & 3) * 8;
    flash_gload(klane, vlane, a.s_pad, kb + blk(0) * FB, rk, rv);
    flash_sstore(sk0, sv0, qtid, rk, rv);
    __syncthreads();
    for (int i = 0; i < NBQ; ++i) {
        const int buf = i & 1;
        const bf16_t *sk = buf ? sk1 : sk0;
        const bf16_t *sv = buf ? sv1 : sv0;
        flash_gload(klane, vlane, a.s_pad, kb + blk(i + 1) * FB, rk, rv);  // unconditional (clamped)
        // keep the prefetch at the top of the iteration: it has the whole block to arrive
        __builtin_amdgcn_sched_barrier(0);
        const bool valid = i < nb_mine;
        const int kbase = kb + blk(i) * FB;

        bf16x8_t kf[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            kf[ks] = *reinterpret_cast<const bf16x8_t *>(&sk[fq * LDKF + ks * 16 + h * 8]);
        // The two waves of a SIMD reach the score products together; the wave that issues
        // them first at raised priority runs its chain while the other waits for the matrix
        // core, then its softmax overlaps the other's products (21.7 -> 20.7 us; a fixed
        // priority per wave, or raising it for the V products too, did no better).
        __builtin_amdgcn_s_setprio(1);
        f32x16_t s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        // V^T fragments are independent of the softmax: their reads overlap it
        bf16x8_t vfr[4][2];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                vfr[dt][kk] = *reinterpret_cast<const bf16x8_t *>(&sv[(dt * 32 + fq) * LDVF + kk * 16 + h * 8]);
            }
        // mask keys past the sequence (and the blocks of a finished quarter): only partial blocks
        if (!(valid && kbase + FB <= k_all)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kbase + (r >> 3) * 16 + h * 8 + (r & 7);
                if (!(valid && key < ke && (!causal || key <= q_pos))) s[r] = -INFINITY;
            }
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE)) * a.scale_log2;  // scale > 0 commutes with max
        // Lazy rescaling: the weights are taken relative to a reference max m_ref that is
        // raised (and O, l rescaled) only when some query of the wave sees a score more
        // than 2^8 above it, so a weight never exceeds 2^8 and most blocks skip the
        // rescale.  The normalisation by l at the end cancels the reference.
        if (__any(mx > m_run + 8.0f)) {
            const float m_new = fmaxf(m_run, mx);
            const float sc = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
            m_run = m_new;
            l_run *= sc;
#pragma unroll
            for (int d = 0; d < 4; ++d) o[d] *= sc;
        }
        const float m_neg = m_run == -INFINITY ? 0.f : -m_run;  // nothing seen yet: all weights 0

        // P^T operand of the 16-key chunk kk: slot e <- accumulator entry 8kk + e, i.e.
        // key 16kk + 8h + e
        bf16x8_t pb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + e], a.scale_log2, m_neg));
                l_run += p;
                pb[kk][e] = (__bf16)p;
            }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[dt][kk], pb[kk], o[dt], 0, 0, 0);
        if (i + 1 < NBQ) flash_sstore(buf ? sk0 : sk1, buf ? sv0 : sv1, qtid, rk, rv);
        __syncthreads();
    }

    // hand-over: quarters 1-3 -> quarter 0 through the (now idle) tiles; 66 values per
    // lane, stored with a stride of 128 lanes (the two waves of a quarter side by side)
    float *ex = reinterpret_cast<float *>(smem);
    constexpr int EXS = 66 * 128;  // floats per quarter
    static_assert(3 * EXS * 4 <= 8 * (KTILE + VTILE) * 2, "hand-over fits the tiles");
    if (qq > 0) {
        float *e = ex + (qq - 1) * EXS + u * 64 + lane;
        e[0] = m_run;
        e[128] = l_run;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) e[(2 + d * 16 + r) * 128] = o[d][r];
    }
    __syncthreads();
    if (qq > 0) return;
    {
        float mq[3], M = m_run;  // finite: quarter 0 always holds key 0 (the references merge
                                 // like maxima: each state is exact relative to its own)
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            mq[k] = ex[k * EXS + u * 64 + lane];
            M = fmaxf(M, mq[k]);
        }
        const float f0 = exp2f(m_run - M);
        l_run *= f0;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] *= f0;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const float *e = ex + k * EXS + u * 64 + lane;
            const float f = exp2f(mq[k] - M);  // an empty quarter (reference -inf) weighs 0
            l_run += e[128] * f;
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[d][r] += e[(2 + d * 16 + r) * 128] * f;
        }
    }

    l_run += __shfl_xor(l_run, 32, WAVE);
    const float inv = 1.0f / l_run;
    // O goes out through LDS, past the hand-over area, each wave in rows of its own (row
    // stride 272 bytes: 8-byte writes of 32 queries spread over the banks); read back, 16
    // consecutive lanes then store one query's whole 256-byte row of O (before: each
    // store touched 32 rows)
    constexpr int OST = 272;
    static_assert(3 * EXS * 4 + 2 * 32 * OST <= 8 * (KTILE + VTILE) * 2, "O staging fits");
    unsigned char *stg = reinterpret_cast<unsigned char *>(smem) + 3 * EXS * 4 + u * 32 * OST;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint2 w;
            w.x = (uint32_t)f32_to_bf16(o[dt][4 * j] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * j + 1] * inv) << 16);
            w.y = (uint32_t)f32_to_bf16(o[dt][4 * j + 2] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * j + 3] * inv) << 16);
            *reinterpret_cast<uint2 *>(stg + fq * OST + (dt * 32 + j * 8 + h * 4) * 2) = w;
        }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int row = it * 4 + (lane >> 4), c16 = lane & 15, qi = q0 + row;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stg + row * OST + c16 * 16);
        if (qi < a.S) *reinterpret_cast<u32x4_t *>(a.out + (int64_t)qi * ldq + head * 128 + c16 * 8) = v;
    }
}

void launch_flash_attn(const FlashArgs &a, hipStream_t s) {
    if (a.S <= 0) return;
    const int group = a.H / a.Hkv;
    const int qpb = group == 2 ? 32 : 64;  // queries per block
    const dim3 grid(((a.S + qpb - 1) / qpb) * a.Hkv);
    if (group == 2) hipLaunchKernelGGL(flash_kernel<2>, grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL(flash_kernel<1>, grid, dim3(512), 0, s, a);
}

}  // namespace ttsbb

namespace ttsbb {

// fp32 form of the bidirectional attention (the MaskGIT pass of an fp32 context): plain
// fp32 arithmetic, no MFMA.  One wave per (query row, head): lane l holds dims 2l, 2l + 1
// of q and of the output; each key's score is a wave sum, the softmax is online (running
// max m, normaliser l, output rescaled when m rises) with expf.  Rows [0, len0) attend to
// keys [0, len0); with seg1 > 0, rows [seg1, seg1 + len1) to keys [seg1, seg1 + len1);
// padding rows between get zeros.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnF32Args a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), head = blockIdx.y;
    if (row >= a.S) return;
    const int kvh = head / (a.H / a.Hkv);
    const bool second = a.seg1 > 0 && row >= a.seg1;
    const int kb = second ? a.seg1 : 0, ke = kb + (second ? a.len1 : a.len0);
    float *out = a.out + (int64_t)row * a.H * 128 + head * 128 + 2 * lane;
    if (row >= ke) {  // padding row
        out[0] = 0.f;
        out[1] = 0.f;
        return;
    }
    const float *q = a.q + (int64_t)row * a.H * 128 + head * 128 + 2 * lane;
    const float q0 = q[0] * a.scale, q1 = q[1] * a.scale;
    const float *K = a.k + (int64_t)kvh * a.s_pad * 128 + 2 * lane;
    const float *V = a.v + (int64_t)kvh * a.s_pad * 128 + 2 * lane;
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int j = kb; j < ke; ++j) {
        const float s = wave_sum(fmaf(q0, K[(int64_t)j * 128], q1 * K[(int64_t)j * 128 + 1]));
        if (s > m) {  // wave-uniform: s is a wave sum
            const float f = expf(m - s);  // m = -inf at the first key: 0
            l *= f;
            o0 *= f;
            o1 *= f;
            m = s;
        }
        const float p = expf(s - m);
        l += p;
        o0 = fmaf(p, V[(int64_t)j * 128], o0);
        o1 = fmaf(p, V[(int64_t)j * 128 + 1], o1);
    }
    out[0] = o0 / l;
    out[1] = o1 / l;
}

void launch_attn_f32(const AttnF32Args &a, hipStream_t s) {
    if (a.S <= 0) return;
    hipLaunchKernelGGL(attn_f32_kernel, dim3((a.S + 3) / 4, a.H), dim3(256), 0, s, a);
}

}  // namespace ttsbb
