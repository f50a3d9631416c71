// K3: the bias-free projections of the decoder layer (OmniVoice ARCHITECTURE, "Qwen3
// 0.6B backbone with custom IO": q/k/v/o and gate/up/down projections without bias, the
// SwiGLU MLP; "Tensor shape and layout": a Linear weight is [out][in], the product is
// A @ W^T).
//
//   Y[M][N] = A[M][K] * W[N][K]^T, both operands K-contiguous, fp32 accumulation.
//
// Kernels (routing in launch_gemm):
// * gemm_lds (M > 64): 32x32x16 MFMA on 128x128 or 64x64 block tiles whose K tiles are
//   fetched by LDS DMA into a ring of buffers several tiles ahead; XCD-aware tile order
//   (each XCD works on a contiguous N range: weight reuse in its L2); split-K with
//   deferred residual update for the hidden-width residual-add products.
// * gemm_skinny (8 < M <= 64, the batched decode step): weight streaming through MFMA,
//   every load issued up front, split-K with deferred residual update.
// * gemm_mfma: 16x16x32 MFMA on register-staged LDS tiles with optional split-K and a
//   reduce kernel: the fallback for M <= 64 shapes the skinny kernel does not take.
// * gemv: weight streaming for M <= 8 and for fp32: each wave owns two output columns,
//   streams their weight rows once with 16-byte loads and reuses them for all M rows.
//
// Epilogues: store fp32, add into the fp32 residual stream (o_proj, down_proj), and
// SwiGLU, where the gate and up weights are read as interleaved groups of 16 rows so
// that silu(gate) * up pairs within a lane's own accumulators.
#include "common.h"
#include "kernels.h"

namespace ttsbb {

// Pointer to row n (logical) of the weight set.
template <typename T>
__device__ __forceinline__ const T *wrow(const WSrc &w, int epi, int n, int K) {
    if (epi == EPI_SWIGLU) {
        const int pair = n >> 5, half = (n >> 4) & 1, r = n & 15;
        const T *base = reinterpret_cast<const T *>(half ? w.p[1] : w.p[0]);
        return base + (int64_t)(pair * 16 + r) * K;
    }
    // select with branches, not a runtime array index: indexing an array of the kernel
    // argument struct would move the struct into scratch memory
    if (w.nseg > 2 && n >= w.start[2]) return reinterpret_cast<const T *>(w.p[2]) + (int64_t)(n - w.start[2]) * K;
    if (w.nseg > 1 && n >= w.start[1]) return reinterpret_cast<const T *>(w.p[1]) + (int64_t)(n - w.start[1]) * K;
    return reinterpret_cast<const T *>(w.p[0]) + (int64_t)n * K;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// ------------------------------------------------------------------------------------
// MFMA tile GEMM (bf16)
// ------------------------------------------------------------------------------------
constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int EPI_PARTIAL = 3;  // fp32 partial sums of one K split: C + z * M * N
constexpr int EPI_QKV = 4;      // fused per-head RMSNorm + RoPE + dense q / K / V^T layout
constexpr int EPI_SCORES = 5;   // per-row, per-group partial log-softmax statistics of the tile

// Tile order: block ids are dealt round-robin to the 8 XCDs, so block b runs on XCD
// b % 8.  Tiles are renumbered so that each XCD receives a contiguous run of the
// N-major tile order (all M tiles of a few N tiles): a weight slice is then fetched
// into one XCD's L2 and reused there by every M tile.
__device__ __forceinline__ int xcd_tile(int b, int n_tiles) {
    const int per = n_tiles / 8;
    const int x = b % 8, i = b / 8;
    if (i < per) return x * per + i;  // the evenly dealt part
    return 8 * per + x;               // the n_tiles % 8 remainder, one per XCD
}

// Pipeline pieces (device functions rather than lambdas: arrays captured by a lambda
// end up in scratch memory, arrays passed by reference to an inlined function stay in
// registers).
template <int ACH, int BCH> struct Stage {
    u32x4_t a[ACH];
    u32x4_t b[BCH];
};

template <int ACH, int BCH>
__device__ __forceinline__ Stage<ACH, BCH> gemm_gload(const bf16_t *const (&arow)[ACH],
                                                      const bf16_t *const (&brow)[BCH], int k0) {
    Stage<ACH, BCH> st;
#pragma unroll
    for (int c = 0; c < ACH; ++c) st.a[c] = *reinterpret_cast<const u32x4_t *>(arow[c] + k0);
#pragma unroll
    for (int c = 0; c < BCH; ++c) st.b[c] = *reinterpret_cast<const u32x4_t *>(brow[c] + k0);
    return st;
}

template <int ACH, int BCH>
__device__ __forceinline__ void gemm_sstore(bf16_t *sa, bf16_t *sb, const int (&aoff)[ACH], const int (&boff)[BCH],
                                            const Stage<ACH, BCH> &st) {
#pragma unroll
    for (int c = 0; c < ACH; ++c) *reinterpret_cast<u32x4_t *>(&sa[aoff[c]]) = st.a[c];
#pragma unroll
    for (int c = 0; c < BCH; ++c) *reinterpret_cast<u32x4_t *>(&sb[boff[c]]) = st.b[c];
}

template <int TM, int TN>
__device__ __forceinline__ void gemm_mma(const bf16_t *sa, const bf16_t *sb, int fr, int fk,
                                         f32x4_t (&acc)[TM][TN]) {
#pragma unroll
    for (int ks = 0; ks < 64 / 32; ++ks) {
        bf16x8_t af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t *>(&sa[(i * 16 + fr) * (64 + 8) + ks * 32 + fk]);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8_t *>(&sb[(j * 16 + fr) * (64 + 8) + ks * 32 + fk]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_mfma(GemmArgs g, int k_split) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int ACH = BM * 8 / 256;  // 16-byte chunks per thread of the A tile
    constexpr int BCH = BN * 8 / 256;
    static_assert(ACH >= 1 && BCH >= 1, "tile too small");
    static_assert(EPI != EPI_SWIGLU || (TN % 2 == 0), "swiglu needs gate/up tile pairs");

    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (g.M + BM - 1) / BM;
    const int tiles_n = (g.N + BN - 1) / BN;
    const int t = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int tile_n = t / tiles_m, tile_m = t % tiles_m;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int k_begin = blockIdx.z * k_split;
    const int KT = min(k_split, g.K - k_begin) / BK;

    const bf16_t *A = reinterpret_cast<const bf16_t *>(g.A);
    const bf16_t *arow[ACH];
    const bf16_t *brow[BCH];
    int aoff[ACH], boff[BCH];
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int ch = tid + 256 * c, r = ch >> 3, kc = (ch & 7) * 8;
        // rows past M read row M-1: they only feed output rows that are never stored,
        // and unconditional loads let the compiler count them in flight
        const int m = min(m0 + r, g.M - 1);
        arow[c] = A + (int64_t)m * g.lda + k_begin + kc;
        aoff[c] = r * LDK + kc;
    }
#pragma unroll
    for (int c = 0; c < BCH; ++c) {
        const int ch = tid + 256 * c, r = ch >> 3, kc = (ch & 7) * 8;
        const int n = min(n0 + r, g.N - 1);  // likewise for columns past N
        // g.epi (not EPI): a split of a SwiGLU product still reads the interleaved rows
        brow[c] = wrow<bf16_t>(g.w, g.epi, n, g.K) + k_begin + kc;
        boff[c] = r * LDK + kc;
    }

    // Two register staging sets: the loads of tile k+2 are issued while tile k is
    // multiplied; tile k+1 (loaded one iteration earlier) goes to LDS after it.  The
    // prefetch tile index is clamped to the last tile (a read past the end re-reads it
    // unused), so the loads are unconditional and their count in flight is static: the
    // wait before each LDS store covers only the set that is being stored.  Staging
    // uses native vector types so that it lives in registers.
    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15, fk = (lane >> 4) * 8;
    const bf16_t *sa0 = &sA[0][wm * WM * LDK], *sa1 = &sA[1][wm * WM * LDK];
    const bf16_t *sb0 = &sB[0][wn * WN * LDK], *sb1 = &sB[1][wn * WN * LDK];
    if (KT > 0) {
        Stage<ACH, BCH> s0 = gemm_gload<ACH, BCH>(arow, brow, 0);
        Stage<ACH, BCH> s1 = gemm_gload<ACH, BCH>(arow, brow, min(1, KT - 1) * BK);
        gemm_sstore<ACH, BCH>(sA[0], sB[0], aoff, boff, s0);
        __syncthreads();
        for (int kt = 0; kt < KT; kt += 2) {
            s0 = gemm_gload<ACH, BCH>(arow, brow, min(kt + 2, KT - 1) * BK);
            gemm_mma<TM, TN>(sa0, sb0, fr, fk, acc);
            gemm_sstore<ACH, BCH>(sA[1], sB[1], aoff, boff, s1);
            __syncthreads();
            if (kt + 1 < KT) {
                s1 = gemm_gload<ACH, BCH>(arow, brow, min(kt + 3, KT - 1) * BK);
                gemm_mma<TM, TN>(sa1, sb1, fr, fk, acc);
                gemm_sstore<ACH, BCH>(sA[0], sB[0], aoff, boff, s0);
                __syncthreads();
            }
        }
    }

    // Epilogue.  Accumulator element r of tile (i, j) is row 4*(lane/16) + r, column lane%16.
    const int rbase = m0 + wm * WM + (lane >> 4) * 4;
    const int cbase = n0 + wn * WN + (lane & 15);
    if (EPI == EPI_SWIGLU) {
        bf16_t *C = reinterpret_cast<bf16_t *>(g.C);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; j += 2) {
                const int ncol = n0 + wn * WN + j * 16;  // first logical column of the gate tile
                const int ocol = (ncol >> 5) * 16 + (lane & 15);
                if (ncol >= g.N) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = rbase + i * 16 + r;
                    if (row < g.M)
                        C[(int64_t)row * g.ldc + ocol] = f32_to_bf16(silu_f(acc[i][j][r]) * acc[i][j + 1][r]);
                }
            }
    } else {
        float *C = reinterpret_cast<float *>(g.C);
        int64_t ldc = g.ldc;
        if (EPI == EPI_PARTIAL) {
            C += (int64_t)blockIdx.z * g.M * g.N;
            ldc = g.N;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = cbase + j * 16;
                if (col >= g.N) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = rbase + i * 16 + r;
                    if (row >= g.M) continue;
                    float *p = C + (int64_t)row * ldc + col;
                    if (EPI == EPI_ADD) *p += acc[i][j][r];
                    else *p = acc[i][j][r];
                }
            }
    }
}

// Sum of the K-split partials in split order, then the real epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce(GemmArgs g, const float *part, int splits) {
    const int64_t total = (EPI == EPI_SWIGLU) ? (int64_t)g.M * (g.N / 2) : (int64_t)g.M * g.N;
    const int64_t stride = (int64_t)g.M * g.N;
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        if (EPI == EPI_SWIGLU) {
            const int half = g.N / 2;
            const int m = (int)(i / half), j = (int)(i % half);
            const int ng = (j >> 4) * 32 + (j & 15);  // logical gate column; up is ng + 16
            float gs = 0.f, us = 0.f;
            for (int z = 0; z < splits; ++z) {
                gs += part[z * stride + (int64_t)m * g.N + ng];
                us += part[z * stride + (int64_t)m * g.N + ng + 16];
            }
            reinterpret_cast<bf16_t *>(g.C)[(int64_t)m * g.ldc + j] = f32_to_bf16(silu_f(gs) * us);
        } else {
            const int m = (int)(i / g.N), n = (int)(i % g.N);
            float v = 0.f;
            for (int z = 0; z < splits; ++z) v += part[z * stride + i];
            float *c = reinterpret_cast<float *>(g.C) + (int64_t)m * g.ldc + n;
            if (EPI == EPI_ADD) *c += v;
            else *c = v;
        }
    }
}


// ------------------------------------------------------------------------------------
// Operand layout of the 32x32x16 MFMA kernels.  v_mfma_f32_32x32x16_bf16 runs at about
// twice the rate per flop of the 16x16x32 form on gfx950.  A lane of one 32x32x16
// product supplies A[row = l%32][k = 8*(l/32)..+7] and B[k = 8*(l/32)..+7][col = l%32]
// and receives rows 8*j + 4*(l/32) + i (j, i < 4) of column l%32 as acc[4*j + i].  The
// SwiGLU weights interleave in groups of 32 rows (gate, up) so a lane's pair of
// accumulator tiles holds matching gate and up columns.
// ------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

template <typename T>
__device__ __forceinline__ const T *wrow32(const WSrc &w, int epi, int n, int K) {
    if (epi == EPI_SWIGLU) {
        const int pair = n >> 6, half = (n >> 5) & 1, r = n & 31;
        // integer select between the two (uniform) bases: a select of the two pointer
        // arguments would be turned into a per-lane load of the argument array
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(w.p[0]), a1 = reinterpret_cast<uintptr_t>(w.p[1]);
        const T *base = reinterpret_cast<const T *>(a0 + (half ? a1 - a0 : (uintptr_t)0));
        return base + (int64_t)(pair * 32 + r) * K;
    }
    return wrow<T>(w, EPI_STORE, n, K);
}

// ------------------------------------------------------------------------------------
// Multi-stage LDS-DMA GEMM (bf16, 32x32x16 MFMA) for M > 64.  With one 128x128 tile
// per CU (the MaskGIT pass at S = 950 has 256 such tiles in its widest projection) the
// global-load latency has to be covered by prefetch depth inside the block, not by
// other blocks.  Operand tiles of 64 K-elements go straight from global memory into
// LDS (global_load_lds_dwordx4: no staging registers, no LDS store instructions) into a
// ring of STAGES buffers, STAGES-1 tiles ahead of the products.  A wave's DMA
// instruction fills 1 KB of LDS in lane order (8 rows x 8 16-byte chunks); the lane ->
// global chunk assignment applies the XOR swizzle chunk ^ (row % 8), so the 16-byte
// fragment reads of 8 consecutive rows hit distinct banks.  Each wave waits only for
// its own DMA of the tile it is about to read (vmcnt), then the block barrier makes
// every wave's part visible; a buffer is refilled only after the barrier that follows
// its last use.  Prefetches past the last tile are not issued; the waits count that.
// ------------------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // vmcnt[3:0] | expcnt (7: no wait) | lgkmcnt (15: no wait) | vmcnt[5:4]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void dma16(const bf16_t *src, bf16_t *lds_wave_dst) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src),
                                     (__attribute__((address_space(3))) void *)(lds_wave_dst), 16, 0,
                                     0);
}

// DMA of K tile kt of both operands into one ring buffer (st).
template <int BM, int AI, int BI>
__device__ __forceinline__ void lds_issue(const bf16_t *const (&asrc)[AI], const bf16_t *const (&bsrc)[BI],
                                          bf16_t *st, int wave, int kt) {
#pragma unroll
    for (int c = 0; c < AI; ++c) dma16(asrc[c] + kt * 64, st + (wave * AI + c) * 512);
#pragma unroll
    for (int c = 0; c < BI; ++c) dma16(bsrc[c] + kt * 64, st + BM * 64 + (wave * BI + c) * 512);
}

// 32x32x16 operand fragments of one K step from the swizzled tiles: row (i*32 + lane%32)
// of the wave's A (B) rows, physical chunk ph (the caller's swizzled K chunk).
template <int TM, int TN>
__device__ __forceinline__ void lds_frags(const bf16_t *sa, const bf16_t *sb, int ph, bf16x8_t (&af)[TM],
                                          bf16x8_t (&bfr)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8_t *>(sa + i * 32 * 64 + ph);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t *>(sb + j * 32 * 64 + ph);
}

// Fused epilogue of the full-sequence q/k/v projection (one 128 x 128 tile = 128
// tokens x one head of the qkv output; block of 4 waves in 2 x 2, wave tile 64 x 64).
// The fp32 tile goes through LDS in two halves of 64 tokens (row stride 132 floats);
// for a q or k head each token's 128 values get the per-head RMSNorm (eight threads per
// token, 8 RoPE pairs each, sum of squares over the eight) and the half-rotate RoPE at
// position = token index (minus seg1 in a second sequence), then go out as bf16 q
// [S][H*128] or K [Hkv][s_pad][128];
// a v head goes out transposed, V^T [Hkv][128][s_pad], 8 tokens per 16-byte store.
template <int TM, int TN>
__device__ __forceinline__ void qkv_dense_epilogue(const f32x16_t (&acc)[TM][TN], float *tile, int m0, int n0,
                                                   int M, const RopeKvArgs &rk) {
    constexpr int LDT = 132;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int head = n0 / 128;
    const bool is_v = head >= rk.H + rk.Hkv;
    const bool is_q = head < rk.H;
    // q / k heads: the gains and every RoPE entry of this thread's tokens and dims are
    // requested before the tile goes through LDS (their latency overlaps it).  Eight
    // threads per token, each with dims q8*8 .. +7 and their RoPE partners 64 + q8*8 ..,
    // so that eight consecutive lanes store one whole 128-byte line of each half.
    const int q8 = tid & 7;
    float2 csr[2][2][8];
    float glo[8], ghi[8];
    if (!is_v) {
        const float *gain = is_q ? rk.q_gain : rk.k_gain;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            glo[e] = gain[q8 * 8 + e];
            ghi[e] = gain[q8 * 8 + 64 + e];
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                const int m = m0 + hf * 64 + ps * 32 + (tid >> 3);
                const int pos = rk.seg1 > 0 && m >= rk.seg1 ? m - rk.seg1 : m;  // second sequence
                const float2 *cs = rk.rope + (int64_t)min(pos, rk.max_pos - 1) * 64 + q8 * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) csr[hf][ps][e] = cs[e];
            }
    }
    // LDS-only barriers: __syncthreads() would also wait for the table loads above
    auto lds_barrier = []() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
        __builtin_amdgcn_s_barrier();
    };
    for (int half = 0; half < 2; ++half) {
        lds_barrier();  // the previous use of the LDS (ring buffers / first half) is over
        if (wm == half) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                        tile[row * LDT + wn * 64 + j * 32 + (lane & 31)] = acc[i][j][r];
                    }
        }
        lds_barrier();
        const int t0 = m0 + half * 64;
        if (!is_v) {
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                const int row = ps * 32 + (tid >> 3), m = t0 + row;
                const float *x = tile + row * LDT + q8 * 8;
                float lo[8], hi[8];
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    lo[e] = x[e];
                    hi[e] = x[64 + e];
                    ss += lo[e] * lo[e] + hi[e] * hi[e];
                }
                ss = group_sum<8>(ss);
                const float inv = 1.0f / sqrtf(ss / 128.0f + rk.eps);
                uint32_t wlo[4], whi[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float o[2][2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const float x0 = lo[e + u] * inv * glo[e + u], x1 = hi[e + u] * inv * ghi[e + u];
                        const float2 c = csr[half][ps][e + u];
                        o[0][u] = x0 * c.x - x1 * c.y;
                        o[1][u] = x1 * c.x + x0 * c.y;
                    }
                    wlo[e / 2] = (uint32_t)f32_to_bf16(o[0][0]) | ((uint32_t)f32_to_bf16(o[0][1]) << 16);
                    whi[e / 2] = (uint32_t)f32_to_bf16(o[1][0]) | ((uint32_t)f32_to_bf16(o[1][1]) << 16);
                }
                if (m < M) {
                    bf16_t *dst = is_q ? reinterpret_cast<bf16_t *>(rk.q_out) + ((int64_t)m * rk.H + head) * 128
                                       : rk.kbuf + ((int64_t)(head - rk.H) * rk.s_pad + m) * 128;
                    *reinterpret_cast<u32x4_t *>(dst + q8 * 8) = u32x4_t{wlo[0], wlo[1], wlo[2], wlo[3]};
                    *reinterpret_cast<u32x4_t *>(dst + 64 + q8 * 8) = u32x4_t{whi[0], whi[1], whi[2], whi[3]};
                }
            }
        } else {
            bf16_t *vt = rk.vtbuf + (int64_t)(head - rk.H - rk.Hkv) * 128 * rk.s_pad;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int item = tid + 256 * u, d = item & 127, sg = item >> 7;  // 8 groups of 8 tokens
                const int m = t0 + sg * 8;
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2)
                    w[e / 2] = (uint32_t)f32_to_bf16(tile[(sg * 8 + e) * LDT + d]) |
                               ((uint32_t)f32_to_bf16(tile[(sg * 8 + e + 1) * LDT + d]) << 16);
                bf16_t *dst = vt + (int64_t)d * rk.s_pad + m;
                if (m + 8 <= M) {
                    *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (m + e < M) dst[e] = (bf16_t)(w[e / 2] >> (16 * (e & 1)));
                }
            }
        }
    }
}

// Scoring epilogue of the head product (one 128 x 128 tile; block of 4 waves in 2 x 2).
// The fp32 tile goes through LDS in two halves of 64 rows; there, column c of a row sits
// at (c / 32) * 36 + c % 32 of a 144-float row, so that the row's four threads, each
// reading its 32 consecutive columns as eight 16-byte loads, and the next rows' threads
// fall in distinct banks.  Each thread reduces, per group of g.gv columns met by the
// tile (at most two: the tile's first group k0, and k0 + 1 from column `cut` on), the
// maximum over all classes, the best non-mask class (ties: lowest id) and the sum of
// exp(y - max); the four threads' statistics merge by lane exchanges, and the row's first
// thread stores them.
template <int TM, int TN>
__device__ __forceinline__ void scores_epilogue(const f32x16_t (&acc)[TM][TN], float *tile, int m0, int n0,
                                                int tiles_n, const GemmArgs &g) {
    constexpr int LDT = 144, SEG = 36;
    const float LOG2E = 1.4426950408889634f;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int V = g.gv, k0 = n0 / V;
    const int cut = min(128, (k0 + 1) * V - n0);  // tile columns [0, cut) are group k0, the rest k0 + 1
    const int tn = n0 / 128;
    const int row = tid >> 2, q = tid & 3;
    const int cbase = q * 32;                           // this thread's columns [cbase, cbase + 32)
    const int nvalid = min(32, g.N - n0 - cbase);       // of which those below N (may be <= 0)
    const int cls0 = n0 + cbase - k0 * V;               // class of column cbase in group k0
    auto lds_barrier = []() {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    };
    for (int half = 0; half < 2; ++half) {
        lds_barrier();  // the ring's (or the first half's) last reads are done
        if (wm == half) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rr = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                        tile[rr * LDT + (wn * 2 + j) * SEG + (lane & 31)] = acc[i][j][r];
                    }
        }
        lds_barrier();
        float v[32];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float4 t = *reinterpret_cast<const float4 *>(tile + row * LDT + q * SEG + c * 4);
            v[c * 4] = t.x;
            v[c * 4 + 1] = t.y;
            v[c * 4 + 2] = t.z;
            v[c * 4 + 3] = t.w;
        }
        // Per thread: (max, sum of exp relative to it, best non-mask value, its class) of
        // group k0 over its columns [0, lim0) and of group k0 + 1 over [split, nvalid).
        // Argmax ties go to the first (lowest) class, as argmax_merge orders them.
        float mx[2] = {-INFINITY, -INFINITY}, best[2] = {-INFINITY, -INFINITY}, se[2] = {0.f, 0.f};
        int bi[2] = {0x7FFFFFFF, 0x7FFFFFFF};
        int z;  // an opaque zero: keeps the per-column masks below from being hoisted out of the loop
        asm volatile("s_mov_b32 %0, 0" : "=s"(z));
        const int split = min(32, max(0, cut - cbase)) + z;  // columns [0, split) are group k0
        const int lim0 = min(split, nvalid);
        const int g0 = g.gmask - cls0 + z, g1 = g0 + V;       // the mask's column in group k0, k0 + 1
        const int sg = split == 32 ? 0 : 1;                    // a one-group thread's group
        const bool simple = nvalid == 32 && (split == 0 || split == 32) && (unsigned)(sg ? g1 : g0) >= 32u;
        if (__builtin_amdgcn_read_exec() == __ballot(simple)) {
            // whole wave: all 32 columns valid, in one group, none the mask
            float m = v[0];
#pragma unroll
            for (int i = 1; i < 32; ++i) m = fmaxf(m, v[i]);
            const float mb = m * LOG2E;
            float e = 0.f;
            int idx = 0x7FFFFFFF;
#pragma unroll
            for (int i = 31; i >= 0; --i) {
                e += __builtin_amdgcn_exp2f(v[i] * LOG2E - mb);
                idx = v[i] == m ? i : idx;
            }
            const int cls = idx == 0x7FFFFFFF ? idx : cls0 - sg * V + idx;
            mx[sg] = m;
            se[sg] = e;
            best[sg] = m;
            bi[sg] = cls;
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const bool a0 = i < lim0, a1 = (i >= split) & (i < nvalid);
                const float x0 = a0 ? v[i] : -INFINITY, x1 = a1 ? v[i] : -INFINITY;
                mx[0] = fmaxf(mx[0], x0);
                mx[1] = fmaxf(mx[1], x1);
                const bool u0 = a0 & (i != g0) & ((x0 > best[0]) | ((x0 == best[0]) & (bi[0] == 0x7FFFFFFF)));
                const bool u1 = a1 & (i != g1) & ((x1 > best[1]) | ((x1 == best[1]) & (bi[1] == 0x7FFFFFFF)));
                best[0] = u0 ? x0 : best[0];
                bi[0] = u0 ? cls0 + i : bi[0];
                best[1] = u1 ? x1 : best[1];
                bi[1] = u1 ? cls0 + i - V : bi[1];
            }
            const float mb0 = mx[0] * LOG2E, mb1 = mx[1] * LOG2E;
            int z2;  // the masks again from fresh bounds, not kept alive from the first loop
            asm volatile("s_mov_b32 %0, 0" : "=s"(z2));
            const int split2 = split + z2, lim2 = lim0 + z2, nv2 = nvalid + z2;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const bool a0 = i < lim2, a1 = (i >= split2) & (i < nv2);
                se[0] += a0 ? __builtin_amdgcn_exp2f(v[i] * LOG2E - mb0) : 0.f;
                se[1] += a1 ? __builtin_amdgcn_exp2f(v[i] * LOG2E - mb1) : 0.f;
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int o = 1; o <= 2; o <<= 1) {
                const float m2 = __shfl_xor(mx[s], o, WAVE), s2 = __shfl_xor(se[s], o, WAVE);
                const float b2 = __shfl_xor(best[s], o, WAVE);
                const int i2 = __shfl_xor(bi[s], o, WAVE);
                const float M = fmaxf(mx[s], m2);
                const float f1 = mx[s] == -INFINITY ? 0.f : exp2f((mx[s] - M) * LOG2E);
                const float f2 = m2 == -INFINITY ? 0.f : exp2f((m2 - M) * LOG2E);
                se[s] = se[s] * f1 + s2 * f2;
                mx[s] = M;
                argmax_merge(best[s], bi[s], b2, i2);
            }
        const int m = m0 + half * 64 + row;
        if (q == 0 && m < g.M) {
            float4 *dst = g.spart + ((int64_t)m * tiles_n + tn) * 2;
            dst[0] = make_float4(mx[0], se[0], best[0], __int_as_float(bi[0]));
            if (cut < 128) dst[1] = make_float4(mx[1], se[1], best[1], __int_as_float(bi[1]));
        }
    }
}

template <int BM, int BN, int STAGES, int EPI>
__global__ __launch_bounds__(256) void gemm_lds(GemmArgs g, int k_split, RopeKvArgs rk) {
    constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
    constexpr int AI = BM / 32, BI = BN / 32;  // DMA instructions per wave per stage
    constexpr int LPS = AI + BI;               // vector-memory ops per wave per stage
    constexpr int TILE = (BM + BN) * 64;       // elements per stage
    static_assert(TM >= 1 && TN >= 1 && AI >= 1 && BI >= 1, "tile too small");
    static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "swiglu needs gate/up tile pairs");
    static_assert(STAGES >= 2 && STAGES <= 4, "stages");
    __shared__ __attribute__((aligned(1024))) bf16_t smem[STAGES * TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    const int t = xcd_tile(blockIdx.x, tiles_m * tiles_n);
    const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;
    const int k_begin = blockIdx.z * k_split;
    const int KT = min(k_split, g.K - k_begin) / 64;

    // Lane sources: instruction c of this wave covers tile rows (wave*I + c)*8 .. +7;
    // lane i lands in LDS chunk i of that 1 KB, i.e. row r = +i/8, physical chunk i%8, and
    // fetches logical chunk (i%8) ^ ((r / 2) % 8) of its row.  A row is 128 bytes, half of
    // the 64 four-byte banks, and a 16-byte fragment read serves 16 lanes (rows fr..fr+15)
    // per cycle: with the swizzle taken from row bits 1..3 (rows of one parity share a half
    // of the banks), those 16 rows' chunks fall in 16 distinct bank quads.  (I is even, so
    // (r / 2) % 8 = 4 (c % 2) + (i / 8) / 2.)
    const int lrow = lane >> 3;
    const bf16_t *A = reinterpret_cast<const bf16_t *>(g.A);
    const bf16_t *asrc[AI];
    const bf16_t *bsrc[BI];
    static_assert(AI % 2 == 0 && BI % 2 == 0, "swizzle assumes an even number of 8-row blocks per wave");
#pragma unroll
    for (int c = 0; c < AI; ++c) {
        const int r = (wave * AI + c) * 8 + lrow;
        const int lchunk = (lane & 7) ^ (((c & 1) << 2) | (lrow >> 1));
        asrc[c] = A + (int64_t)min(m0 + r, g.M - 1) * g.lda + k_begin + lchunk * 8;  // rows past M: unstored
    }
#pragma unroll
    for (int c = 0; c < BI; ++c) {
        const int r = (wave * BI + c) * 8 + lrow;
        const int lchunk = (lane & 7) ^ (((c & 1) << 2) | (lrow >> 1));
        // split partials come only from residual-add products: plain row order
        bsrc[c] = wrow32<bf16_t>(g.w, EPI == EPI_SWIGLU ? EPI_SWIGLU : EPI_STORE, min(n0 + r, g.N - 1), g.K) +
                  k_begin + lchunk * 8;
    }

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < KT) lds_issue<BM, AI, BI>(asrc, bsrc, smem + s * TILE, wave, s);

    const int fr = lane & 31, fh = lane >> 5, sw = (lane >> 1) & 7;  // (fr / 2) % 8: the row's swizzle
    for (int kt = 0; kt < KT; ++kt) {
        // this wave's DMA of tile kt is done once at most (tiles issued after it) x LPS
        // operations are outstanding
        const int after = min(STAGES - 2, KT - 1 - kt);
        if (after >= 2) wait_vmcnt<2 * LPS>();
        else if (after == 1) wait_vmcnt<LPS>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        if (kt + STAGES - 1 < KT)  // refills the buffer of tile kt-1
            lds_issue<BM, AI, BI>(asrc, bsrc, smem + ((kt + STAGES - 1) % STAGES) * TILE, wave, kt + STAGES - 1);

        const bf16_t *sa = smem + (kt % STAGES) * TILE + (wm * WM) * 64 + fr * 64;
        const bf16_t *sb = smem + (kt % STAGES) * TILE + BM * 64 + (wn * WN) * 64 + fr * 64;
        // All four 16-deep steps' fragments in registers of their own, read in two halves:
        // the second half's reads go out between the first half's products, so the LDS
        // latency is waited for once per 64-deep step instead of once per 16.
        bf16x8_t af[4][TM], bfr[4][TN];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) lds_frags<TM, TN>(sa, sb, ((ks * 2 + fh) ^ sw) * 8, af[ks], bfr[ks]);
#pragma unroll
        for (int ks = 2; ks < 4; ++ks) lds_frags<TM, TN>(sa, sb, ((ks * 2 + fh) ^ sw) * 8, af[ks], bfr[ks]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
        constexpr int NR = 2 * (TM + TN), NP = 2 * TM * TN, NI = NR < NP ? NR : NP;
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // reads of steps 0, 1
#pragma unroll
        for (int q = 0; q < NI; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a product of steps 0, 1
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // a read of steps 2, 3
        }
        if (NR > NI) __builtin_amdgcn_sched_group_barrier(0x100, NR - NI, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * TM * TN - NI, 0);  // the rest
    }

    if constexpr (EPI == EPI_QKV) {
        static_assert(BM == 128 && BN == 128, "one tile = 128 tokens x one head");
        qkv_dense_epilogue<TM, TN>(acc, reinterpret_cast<float *>(smem), m0, n0, g.M, rk);
        return;
    }
    if constexpr (EPI == EPI_SCORES) {
        static_assert(BM == 128 && BN == 128 && STAGES * TILE * 2 >= 64 * 144 * 4, "64-row halves staged");
        scores_epilogue<TM, TN>(acc, reinterpret_cast<float *>(smem), m0, n0, tiles_n, g);
        return;
    }
    const int rb0 = m0 + wm * WM + (lane >> 5) * 4, cb0 = n0 + wn * WN + (lane & 31);
    if constexpr (EPI == EPI_SWIGLU) {
        // the BM x BN/2 bf16 tile of m goes through the (now idle) ring buffer, row stride
        // BN/2 + 8 elements, so that eight consecutive lanes store one whole 128-byte line
        constexpr int OW = BN / 2, LDO = OW + 8;
        static_assert(BM * LDO <= STAGES * TILE && (BM * OW / 8) % 256 == 0, "m tile staging");
        __syncthreads();  // every wave's last fragment reads are done
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; j += 2) {
                const int ocol = (wn * WN + j * 32) / 2 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    smem[row * LDO + ocol] = f32_to_bf16(silu_f(acc[i][j][r]) * acc[i][j + 1][r]);
                }
            }
        __syncthreads();
        bf16_t *C = reinterpret_cast<bf16_t *>(g.C);
#pragma unroll
        for (int it = 0; it < BM * OW / 8 / 256; ++it) {
            const int idx = it * 256 + tid, row = idx / (OW / 8), c8 = (idx % (OW / 8)) * 8;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + row * LDO + c8);
            if (m0 + row < g.M && n0 / 2 + c8 < g.N / 2)
                *reinterpret_cast<u32x4_t *>(C + (int64_t)(m0 + row) * g.ldc + n0 / 2 + c8) = v;
        }
    } else {
        float *C = reinterpret_cast<float *>(g.C);
        int64_t ldc = g.ldc;
        if (EPI == EPI_PARTIAL) {
            C += (int64_t)blockIdx.z * g.M * g.N;
            ldc = g.N;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = cb0 + j * 32;
                if (col >= g.N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = rb0 + i * 32 + (r >> 2) * 8 + (r & 3);
                    if (row >= g.M) continue;
                    float *p = C + (int64_t)row * ldc + col;
                    if (EPI == EPI_ADD) *p += acc[i][j][r];
                    else *p = acc[i][j][r];
                }
            }
    }
}

// Launch of the LDS-DMA GEMM; splits > 1 writes partials [splits][M][N] into part and
// returns splits (EPI_ADD only: the caller adds them), else returns 0.
template <int BM, int BN, int STAGES>
static int launch_gemm_lds(const GemmArgs &g, int splits, float *part, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    const int kt = g.K / 64;
    const int k_split = ((kt + splits - 1) / splits) * 64;
    splits = (g.K + k_split - 1) / k_split;
    const dim3 grid(tiles, 1, splits);
    if (splits > 1) {
        GemmArgs gp = g;
        gp.C = part;
        gp.ldc = g.N;
        hipLaunchKernelGGL((gemm_lds<BM, BN, STAGES, EPI_PARTIAL>), grid, dim3(256), 0, s, gp, k_split, RopeKvArgs{});
        return splits;
    }
    switch (g.epi) {
        case EPI_STORE:
            hipLaunchKernelGGL((gemm_lds<BM, BN, STAGES, EPI_STORE>), grid, dim3(256), 0, s, g, k_split, RopeKvArgs{});
            break;
        case EPI_ADD:
            hipLaunchKernelGGL((gemm_lds<BM, BN, STAGES, EPI_ADD>), grid, dim3(256), 0, s, g, k_split, RopeKvArgs{});
            break;
        default:
            if constexpr ((BN / 2 / 32) % 2 == 0)
                hipLaunchKernelGGL((gemm_lds<BM, BN, STAGES, EPI_SWIGLU>), grid, dim3(256), 0, s, g, k_split,
                                   RopeKvArgs{});
            break;
    }
    return 0;
}

// ------------------------------------------------------------------------------------
// Skinny MFMA GEMM for 8 < M <= 64 (the batched decode step): a weight-streaming kernel.
// At M = 64 a projection reads each weight once and does 64 flops per weight element,
// so it is bound by HBM bandwidth and by the latency of getting the weights in flight.
// A block owns a slice of 16 output columns (16 gate + 16 up for SwiGLU) over one K
// range, split into four per-wave K ranges of STEPS x 32.  Every lane issues all of its
// loads up front: its weight row segments (16 bytes per step, straight into the MFMA B
// operand: lane l holds W[col l%16][k 8*(l/16)..+7]) and the activation fragments of
// the MT 16-row tiles (A operand: row l%16 of the tile, same k), then runs the
// STEPS x MT x NT products.  The four waves' accumulators are summed in LDS in wave
// order.  Only a residual-add product is split over K (grid = slices x splits, to give
// the N = hidden projections enough blocks): each block writes its fp32 partial sums
// and the residual update is left to the RMSNorm that reads the residual next, which
// adds the partials in split order (deterministic, and no extra launch or cross-block
// synchronisation).
// ------------------------------------------------------------------------------------
constexpr int SK_MAX_SPLIT = 8;

template <int MT, int STEPS, int EPI>
__global__ __launch_bounds__(256) void gemm_skinny(GemmArgs g, float *part, int n_split) {
    constexpr int NT = (EPI == EPI_SWIGLU) ? 2 : 1;
    __shared__ float red[4][NT][MT][4][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = blockIdx.x / n_split, ks = blockIdx.x % n_split;
    const int fr = lane & 15;
    const int k0 = (ks * 4 + wave) * STEPS * 32 + (lane >> 4) * 8;
    const bf16_t *A = reinterpret_cast<const bf16_t *>(g.A);

    u32x4_t wv[NT][STEPS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        // columns past N read column N-1: their results are never stored
        const bf16_t *wp;
        if (EPI == EPI_SWIGLU)  // tile 0: gate rows, tile 1: up rows of the same 16 outputs
            wp = reinterpret_cast<const bf16_t *>(g.w.p[nt]) + (int64_t)min(slice * 16 + fr, g.N / 2 - 1) * g.K;
        else
            wp = wrow<bf16_t>(g.w, EPI_STORE, min(slice * 16 + fr, g.N - 1), g.K);
        wp += k0;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) wv[nt][s] = *reinterpret_cast<const u32x4_t *>(wp + s * 32);
    }
    u32x4_t av[MT][STEPS];
    if (g.a_mt > 0) {
        // fragment-major A (a_mt == MT): fragment (k step kc, tile mt) is one contiguous 1 KB;
        // rows past M hold anything (their results are never stored)
        const int kc0 = (ks * 4 + wave) * STEPS;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
                av[mt][s] = *reinterpret_cast<const u32x4_t *>(A + ((int64_t)(kc0 + s) * MT + mt) * 512 + lane * 8);
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const bf16_t *ap = A + (int64_t)min(mt * 16 + fr, g.M - 1) * g.lda + k0;  // rows past M: unstored
#pragma unroll
            for (int s = 0; s < STEPS; ++s) av[mt][s] = *reinterpret_cast<const u32x4_t *>(ap + s * 32);
        }
    }
    // keep every load ahead of the products: all of them in flight at once
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t acc[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, av[mt][s]), __builtin_bit_cast(bf16x8_t, wv[nt][s]), acc[nt][mt],
                    0, 0, 0);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][nt][mt][r][lane] = acc[nt][mt][r];
    __syncthreads();

    // Thread (r = wave, l = lane) finishes element r of lane l's accumulators in every
    // M tile: row mt*16 + 4*(l/16) + r, column l%16 of the slice.
    const int r = wave, l = lane;
    float v[NT][MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            v[nt][mt] = ((red[0][nt][mt][r][l] + red[1][nt][mt][r][l]) + red[2][nt][mt][r][l]) + red[3][nt][mt][r][l];
    const int col = slice * 16 * NT + (l & 15);  // logical column of the first N tile

    if (EPI == EPI_ADD && n_split > 1) {  // partial sums; the residual update is deferred
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = mt * 16 + 4 * (l >> 4) + r;
            if (row < g.M && col < g.N) part[((int64_t)ks * g.M + row) * g.N + col] = v[0][mt];
        }
        return;
    }

    float prev[MT];  // residual values, all loaded before any store
    if (EPI == EPI_ADD) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            prev[mt] = reinterpret_cast<const float *>(g.C)[(int64_t)min(mt * 16 + 4 * (l >> 4) + r, g.M - 1) * g.ldc +
                                                           min(col, g.N - 1)];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = mt * 16 + 4 * (l >> 4) + r;
        if (row >= g.M) continue;
        if (EPI == EPI_SWIGLU) {
            const int oc = slice * 16 + (l & 15);  // output column (the next product's K index)
            if (col < g.N)
                reinterpret_cast<bf16_t *>(g.C)[g.c_mt > 0 ? frag_index(row, oc, g.c_mt) : (int64_t)row * g.ldc + oc] =
                    f32_to_bf16(silu_f(v[0][mt]) * v[NT - 1][mt]);
        } else if (col < g.N) {
            float *p = reinterpret_cast<float *>(g.C) + (int64_t)row * g.ldc + col;
            *p = EPI == EPI_ADD ? prev[mt] + v[0][mt] : v[0][mt];
        }
    }
}

template <int MT, int STEPS>
static void launch_skinny_mt(const GemmArgs &g, int slices, int n_split, float *part, hipStream_t s) {
    const dim3 grid(slices * n_split);
    switch (g.epi) {
        case EPI_STORE:
            hipLaunchKernelGGL((gemm_skinny<MT, STEPS, EPI_STORE>), grid, dim3(256), 0, s, g, part, n_split);
            break;
        case EPI_ADD:
            hipLaunchKernelGGL((gemm_skinny<MT, STEPS, EPI_ADD>), grid, dim3(256), 0, s, g, part, n_split);
            break;
        default:
            hipLaunchKernelGGL((gemm_skinny<MT, STEPS, EPI_SWIGLU>), grid, dim3(256), 0, s, g, part, n_split);
            break;
    }
}

// Slices of 16 (SwiGLU: 32) logical columns; each wave runs STEPS = 8 or 4 K steps of
// 32.  A residual-add product takes the fewest K splits (at most SK_MAX_SPLIT) that
// give >= 256 blocks; the others are not split.  Returns -1 when the shape does not
// fit (the tile kernels then run it), else the number of splits.
static int skinny_plan(const GemmArgs &g, int64_t part_cap, int &slices, int &steps) {
    const int width = g.epi == EPI_SWIGLU ? 32 : 16;
    if (g.M > 64 || g.K % 512 != 0 || (g.epi == EPI_SWIGLU && g.N % 32 != 0)) return -1;
    slices = (g.N + width - 1) / width;
    int n_split = 0;
    const int zmax = g.epi == EPI_ADD ? SK_MAX_SPLIT : 1;
    for (int z = 1; z <= zmax; ++z) {
        if (g.K % (z * 128) != 0) continue;
        const int st = g.K / (z * 128);
        if (st != 8 && st != 4) continue;
        n_split = z;
        steps = st;
        if (slices * z >= 256) break;
    }
    if (n_split == 0) return -1;
    if (n_split > 1 && (int64_t)n_split * g.M * g.N > part_cap) return -1;
    return n_split;
}

int skinny_tiles(const GemmArgs &g, int64_t part_cap) {
    if (g.M <= 8 || g.M > 64) return 0;  // M <= 8: the GEMV
    int slices, steps;
    if (skinny_plan(g, part_cap, slices, steps) < 0) return 0;
    const int mt = (g.M + 15) / 16;
    return mt <= 2 ? mt : 4;
}

static int launch_skinny(const GemmArgs &g, float *part, int64_t part_cap, hipStream_t s) {
    int slices, steps;
    const int n_split = skinny_plan(g, part_cap, slices, steps);
    if (n_split < 0) return -1;
    const int mt = (g.M + 15) / 16;
    if (steps == 8) {
        if (mt == 1) launch_skinny_mt<1, 8>(g, slices, n_split, part, s);
        else if (mt == 2) launch_skinny_mt<2, 8>(g, slices, n_split, part, s);
        else launch_skinny_mt<4, 8>(g, slices, n_split, part, s);
    } else {
        if (mt == 1) launch_skinny_mt<1, 4>(g, slices, n_split, part, s);
        else if (mt == 2) launch_skinny_mt<2, 4>(g, slices, n_split, part, s);
        else launch_skinny_mt<4, 4>(g, slices, n_split, part, s);
    }
    return n_split > 1 ? n_split : 0;
}

// ------------------------------------------------------------------------------------
// Weight-streaming GEMV for M <= 8 (bf16 or fp32)
// ------------------------------------------------------------------------------------
constexpr int GEMV_MAXM = 8;
constexpr int GEMV_UNITS = 2;  // output columns per wave

// 16-byte loads widened to fp32; load_nt is the non-temporal form for the GEMV's weights,
// which a step reads once (batch-1 loop: 0.845 -> 0.807 ms per step; the skinny kernel's
// weight loads stay plain -- non-temporal there made the 64-stream step slower)
template <typename T> struct Vec;
template <> struct Vec<bf16_t> {
    static constexpr int N = 8;
    __device__ static void load(const bf16_t *p, float v[8]) {
        uint4 t = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ static void load_nt(const bf16_t *p, float v[8]) {
        const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(t[i] << 16);
            v[2 * i + 1] = __uint_as_float(t[i] & 0xFFFF0000u);
        }
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void load(const float *p, float v[4]) {
        float4 t = *reinterpret_cast<const float4 *>(p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
    __device__ static void load_nt(const float *p, float v[4]) {
        const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
        v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
    }
};

// KI > 0: K is exactly KI chunks of 64 lanes x V elements and every weight load of the
// wave is issued up front; KI == 0: any K, one chunk per loop trip.  NORM: the A operand
// is RMSNorm(x) * gain computed in the prologue from the fp32 residual rows g.nx (the
// row's sum of squares is reduced with the thread -> column mapping and the order of the
// RMSNorm kernel, and the operand is rounded to T as that kernel stores it, so the
// product is bit-identical to RMSNorm followed by the plain GEMV).
template <typename T, int EPI, int KI, bool NORM>
__global__ __launch_bounds__(256) void gemv(GemmArgs g) {
    constexpr int V = Vec<T>::N, CH = 64 * V;
    constexpr int KB = KI > 0 ? KI : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int unit0 = (blockIdx.x * 4 + wave) * GEMV_UNITS;
    const int n_units = (EPI == EPI_SWIGLU) ? g.N / 2 : g.N;
    const T *A = reinterpret_cast<const T *>(g.A);

    const T *wr[2 * GEMV_UNITS];
#pragma unroll
    for (int u = 0; u < GEMV_UNITS; ++u) {
        const int n = unit0 + u < n_units ? unit0 + u : n_units - 1;
        if (EPI == EPI_SWIGLU) {
            wr[2 * u] = reinterpret_cast<const T *>(g.w.p[0]) + (int64_t)n * g.K;
            wr[2 * u + 1] = reinterpret_cast<const T *>(g.w.p[1]) + (int64_t)n * g.K;
        } else {
            wr[u] = wrow<T>(g.w, EPI_STORE, n, g.K);
        }
    }
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 * GEMV_UNITS : GEMV_UNITS;

    float wv[KB][NW][V];
    if (KI > 0) {  // every weight load first: they are the long-latency ones
#pragma unroll
        for (int c = 0; c < KB; ++c)
#pragma unroll
            for (int u = 0; u < NW; ++u) Vec<T>::load_nt(wr[u] + c * CH + lane * V, wv[c][u]);
    }

    // NORM: the normalized operand rows are built once per block in LDS (bf16 or fp32
    // as T, [M][K]); each thread normalizes the float4 columns it reduced
    extern __shared__ __attribute__((aligned(16))) unsigned char gemv_lds[];
    T *An = reinterpret_cast<T *>(gemv_lds);
    if (NORM) {
        __shared__ float red[4];
        constexpr int MAXC = 4;  // float4 columns per thread (K <= 4096)
        float4 gg[MAXC];
#pragma unroll
        for (int i = 0; i < MAXC; ++i) {
            const int c = threadIdx.x * 4 + i * 1024;
            if (c < g.K) gg[i] = *reinterpret_cast<const float4 *>(g.ng + c);
        }
        for (int m = 0; m < g.M; ++m) {
            const float *xr = g.nx + (int64_t)m * g.K;
            float4 v[MAXC];
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < MAXC; ++i) {
                const int c = threadIdx.x * 4 + i * 1024;
                if (c >= g.K) continue;
                v[i] = *reinterpret_cast<const float4 *>(xr + c);
                ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
            }
            ss = block_sum_256(ss, red);
            const float inv = 1.0f / sqrtf(ss / (float)g.K + g.neps);
#pragma unroll
            for (int i = 0; i < MAXC; ++i) {
                const int c = threadIdx.x * 4 + i * 1024;
                if (c >= g.K) continue;
                T *o = An + (int64_t)m * g.K + c;
                o[0] = from_f32<T>(v[i].x * inv * gg[i].x);
                o[1] = from_f32<T>(v[i].y * inv * gg[i].y);
                o[2] = from_f32<T>(v[i].z * inv * gg[i].z);
                o[3] = from_f32<T>(v[i].w * inv * gg[i].w);
            }
        }
        __syncthreads();
    }

    float acc[GEMV_MAXM][2 * GEMV_UNITS];
#pragma unroll
    for (int m = 0; m < GEMV_MAXM; ++m)
#pragma unroll
        for (int u = 0; u < 2 * GEMV_UNITS; ++u) acc[m][u] = 0.f;

    if (KI > 0) {
        // weights are in registers: per row, all of its operand chunks in one round of loads
#pragma unroll
        for (int m = 0; m < GEMV_MAXM; ++m) {
            if (m >= g.M) break;
            float av[KB][V];
#pragma unroll
            for (int c = 0; c < KB; ++c) {
                const int k0 = c * CH + lane * V;
                if (NORM) Vec<T>::load(An + (int64_t)m * g.K + k0, av[c]);
                else Vec<T>::load(A + (int64_t)m * g.lda + k0, av[c]);
            }
#pragma unroll
            for (int c = 0; c < KB; ++c)
#pragma unroll
                for (int u = 0; u < NW; ++u) {
                    float s = acc[m][u];
#pragma unroll
                    for (int e = 0; e < V; ++e) s = fmaf(av[c][e], wv[c][u][e], s);
                    acc[m][u] = s;
                }
        }
    } else {
        for (int k0 = lane * V; k0 < g.K; k0 += CH) {
            float wl[NW][V];
#pragma unroll
            for (int u = 0; u < NW; ++u) Vec<T>::load_nt(wr[u] + k0, wl[u]);
#pragma unroll
            for (int m = 0; m < GEMV_MAXM; ++m) {
                if (m >= g.M) break;
                float av[V];
                if (NORM) Vec<T>::load(An + (int64_t)m * g.K + k0, av);
                else Vec<T>::load(A + (int64_t)m * g.lda + k0, av);
#pragma unroll
                for (int u = 0; u < NW; ++u) {
                    float s = acc[m][u];
#pragma unroll
                    for (int e = 0; e < V; ++e) s = fmaf(av[e], wl[u][e], s);
                    acc[m][u] = s;
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < GEMV_MAXM; ++m) {
        if (m >= g.M) break;
#pragma unroll
        for (int u = 0; u < NW; ++u) acc[m][u] = wave_sum(acc[m][u]);
    }
    if (lane != 0) return;
#pragma unroll
    for (int m = 0; m < GEMV_MAXM; ++m) {
        if (m >= g.M) break;
#pragma unroll
        for (int u = 0; u < GEMV_UNITS; ++u) {
            const int n = unit0 + u;
            if (n >= n_units) continue;
            if (EPI == EPI_SWIGLU) {
                T *C = reinterpret_cast<T *>(g.C);
                C[(int64_t)m * g.ldc + n] = from_f32<T>(silu_f(acc[m][2 * u]) * acc[m][2 * u + 1]);
            } else {
                float *C = reinterpret_cast<float *>(g.C);
                if (EPI == EPI_ADD) C[(int64_t)m * g.ldc + n] += acc[m][u];
                else C[(int64_t)m * g.ldc + n] = acc[m][u];
            }
        }
    }
}

template <typename T, int KI, bool NORM>
static void launch_gemv_k(const GemmArgs &g, int blocks, hipStream_t s) {
    const size_t lds = NORM ? (size_t)g.M * g.K * sizeof(T) : 0;  // <= 64 KB (checked by the caller)
    switch (g.epi) {
        case EPI_STORE: hipLaunchKernelGGL((gemv<T, EPI_STORE, KI, NORM>), dim3(blocks), dim3(256), lds, s, g); break;
        case EPI_ADD: hipLaunchKernelGGL((gemv<T, EPI_ADD, KI, NORM>), dim3(blocks), dim3(256), lds, s, g); break;
        default: hipLaunchKernelGGL((gemv<T, EPI_SWIGLU, KI, NORM>), dim3(blocks), dim3(256), lds, s, g); break;
    }
}

template <typename T>
static void launch_gemv(const GemmArgs &g, hipStream_t s) {
    const int n_units = (g.epi == EPI_SWIGLU) ? g.N / 2 : g.N;
    const int blocks = (n_units + 4 * GEMV_UNITS - 1) / (4 * GEMV_UNITS);
    constexpr int CH = 64 * Vec<T>::N;
    const int ki = g.K % CH == 0 ? g.K / CH : 0;
    if (g.nx) {
        if (ki == 2) launch_gemv_k<T, 2, true>(g, blocks, s);
        else if (ki == 4) launch_gemv_k<T, 4, true>(g, blocks, s);
        else launch_gemv_k<T, 0, true>(g, blocks, s);
        return;
    }
    switch (ki) {
        case 1: launch_gemv_k<T, 1, false>(g, blocks, s); break;
        case 2: launch_gemv_k<T, 2, false>(g, blocks, s); break;
        case 3: launch_gemv_k<T, 3, false>(g, blocks, s); break;
        case 4: launch_gemv_k<T, 4, false>(g, blocks, s); break;
        case 6: launch_gemv_k<T, 6, false>(g, blocks, s); break;
        case 8: launch_gemv_k<T, 8, false>(g, blocks, s); break;
        default: launch_gemv_k<T, 0, false>(g, blocks, s); break;
    }
}

template <int BM, int BN>
static void launch_mfma(const GemmArgs &g, int splits, float *part, hipStream_t s) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    const int kt = g.K / BK;
    const int k_split = ((kt + splits - 1) / splits) * BK;
    splits = (g.K + k_split - 1) / k_split;
    if (splits > 1) {
        GemmArgs gp = g;  // the partial pass writes [splits][M][N] into the workspace
        gp.C = part;
        gp.ldc = g.N;
        hipLaunchKernelGGL((gemm_mfma<BM, BN, EPI_PARTIAL>), dim3(tiles, 1, splits), dim3(256), 0, s, gp, k_split);
        const int64_t outs = (g.epi == EPI_SWIGLU) ? (int64_t)g.M * (g.N / 2) : (int64_t)g.M * g.N;
        int blocks = (int)((outs + 255) / 256);
        if (blocks > 2048) blocks = 2048;
        switch (g.epi) {
            case EPI_STORE: hipLaunchKernelGGL(splitk_reduce<EPI_STORE>, dim3(blocks), dim3(256), 0, s, g, part, splits); break;
            case EPI_ADD: hipLaunchKernelGGL(splitk_reduce<EPI_ADD>, dim3(blocks), dim3(256), 0, s, g, part, splits); break;
            default: hipLaunchKernelGGL(splitk_reduce<EPI_SWIGLU>, dim3(blocks), dim3(256), 0, s, g, part, splits); break;
        }
        return;
    }
    switch (g.epi) {
        case EPI_STORE: hipLaunchKernelGGL((gemm_mfma<BM, BN, EPI_STORE>), dim3(tiles), dim3(256), 0, s, g, g.K); break;
        case EPI_ADD: hipLaunchKernelGGL((gemm_mfma<BM, BN, EPI_ADD>), dim3(tiles), dim3(256), 0, s, g, g.K); break;
        default: hipLaunchKernelGGL((gemm_mfma<BM, BN, EPI_SWIGLU>), dim3(tiles), dim3(256), 0, s, g, g.K); break;
    }
}

// Split count: enough blocks to cover the 256 CUs once, at least 2 K tiles per
// split, and a partial buffer that fits the workspace.
static int choose_splits(const GemmArgs &g, int tiles, int64_t part_cap) {
    const int kt = g.K / BK;
    int splits = 1;
    while (tiles * splits < 256 && 2 * (splits * 2) <= kt &&
           (int64_t)(splits * 2) * g.M * g.N <= part_cap)
        splits *= 2;
    return splits;
}

bool launch_head_scores(const GemmArgs &g, hipStream_t s) {
    if (g.M <= 64 || g.K % 64 != 0 || g.gv < 128 || !g.spart) return false;
    const int tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128);
    hipLaunchKernelGGL((gemm_lds<128, 128, 2, EPI_SCORES>), dim3(tiles), dim3(256), 0, s, g, g.K, RopeKvArgs{});
    return true;
}

bool launch_qkv_dense(const GemmArgs &g, const RopeKvArgs &rk, hipStream_t s) {
    // one tile per (128 tokens, head): needs M > 64 (the LDS-DMA kernel), 128-wide heads
    if (g.M <= 64 || g.K % 64 != 0 || g.N != (rk.H + 2 * rk.Hkv) * 128 || g.epi != EPI_STORE) return false;
    const int tiles = ((g.M + 127) / 128) * (g.N / 128);
    // one tile per CU or fewer: the 4-stage ring (128 KB, one block per CU) hides more of
    // the operand latency (M = 950: 21.8 -> 19.1 us); more tiles: two stages, two blocks
    // per CU (four stages made the 1728-row guided product slower)
    if (tiles <= 256) hipLaunchKernelGGL((gemm_lds<128, 128, 4, EPI_QKV>), dim3(tiles), dim3(256), 0, s, g, g.K, rk);
    else hipLaunchKernelGGL((gemm_lds<128, 128, 2, EPI_QKV>), dim3(tiles), dim3(256), 0, s, g, g.K, rk);
    return true;
}

int launch_gemm(const GemmArgs &g, DType dt, float *part, int64_t part_cap, hipStream_t s) {
    if (g.M <= 0) return 0;
    if (dt == DT_F32) {
        // fp32 mode streams weights; larger M is processed GEMV_MAXM rows at a time
        for (int m0 = 0; m0 < g.M; m0 += GEMV_MAXM) {
            GemmArgs h = g;
            h.M = g.M - m0 < GEMV_MAXM ? g.M - m0 : GEMV_MAXM;
            h.A = reinterpret_cast<const float *>(g.A) + (int64_t)m0 * g.lda;
            h.C = reinterpret_cast<float *>(g.C) + (int64_t)m0 * g.ldc;
            if (g.nx) h.nx = g.nx + (int64_t)m0 * g.K;
            launch_gemv<float>(h, s);
        }
        return 0;
    }
    if (g.M <= GEMV_MAXM) {
        launch_gemv<bf16_t>(g, s);
        return 0;
    }
    if (g.M <= 64) {
        const int pending = launch_skinny(g, part, part_cap, s);
        if (pending >= 0) return pending;
    }
    // M > 64 (the MaskGIT pass, prefill-sized products): the LDS-DMA kernel.  Tile
    // choice from measured sweeps and whole-pass runs on MI355X at the backbone's shapes:
    // * 128x128 tiles with a two-stage ring (64 KB of LDS: two blocks fit on a CU) when
    //   there are >= 128 of them; but gate|up, when 192x128 tiles fit the CUs once, runs
    //   those in a three-stage ring (120 KB, one block per CU: M = 950 23.4 -> 21.4 us;
    //   256x128 tiles were slower, 25.3 us);
    // * a residual-add product whose 128x64 tiles, split over K in 2 or 4, make 224..256
    //   blocks (one per CU): a four-stage ring of those (M = 950: o 12.8 -> 11.9 us, down
    //   17.1 -> 15.4 us); with fewer or more blocks this lost to the next rule;
    // * otherwise 64x64 tiles, and a residual-add product is split over K until there
    //   are >= 256 blocks.
    // Split partials are deferred to the next RMSNorm.
    if (g.M > 64 && g.K % 64 == 0) {
        const int t128 = ((g.M + 127) / 128) * ((g.N + 127) / 128);
        if (t128 >= 128) {
            if (g.epi == EPI_SWIGLU && ((g.M + 191) / 192) * ((g.N + 127) / 128) <= 256)
                return launch_gemm_lds<192, 128, 3>(g, 1, part, s);
            return launch_gemm_lds<128, 128, 2>(g, 1, part, s);
        }
        if (g.epi == EPI_SWIGLU) return launch_gemm_lds<64, 128, 4>(g, 1, part, s);
        if (g.epi == EPI_ADD) {
            const int t = ((g.M + 127) / 128) * ((g.N + 63) / 64);
            int sp = 1;
            while (t * sp * 2 <= 256 && g.K / 64 >= 8 * sp && sp < 4 && (int64_t)(sp * 2) * g.M * g.N <= part_cap)
                sp *= 2;
            if (sp >= 2 && t * sp >= 224) return launch_gemm_lds<128, 64, 4>(g, sp, part, s);
        }
        const int t64 = ((g.M + 63) / 64) * ((g.N + 63) / 64);
        int splits = 1;
        if (g.epi == EPI_ADD)
            while (t64 * splits < 256 && g.K / 64 >= 8 * splits && splits < 4 &&
                   (int64_t)(splits * 2) * g.M * g.N <= part_cap)
                splits *= 2;
        return launch_gemm_lds<64, 64, 4>(g, splits, part, s);
    }
    // Small M or N = hidden: 32x64 tiles of the 16x16x32 kernel (more blocks in flight),
    // split over K only when there are few tiles.
    const int t32 = ((g.M + 31) / 32) * ((g.N + 63) / 64);
    launch_mfma<32, 64>(g, t32 < 64 ? choose_splits(g, t32, part_cap) : 1, part, s);
    return 0;
}

}  // namespace ttsbb
