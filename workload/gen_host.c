/* Host fast path of the seeded input generator in workload/gen.py.
 *
 * Same definition: element e of stream s under seed is word (e % 4) of
 * Philox4x32-10(counter = (e/4 lo, e/4 hi, s, 0), key = (seed lo, seed hi)),
 * then the integer Irwin-Hall variate k in [-1535, 1535] and fp32(k) * scale.
 * Holds no model arithmetic.  Built with plain gcc; no fast-math.
 */
#include <stdint.h>
#include <string.h>

static void philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

static inline int32_t normal_k(uint32_t w) {
    return (int32_t)(w & 1023u) + (int32_t)((w >> 10) & 1023u) + (int32_t)((w >> 20) & 1023u) +
           (int32_t)((w >> 30) & 1u) - 1535;
}

static inline uint16_t bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* out[i] = word for element start+i */
void wl_words(uint64_t seed, uint32_t stream, uint64_t start, int64_t n, uint32_t *out) {
    if (n <= 0) return;
    int64_t b0 = (int64_t)(start >> 2), b1 = (int64_t)((start + (uint64_t)n + 3) >> 2);
#pragma omp parallel for schedule(static)
    for (int64_t b = b0; b < b1; ++b) {
        uint32_t c[4] = {(uint32_t)b, (uint32_t)((uint64_t)b >> 32), stream, 0u};
        philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
        for (int j = 0; j < 4; ++j) {
            int64_t i = 4 * b + j - (int64_t)start;
            if (i >= 0 && i < n) out[i] = c[j];
        }
    }
}

/* fp32 normal variates (mode 0) or their bf16 bit patterns (mode 1). */
void wl_normal(uint64_t seed, uint32_t stream, uint64_t start, int64_t n, float scale, int mode,
               void *out) {
    if (n <= 0) return;
    float *of = (float *)out;
    uint16_t *ob = (uint16_t *)out;
    int64_t b0 = (int64_t)(start >> 2), b1 = (int64_t)((start + (uint64_t)n + 3) >> 2);
#pragma omp parallel for schedule(static)
    for (int64_t b = b0; b < b1; ++b) {
        uint32_t c[4] = {(uint32_t)b, (uint32_t)((uint64_t)b >> 32), stream, 0u};
        philox(c, (uint32_t)seed, (uint32_t)(seed >> 32));
        for (int j = 0; j < 4; ++j) {
            int64_t i = 4 * b + j - (int64_t)start;
            if (i < 0 || i >= n) continue;
            float v = (float)normal_k(c[j]) * scale; /* one rounded fp32 product */
            if (mode == 0) of[i] = v; else ob[i] = bf16_rne(v);
        }
    }
}
