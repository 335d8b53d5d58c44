/*
 * synth.c - seeded, counter-based generator of synthetic input tensors.
 *
 * Holds none of the convolution / pooling arithmetic: it only turns
 * (seed, stream, element index) into numbers, so that the GPU library's
 * tests, the CPU oracle and the benchmark all see identical inputs, and any
 * element range can be regenerated on its own.
 *
 * Bits: Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 128-bit
 * counter and a 64-bit key pass through 10 rounds of two 32x32->64-bit
 * multiplies (constants 0xD2511F53, 0xCD9E8D57) with a Weyl key schedule
 * (0x9E3779B9, 0xBB67AE85).
 *
 * Mapping: element i of a tensor drawn from (seed, stream) takes word (i & 3)
 * of the Philox block with counter {lo32(i>>2), hi32(i>>2), stream, 0} and
 * key {lo32(seed), hi32(seed)}.
 *   uniform [lo, hi):  u = (word >> 8) * 2^-24, value = lo + (hi - lo) * u
 *   normal N(0,1):     Box-Muller on the word pair {2j, 2j+1} (j = (i&3) >> 1):
 *                      u1 = (w0 + 1) * 2^-32, u2 = w1 * 2^-32,
 *                      r = sqrt(-2 ln u1), even i -> r cos(2 pi u2),
 *                      odd i -> r sin(2 pi u2)
 * computed in double and rounded once to float.
 * bf16: round-to-nearest-even of the float's upper 16 bits (NaN kept quiet).
 */
#include <math.h>
#include <stdint.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                         uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static void block_words(uint64_t seed, uint32_t stream, uint64_t blk, uint32_t w[4])
{
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    synth_philox4x32_10(ctr, key, w);
}

/* out[j] = U[lo, hi) element (first + j) of (seed, stream), j < count. */
void synth_uniform_f32(uint64_t seed, uint32_t stream, uint64_t first,
                       uint64_t count, double lo, double hi, float *out)
{
    const double inv24 = 1.0 / 16777216.0;
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)count; ++j) {
        uint64_t i = first + (uint64_t)j;
        uint32_t w[4];
        block_words(seed, stream, i >> 2, w);
        double u = (double)(w[i & 3u] >> 8) * inv24;
        out[j] = (float)(lo + (hi - lo) * u);
    }
}

/* out[j] = N(0,1) element (first + j) of (seed, stream), j < count.
 * Walks whole Philox blocks (4 elements, two Box-Muller pairs) at a time. */
void synth_normal_f32(uint64_t seed, uint32_t stream, uint64_t first,
                      uint64_t count, float *out)
{
    const double inv32 = 1.0 / 4294967296.0;
    const double two_pi = 6.283185307179586476925286766559;
    if (count == 0) return;
    uint64_t b0 = first >> 2, b1 = (first + count - 1) >> 2;
    #pragma omp parallel for schedule(static)
    for (int64_t bb = 0; bb <= (int64_t)(b1 - b0); ++bb) {
        uint64_t blk = b0 + (uint64_t)bb;
        uint32_t w[4];
        block_words(seed, stream, blk, w);
        double v[4];
        for (int pair = 0; pair < 2; ++pair) {
            double u1 = ((double)w[2 * pair] + 1.0) * inv32;
            double u2 = (double)w[2 * pair + 1] * inv32;
            double r = sqrt(-2.0 * log(u1));
            double t = two_pi * u2;
            v[2 * pair] = r * cos(t);
            v[2 * pair + 1] = r * sin(t);
        }
        for (int e = 0; e < 4; ++e) {
            uint64_t i = blk * 4u + (uint64_t)e;
            if (i < first || i >= first + count) continue;
            out[i - first] = (float)v[e];
        }
    }
}

/* bf16 bits of each float, round to nearest even. */
void synth_f32_to_bf16(const float *in, uint64_t count, uint16_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)count; ++j) {
        union { float f; uint32_t u; } v;
        v.f = in[j];
        uint32_t u = v.u;
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
            out[j] = (uint16_t)((u >> 16) | 0x0040u);
        } else {
            u += 0x7FFFu + ((u >> 16) & 1u);
            out[j] = (uint16_t)(u >> 16);
        }
    }
}
