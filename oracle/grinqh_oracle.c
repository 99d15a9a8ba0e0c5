/*
 * Plain fp64 CPU oracle for the GRINQH batch-1 decode GEMV (C version).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests and by the bench's CPU
 * baseline leg, never by the HIP library, and it includes nothing from it.
 *
 * Source: the page "GRINQH: Graded Input-Based Quantization Hierarchy for
 * Efficient LLM Generation" (papernotes.org note on arXiv 2606.23419),
 * section 方法详解 / 关键设计 (key design), items 1-3:
 *   KD1 bit assignment by comparing |x_i| with ascending thresholds,
 *   KD2 2-bit planes, most significant first, reduction-dim-major, 16 per uint32,
 *   KD3 w_hat = s * (q_b * 2^(b_max - b) + phi) + z with phi = 2^(b_max - b - 1).
 * The readings for points the page leaves open are the same as in the numpy
 * oracle (grinqh_oracle.py): P = b_max/2 thresholds, ties go up, NaN -> 0
 * bits, phi = 1/2 at b = b_max, skipped channels contribute nothing,
 * fragment of output 16w+t at bits [2t, 2t+1] of word w, rows padded to 64.
 *
 * Deliberately naive: one output at a time, one input channel at a time.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* KD1.  x and theta hold the exact fp32/bf16 values widened to double. */
void oracle_assign_bits(const double* x, const double* theta, int d_in, int b_max,
                        uint8_t* bits) {
    int P = b_max / 2;
    for (int i = 0; i < d_in; ++i) {
        double a = fabs(x[i]);
        int level = 0;
        for (int k = 0; k < P; ++k)
            if (theta[k] <= a) level += 1;   /* NaN: every test false */
        bits[i] = (uint8_t)(2 * level);
    }
}

/* KD2.  q is uint8 [d_out][d_in]; planes is uint32 [d_in][P][W_row]. */
void oracle_pack(const uint8_t* q, int d_in, int d_out, int b_max, uint32_t* planes) {
    int P = b_max / 2;
    int W = ((d_out + 63) / 64) * 4;
    unsigned mask = (1u << b_max) - 1u;
    for (int i = 0; i < d_in; ++i)
        for (int p = 0; p < P; ++p)
            for (int w = 0; w < W; ++w) {
                uint32_t word = 0;
                for (int t = 0; t < 16; ++t) {
                    int j = 16 * w + t;
                    if (j >= d_out) continue;
                    unsigned code = q[(size_t)j * d_in + i] & mask;
                    unsigned frag = (code >> (b_max - 2 * p - 2)) & 3u;
                    word |= (uint32_t)frag << (2 * t);
                }
                planes[((size_t)i * P + p) * W + w] = word;
            }
}

/* KD1 + KD3.  q holds n_out rows of d_in codes (any subset of output channels,
 * with s and z for the same rows); y gets n_out values. */
void oracle_gemv(const double* x, const double* theta, const uint8_t* q,
                 const double* s, const double* z, int d_in, int n_out, int b_max,
                 uint8_t* scratch_bits, double* y) {
    unsigned mask = (1u << b_max) - 1u;
    oracle_assign_bits(x, theta, d_in, b_max, scratch_bits);
    for (int j = 0; j < n_out; ++j) {
        double sum = 0.0;
        const uint8_t* row = q + (size_t)j * d_in;
        for (int i = 0; i < d_in; ++i) {
            int b = scratch_bits[i];
            if (b == 0) continue;                 /* channel not loaded */
            int k = b_max - b;
            unsigned code = ((unsigned)(row[i] & mask) >> k) << k;
            double ph = ldexp(1.0, k - 1);
            double w = s[j] * ((double)code + ph) + z[j];
            sum += x[i] * w;
        }
        y[j] = sum;
    }
}
