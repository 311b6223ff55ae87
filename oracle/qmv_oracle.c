/*
 * qmv_oracle.c -- plain, slow, scalar CPU oracle for the quantized
 * matrix-vector product (MMVQ): K-quant weights (Q6_K, Q4_K, Q5_K) times
 * activations quantized to Q8_1, at 1..8 activation columns, plus the
 * grouped MoE-expert chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code, header, table or constant generator with the GPU library; it is
 * written from the pages' description of the method and from the block
 * layouts they name.
 *
 * Sources (the pages, by title and section):
 *   [P2340] "sycl mmvq: Q6_K decode kernels no longer ALU-bound; Q6_K output
 *           heads as aligned planes; int4 activation loads", section
 *           "What it changes".
 *   [P1774] "sycl opt-in: STRATA_IQ3S_WIDE=1, a wide mmvq kernel for the
 *           dense IQ3_S matrices", section "What changed".
 *   [P2207] "Issue: #1545, #1606 (Arc A-series decode)" (large-GRF launch),
 *           sections "Summary" and "How it was checked".
 *   [P2746] "sycl: use packed word expansion for Q2_0 expert down on
 *           Battlemage", sections "Summary", "B70 validation" and
 *           "Down microbenchmark".
 *   [I2801] "[Feature]: SYCL: cheaper IQ weight decodes in the grouped
 *           expert kernels".
 *
 * What the pages fix: each 32-weight sub-block contributes
 * d_w * scale * d_a * (integer dot of the weight quants with the Q8_1 quants)
 * [P1774 "What changed"]; products accumulate in FP32 after INT8 dot
 * products [P2746 "Summary"]; the weights are GGUF-layout K-quant blocks and
 * the activations Q8_1 blocks with 4-byte aligned quants [P2340 "What it
 * changes"]; the routed-expert kernels run gate/up and down over a window of
 * tokens [I2801].  What the pages leave open (bit layout inside a block,
 * rounding in the activation quantizer, the min term of Q4_K/Q5_K, SiLU) is
 * read as stated at each function below.
 *
 * Floating point: every float result here is computed in fp64 from exact
 * integer block sums, so it equals the plain definition
 *     out[n][r] = sum_i w[r][i] * xhat[n][i]
 * (w the dequantized weight, xhat = d_a * q8 the dequantized activation) up
 * to fp64 rounding of the final sums.  The activation quantizer is the one
 * place that must use fp32, because its output is an integer code: it
 * follows the reading "d = amax/127 in fp32, q = round-half-away(x/d) in
 * fp32".
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 256          /* weights per K-quant superblock */
#define QB 32           /* weights per Q8_1 block / K-quant sub-block */
#define Q6K_BYTES 210
#define Q4K_BYTES 144
#define Q5K_BYTES 176
#define Q81_BYTES 36

/* ------------------------------------------------------------------ fp16 */

/* IEEE 754 binary16 -> double, exact for every pattern (subnormals, inf,
 * NaN).  value = (1024 + m) * 2^(e-25) for normal numbers and
 * m * 2^-24 for subnormals. */
double orc_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* float -> binary16 with round-to-nearest-even.  Works on the exact value
 * in double: scale so that the 11 significant bits become the integer part,
 * round with rint (ties to even under the default rounding mode). */
uint16_t orc_float_to_half(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f)) return sign | 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;          /* rounds past 65504 */
    if (a < ldexp(1.0, -14)) {                          /* subnormal range */
        double q = rint(a * ldexp(1.0, 24));            /* units of 2^-24 */
        return sign | (uint16_t)q;                      /* 1024 -> min normal */
    }
    int ex;
    frexp(a, &ex);                                      /* a = fr*2^ex */
    int E = ex - 1;                                     /* a in [2^E, 2^E+1) */
    double q = rint(ldexp(a, 10 - E));                  /* in [1024, 2048] */
    if (q == 2048.0) { q = 1024.0; E += 1; }
    if (E + 15 >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024));
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = v & 0xff; p[1] = v >> 8; }

/* ------------------------------------------------------ block decoders
 * Bit layouts: the pages name GGUF-layout Q6_K/Q4_K/Q5_K blocks
 * [P2340 "What it changes"] without spelling the bits out; the reading used
 * is the GGUF K-quant convention:
 *   Q6_K (210 B): ql[128] @0, qh[64] @128, int8 scales[16] @192, fp16 d @208.
 *     weight i: h = i/128, c = (i%128)/32, l = i%32,
 *     low4  = (ql[64h + 32(c%2) + l] >> 4(c/2)) & 15,
 *     high2 = (qh[32h + l] >> 2c) & 3,
 *     q6 = low4 | high2<<4 in [0,63];  w = d * scales[i/16] * (q6 - 32).
 *   Q4_K (144 B): fp16 d @0, fp16 dmin @2, scales[12] @4, qs[128] @16.
 *     sub-block j = i/32, l = i%32: q4 = (qs[32(j/2) + l] >> 4(j%2)) & 15,
 *     (sc_j, m_j) 6-bit from the 12 scale bytes (q4k_scale_min),
 *     w = d*sc_j*q4 - dmin*m_j.
 *   Q5_K (176 B): as Q4_K with qh[32] @16 and qs[128] @48;
 *     q5 = q4 | ((qh[l] >> j) & 1) << 4.
 */

void orc_q6k_decode(const uint8_t *blk, int8_t *q, int8_t *sc, double *d) {
    const uint8_t *ql = blk, *qh = blk + 128;
    for (int i = 0; i < QK; i++) {
        int h = i / 128, c = (i % 128) / 32, l = i % 32;
        int low4 = (ql[64 * h + 32 * (c % 2) + l] >> (4 * (c / 2))) & 15;
        int high2 = (qh[32 * h + l] >> (2 * c)) & 3;
        q[i] = (int8_t)((low4 | (high2 << 4)) - 32);
    }
    for (int j = 0; j < 16; j++) sc[j] = (int8_t)blk[192 + j];
    *d = orc_half_to_double(rd16(blk + 208));
}

/* 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes:
 * j < 4: low six bits of bytes j and j+4; j >= 4: the low/high nibble of
 * byte j+4 joined with the top two bits of bytes j-4 / j. */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

void orc_q4k_decode(const uint8_t *blk, uint8_t *q, uint8_t *sc, uint8_t *m,
                    double *d, double *dmin) {
    const uint8_t *qs = blk + 16;
    for (int i = 0; i < QK; i++) {
        int j = i / 32, l = i % 32;
        q[i] = (qs[32 * (j / 2) + l] >> (4 * (j % 2))) & 15;
    }
    for (int j = 0; j < 8; j++) {
        int a, b;
        q4k_scale_min(blk + 4, j, &a, &b);
        sc[j] = (uint8_t)a;
        m[j] = (uint8_t)b;
    }
    *d = orc_half_to_double(rd16(blk));
    *dmin = orc_half_to_double(rd16(blk + 2));
}

void orc_q5k_decode(const uint8_t *blk, uint8_t *q, uint8_t *sc, uint8_t *m,
                    double *d, double *dmin) {
    const uint8_t *qh = blk + 16, *qs = blk + 48;
    for (int i = 0; i < QK; i++) {
        int j = i / 32, l = i % 32;
        int q4 = (qs[32 * (j / 2) + l] >> (4 * (j % 2))) & 15;
        q[i] = (uint8_t)(q4 | (((qh[l] >> j) & 1) << 4));
    }
    for (int j = 0; j < 8; j++) {
        int a, b;
        q4k_scale_min(blk + 4, j, &a, &b);
        sc[j] = (uint8_t)a;
        m[j] = (uint8_t)b;
    }
    *d = orc_half_to_double(rd16(blk));
    *dmin = orc_half_to_double(rd16(blk + 2));
}

/* Full-matrix dequantization to fp64, rows x K, row-major blocks. */
void orc_dequant_q6k(const uint8_t *w, double *out, int64_t rows, int64_t K) {
    int64_t nb = K / QK;
    int8_t q[QK], sc[16];
    double d;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t s = 0; s < nb; s++) {
            orc_q6k_decode(w + (r * nb + s) * Q6K_BYTES, q, sc, &d);
            for (int i = 0; i < QK; i++)
                out[r * K + s * QK + i] = d * (double)sc[i / 16] * (double)q[i];
        }
}

static void dequant_q45(const uint8_t *w, double *out, int64_t rows, int64_t K,
                        int five) {
    int64_t nb = K / QK;
    int bytes = five ? Q5K_BYTES : Q4K_BYTES;
    uint8_t q[QK], sc[8], m[8];
    double d, dmin;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t s = 0; s < nb; s++) {
            const uint8_t *blk = w + (r * nb + s) * bytes;
            if (five) orc_q5k_decode(blk, q, sc, m, &d, &dmin);
            else orc_q4k_decode(blk, q, sc, m, &d, &dmin);
            for (int i = 0; i < QK; i++)
                out[r * K + s * QK + i] =
                    d * (double)sc[i / 32] * (double)q[i] - dmin * (double)m[i / 32];
        }
}
void orc_dequant_q4k(const uint8_t *w, double *out, int64_t rows, int64_t K) {
    dequant_q45(w, out, rows, K, 0);
}
void orc_dequant_q5k(const uint8_t *w, double *out, int64_t rows, int64_t K) {
    dequant_q45(w, out, rows, K, 1);
}

/* ------------------------------------------------------------ Q8_1
 * Q8_1 block (36 B): fp16 d @0, fp16 s @2, int8 q[32] @4 (quants 4-byte
 * aligned, [P2340 "What it changes"]).  Reading of the quantizer, per block
 * of 32 values of one column:
 *   amax = max |x|;  d = amax / 127 (fp32 division);
 *   d == 0: every q = 0;  otherwise q = round-half-away-from-zero(x / d)
 *   (fp32 division), clamped to [-127, 127];
 *   stored d = fp16_rne(d), s = fp16_rne(d * (float)sum(q)) (fp32 product).
 * x is [ncols][K] fp32, xq is [ncols][K/32] blocks.  Inputs must be finite.
 */
void orc_quantize_q8_1(const float *x, uint8_t *xq, int64_t K, int ncols) {
    int64_t nb = K / QB;
    for (int n = 0; n < ncols; n++)
        for (int64_t b = 0; b < nb; b++) {
            const float *xb = x + (int64_t)n * K + b * QB;
            uint8_t *o = xq + ((int64_t)n * nb + b) * Q81_BYTES;
            float amax = 0.0f;
            for (int i = 0; i < QB; i++) {
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            int sum = 0;
            for (int i = 0; i < QB; i++) {
                int qi = 0;
                if (d != 0.0f) {
                    float v = xb[i] / d;
                    float r = roundf(v);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    qi = (int)r;
                }
                o[4 + i] = (uint8_t)(int8_t)qi;
                sum += qi;
            }
            wr16(o, orc_float_to_half(d));
            wr16(o + 2, orc_float_to_half(d * (float)sum));
        }
}

/* RMSNorm of each activation column (the norm ahead of the quantizer whose
 * fused opt-in IQ3 "How it was checked" measures; the pages do not define
 * the norm, read as RMSNorm): r = 1/sqrt(mean(x^2) + eps) and
 * y = x * r * gamma, all in fp64, y rounded to fp32 once.  The fused
 * quantization is then orc_quantize_q8_1 of y. */
void orc_rmsnorm(const float *x, const float *gamma, double eps, float *y, int64_t K, int ncols) {
    for (int n = 0; n < ncols; n++) {
        const float *xc = x + (int64_t)n * K;
        double ss = 0.0;
        for (int64_t i = 0; i < K; i++) ss += (double)xc[i] * (double)xc[i];
        const double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t i = 0; i < K; i++) y[(int64_t)n * K + i] = (float)((double)xc[i] * r * (double)gamma[i]);
    }
}

/* Dequantized activation xhat = d * q (fp64), [ncols][K]. */
void orc_dequant_q8_1(const uint8_t *xq, double *out, int64_t K, int ncols) {
    int64_t nb = K / QB;
    for (int n = 0; n < ncols; n++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = xq + ((int64_t)n * nb + b) * Q81_BYTES;
            double d = orc_half_to_double(rd16(blk));
            for (int i = 0; i < QB; i++)
                out[(int64_t)n * K + b * QB + i] = d * (double)(int8_t)blk[4 + i];
        }
}

/* ------------------------------------------------------- integer sums
 * For column n, row r and Q8_1 block b (= K-quant sub-block b%8 of
 * superblock b/8):
 *   Q6_K: isum = sum over the two 16-weight scale groups g of the sub-block
 *         of scales[g] * sum_{i in g} (q6_i - 32) * q8_i;
 *   Q4_K/Q5_K: dot = sum_{i in b} q_i * q8_i (no scale applied).
 * All exact in int32 (|Q6_K isum| < 2^24).  Output [ncols][rows][K/32].
 * rows_out rows starting at row0 are produced (row0 = 0, rows_out = rows for
 * the whole matrix).
 */
void orc_q6k_isums(const uint8_t *w, const uint8_t *xq, int32_t *isums,
                   int64_t rows, int64_t K, int ncols) {
    int64_t nb = K / QK, nsb = K / QB;
    int8_t q[QK], sc[16];
    double d;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t s = 0; s < nb; s++) {
            orc_q6k_decode(w + (r * nb + s) * Q6K_BYTES, q, sc, &d);
            for (int n = 0; n < ncols; n++)
                for (int j = 0; j < 8; j++) {
                    int64_t b = s * 8 + j;
                    const uint8_t *xb = xq + ((int64_t)n * nsb + b) * Q81_BYTES + 4;
                    int32_t total = 0;
                    for (int g = 0; g < 2; g++) {
                        int32_t dot = 0;
                        for (int i = 0; i < 16; i++)
                            dot += (int32_t)q[32 * j + 16 * g + i] * (int8_t)xb[16 * g + i];
                        total += (int32_t)sc[2 * j + g] * dot;
                    }
                    isums[((int64_t)n * rows + r) * nsb + b] = total;
                }
        }
}

static void q45_dots(const uint8_t *w, const uint8_t *xq, int32_t *dots,
                     int64_t rows, int64_t K, int ncols, int five) {
    int64_t nb = K / QK, nsb = K / QB;
    int bytes = five ? Q5K_BYTES : Q4K_BYTES;
    uint8_t q[QK], sc[8], m[8];
    double d, dmin;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t s = 0; s < nb; s++) {
            const uint8_t *blk = w + (r * nb + s) * bytes;
            if (five) orc_q5k_decode(blk, q, sc, m, &d, &dmin);
            else orc_q4k_decode(blk, q, sc, m, &d, &dmin);
            for (int n = 0; n < ncols; n++)
                for (int j = 0; j < 8; j++) {
                    int64_t b = s * 8 + j;
                    const uint8_t *xb = xq + ((int64_t)n * nsb + b) * Q81_BYTES + 4;
                    int32_t dot = 0;
                    for (int i = 0; i < QB; i++)
                        dot += (int32_t)q[32 * j + i] * (int8_t)xb[i];
                    dots[((int64_t)n * rows + r) * nsb + b] = dot;
                }
        }
}
void orc_q4k_dots(const uint8_t *w, const uint8_t *xq, int32_t *dots,
                  int64_t rows, int64_t K, int ncols) {
    q45_dots(w, xq, dots, rows, K, ncols, 0);
}
void orc_q5k_dots(const uint8_t *w, const uint8_t *xq, int32_t *dots,
                  int64_t rows, int64_t K, int ncols) {
    q45_dots(w, xq, dots, rows, K, ncols, 1);
}

/* ------------------------------------------------------------- MMVQ
 * out[n][r] = sum_b d_w(r, b/8) * d_a(n, b) * isum(n, r, b)      (Q6_K)
 * out[n][r] = sum_b d*d_a*sc_j*dot - dmin*d_a*m_j*S(n, b)         (Q4_K/Q5_K)
 * with S(n, b) the exact integer sum of the block's Q8_1 quants (reading: the
 * min term uses the exact quant sum, so the result equals the plain
 * definition sum_i w_i * xhat_i).  Every product term is exact in fp64; the
 * sum is taken in ascending b.  absum[n][r] = sum of |term| over every term
 * added (both terms for Q4_K/Q5_K), the scale of the fp32 rounding error a
 * reordered sum may carry.  Rows [row0, row0 + nrows) are computed and
 * written at out[n * nrows + (r - row0)].
 */
void orc_mmvq_q6k(const uint8_t *w, const uint8_t *xq, double *out, double *absum,
                  int64_t rows, int64_t K, int ncols, int64_t row0, int64_t nrows) {
    int64_t nb = K / QK, nsb = K / QB;
    int8_t q[QK], sc[16];
    double d;
    (void)rows;
    for (int64_t rr = 0; rr < nrows; rr++) {
        int64_t r = row0 + rr;
        for (int n = 0; n < ncols; n++) {
            out[(int64_t)n * nrows + rr] = 0.0;
            if (absum) absum[(int64_t)n * nrows + rr] = 0.0;
        }
        for (int64_t s = 0; s < nb; s++) {
            orc_q6k_decode(w + (r * nb + s) * Q6K_BYTES, q, sc, &d);
            for (int n = 0; n < ncols; n++)
                for (int j = 0; j < 8; j++) {
                    int64_t b = s * 8 + j;
                    const uint8_t *blk = xq + ((int64_t)n * nsb + b) * Q81_BYTES;
                    double da = orc_half_to_double(rd16(blk));
                    int32_t total = 0;
                    for (int g = 0; g < 2; g++) {
                        int32_t dot = 0;
                        for (int i = 0; i < 16; i++)
                            dot += (int32_t)q[32 * j + 16 * g + i] * (int8_t)blk[4 + 16 * g + i];
                        total += (int32_t)sc[2 * j + g] * dot;
                    }
                    double term = d * da * (double)total;
                    out[(int64_t)n * nrows + rr] += term;
                    if (absum) absum[(int64_t)n * nrows + rr] += fabs(term);
                }
        }
    }
}

static void mmvq_q45(const uint8_t *w, const uint8_t *xq, double *out, double *absum,
                     int64_t K, int ncols, int64_t row0, int64_t nrows, int five) {
    int64_t nb = K / QK, nsb = K / QB;
    int bytes = five ? Q5K_BYTES : Q4K_BYTES;
    uint8_t q[QK], sc[8], m[8];
    double d, dmin;
    for (int64_t rr = 0; rr < nrows; rr++) {
        int64_t r = row0 + rr;
        for (int n = 0; n < ncols; n++) {
            out[(int64_t)n * nrows + rr] = 0.0;
            if (absum) absum[(int64_t)n * nrows + rr] = 0.0;
        }
        for (int64_t s = 0; s < nb; s++) {
            const uint8_t *wb = w + (r * nb + s) * bytes;
            if (five) orc_q5k_decode(wb, q, sc, m, &d, &dmin);
            else orc_q4k_decode(wb, q, sc, m, &d, &dmin);
            for (int n = 0; n < ncols; n++)
                for (int j = 0; j < 8; j++) {
                    int64_t b = s * 8 + j;
                    const uint8_t *blk = xq + ((int64_t)n * nsb + b) * Q81_BYTES;
                    double da = orc_half_to_double(rd16(blk));
                    int32_t dot = 0, qsum = 0;
                    for (int i = 0; i < QB; i++) {
                        int8_t qi = (int8_t)blk[4 + i];
                        dot += (int32_t)q[32 * j + i] * qi;
                        qsum += qi;
                    }
                    double t1 = d * da * (double)sc[j] * (double)dot;
                    double t2 = dmin * da * (double)m[j] * (double)qsum;
                    out[(int64_t)n * nrows + rr] += t1 - t2;
                    if (absum) absum[(int64_t)n * nrows + rr] += fabs(t1) + fabs(t2);
                }
        }
    }
}
void orc_mmvq_q4k(const uint8_t *w, const uint8_t *xq, double *out, double *absum,
                  int64_t rows, int64_t K, int ncols, int64_t row0, int64_t nrows) {
    (void)rows;
    mmvq_q45(w, xq, out, absum, K, ncols, row0, nrows, 0);
}
void orc_mmvq_q5k(const uint8_t *w, const uint8_t *xq, double *out, double *absum,
                  int64_t rows, int64_t K, int ncols, int64_t row0, int64_t nrows) {
    (void)rows;
    mmvq_q45(w, xq, out, absum, K, ncols, row0, nrows, 1);
}

/* ------------------------------------------------------- planar Q6_K
 * Load-time conversion of GGUF Q6_K blocks into aligned planes holding the
 * same number of bytes [P2340 "What it changes": the output heads are
 * converted at load into planes of the same bytes so each lane issues single
 * aligned 16-byte loads].  The plane contents follow the GPU library's
 * published planar layout (its C header), restated here from that text:
 *   NB = rows*K/256 blocks, block t = r*(K/256) + s.
 *   v_i = (q6_i - 32) mod 64 for the 256 weights (six bits each).
 *   Plane A at byte 0, 128 B per block, 16 B per sub-block j (0..7):
 *     byte k (0..15) = v[32j+k] << 2 | spare_A(k).
 *   Plane B at byte 128*NB, 64 B per block, 8 B per sub-block:
 *     byte k (0..7) = v[32j+16+k] << 2 | spare_B(k).
 *   The two spare bits of every byte carry weights 32j+24 .. 32j+31:
 *     for k = 0..3, weight 32j+24+k: bits 0-1 of v in spare_A(k),
 *       bits 2-3 in spare_A(4+k), bits 4-5 in spare_A(8+k);
 *     weight 32j+28+k: bits 0-1 in spare_A(12+k), bits 2-3 in spare_B(k),
 *       bits 4-5 in spare_B(4+k).
 *   Plane SC at byte 192*NB, 16 B per block: the 16 int8 scales unchanged.
 *   Plane D at byte 208*NB, 2 B per block: fp16 d unchanged.
 */
void orc_q6k_to_planar(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K) {
    int64_t NB = rows * (K / QK);
    uint8_t *pa = dst, *pb = dst + 128 * NB, *psc = dst + 192 * NB, *pd = dst + 208 * NB;
    int8_t q[QK], sc[16];
    double d;
    for (int64_t t = 0; t < NB; t++) {
        const uint8_t *blk = src + t * Q6K_BYTES;
        orc_q6k_decode(blk, q, sc, &d);
        for (int j = 0; j < 8; j++) {
            int v[32];
            for (int i = 0; i < 32; i++) v[i] = (q[32 * j + i] + 32) ^ 32; /* (q6-32) mod 64 */
            uint8_t a[16], b[8];
            for (int k = 0; k < 16; k++) a[k] = (uint8_t)(v[k] << 2);
            for (int k = 0; k < 8; k++) b[k] = (uint8_t)(v[16 + k] << 2);
            for (int k = 0; k < 4; k++) {
                int w24 = v[24 + k], w28 = v[28 + k];
                a[k] |= w24 & 3;
                a[4 + k] |= (w24 >> 2) & 3;
                a[8 + k] |= (w24 >> 4) & 3;
                a[12 + k] |= w28 & 3;
                b[k] |= (w28 >> 2) & 3;
                b[4 + k] |= (w28 >> 4) & 3;
            }
            memcpy(pa + t * 128 + 16 * j, a, 16);
            memcpy(pb + t * 64 + 8 * j, b, 8);
        }
        memcpy(psc + t * 16, blk + 192, 16);
        memcpy(pd + t * 2, blk + 208, 2);
    }
}

/* -------------------------------------------------------- tiled Q6_K
 * The planar planes above with each group of 16 consecutive rows
 * interleaved, so that the entries of one position of the 16 rows are
 * adjacent (the same load-time conversion of P2340 "What it changes", laid
 * out for a 16-row operand).  Restated from the GPU library's published
 * layout text (its C header): rows form tiles 16T .. 16T+R_T-1 with
 * R_T = min(16, rows - 16T); for row r of tile T, nsb = K/32, nb = K/256:
 *   A entry (16 B) of sub-block s:  16*T*nsb + s*R_T + r
 *   B entry (8 B) of sub-block s:   16*T*nsb + s*R_T + r
 *   SC entry (8 B) of step z (scale bytes 8*(z%2).. of block z/2):
 *                                   16*T*(nsb/4) + z*R_T + r
 *   D entry (2 B) of block b:       16*T*nb + b*R_T + r
 * with the planes at the planar layout's byte offsets. */
void orc_q6k_to_tiled(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K) {
    const int64_t nb = K / QK, nsb = K / 32, NB = rows * nb;
    uint8_t *pl = (uint8_t *)malloc((size_t)(210 * NB));
    if (!pl) abort();
    orc_q6k_to_planar(src, pl, rows, K);
    for (int64_t row = 0; row < rows; row++) {
        const int64_t T = row / 16, r = row % 16;
        const int64_t R = rows - 16 * T < 16 ? rows - 16 * T : 16;
        for (int64_t s = 0; s < nsb; s++) {
            const int64_t e = 16 * T * nsb + s * R + r, p = row * nsb + s;
            memcpy(dst + 16 * e, pl + 16 * p, 16);
            memcpy(dst + 128 * NB + 8 * e, pl + 128 * NB + 8 * p, 8);
        }
        for (int64_t z = 0; z < nsb / 4; z++) {
            const int64_t e = 16 * T * (nsb / 4) + z * R + r;
            memcpy(dst + 192 * NB + 8 * e, pl + 192 * NB + 16 * (row * nb + z / 2) + 8 * (z % 2), 8);
        }
        for (int64_t b = 0; b < nb; b++) {
            const int64_t e = 16 * T * nb + b * R + r;
            memcpy(dst + 208 * NB + 2 * e, pl + 208 * NB + 2 * (row * nb + b), 2);
        }
    }
    free(pl);
}

/* ------------------------------------------- column-planar Q8_1
 * The Q8_1 blocks of each activation column rearranged inside the column
 * (the int4 activation loads of P2340 "What it changes", laid out so that a
 * column's quants are one aligned run).  Restated from the GPU library's
 * published layout text (its C header): with nb = K/32 and column n at byte
 * 36*nb*n in both forms, block b's quants go to byte 32*b of the column,
 * its fp16 d to byte K + 2*b and its fp16 s to byte K + 2*nb + 2*b. */
void orc_q8_1_to_planar(const uint8_t *src, uint8_t *dst, int64_t K, int ncols) {
    const int64_t nb = K / QB;
    for (int64_t n = 0; n < ncols; n++) {
        const uint8_t *cs = src + n * nb * Q81_BYTES;
        uint8_t *cd = dst + n * nb * Q81_BYTES;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = cs + b * Q81_BYTES;
            memcpy(cd + 32 * b, blk + 4, 32);
            memcpy(cd + K + 2 * b, blk, 2);
            memcpy(cd + K + 2 * nb + 2 * b, blk + 2, 2);
        }
    }
}

/* ----------------------------------------------------------- row gather
 * Row subset of a converted matrix (the draft head gathered from the planar
 * LM head, P2340 "What it changes"): output row j is source row ids[j], in
 * the same layout (0 GGUF, 1 planar, 2 tiled); an id outside [0, rows)
 * gives a row whose bytes are all zero in that layout.  Computed from the
 * GGUF source: gather the GGUF rows, convert, then clear the entries of the
 * rows with a bad id (positions as in the layout text above). */
static void orc_zero_row(uint8_t *dst, int layout, int64_t rows, int64_t K, int64_t row) {
    const int64_t nb = K / QK, nsb = K / 32, NB = rows * nb;
    if (layout == 0) {
        memset(dst + row * nb * Q6K_BYTES, 0, (size_t)(nb * Q6K_BYTES));
        return;
    }
    const int64_t T = row / 16, r = row % 16, R = layout == 2 ? (rows - 16 * T < 16 ? rows - 16 * T : 16) : 0;
    for (int64_t s = 0; s < nsb; s++) {
        const int64_t e = layout == 2 ? 16 * T * nsb + s * R + r : row * nsb + s;
        memset(dst + 16 * e, 0, 16);
        memset(dst + 128 * NB + 8 * e, 0, 8);
    }
    for (int64_t z = 0; z < nsb / 4; z++) {
        const int64_t e = layout == 2 ? 16 * T * (nsb / 4) + z * R + r : row * (nsb / 4) + z;
        memset(dst + 192 * NB + 8 * e, 0, 8);
    }
    for (int64_t b = 0; b < nb; b++) {
        const int64_t e = layout == 2 ? 16 * T * nb + b * R + r : row * nb + b;
        memset(dst + 208 * NB + 2 * e, 0, 2);
    }
}

void orc_q6k_gather(const uint8_t *src, int layout, int64_t rows, int64_t K, const int32_t *ids, int64_t nout,
                    uint8_t *dst) {
    const int64_t rb = K / QK * Q6K_BYTES;
    uint8_t *g = (uint8_t *)malloc((size_t)(rb * nout));
    if (!g) abort();
    for (int64_t j = 0; j < nout; j++) {
        if (ids[j] >= 0 && ids[j] < rows) memcpy(g + j * rb, src + (int64_t)ids[j] * rb, (size_t)rb);
        else memset(g + j * rb, 0, (size_t)rb);
    }
    if (layout == 1) orc_q6k_to_planar(g, dst, nout, K);
    else if (layout == 2) orc_q6k_to_tiled(g, dst, nout, K);
    else memcpy(dst, g, (size_t)(rb * nout));
    for (int64_t j = 0; j < nout; j++)
        if (!(ids[j] >= 0 && ids[j] < rows)) orc_zero_row(dst, layout, nout, K, j);
    free(g);
}

/* ------------------------------------------------------ grouped MoE
 * Routed-expert chain over a window of T tokens [I2801; P2746 "B70
 * validation"], for each token t and slot k (slot index t*topk + k):
 *   e = ids[t][k];
 *   g = MMVQ_Q4K(gate_e, xq_t), u = MMVQ_Q4K(up_e, xq_t)      (fp64, d_ff)
 *   h = fp32(silu(g) * u), silu(g) = g / (1 + exp(-g)) in fp64
 *   hq = quantize_q8_1(h)                                      (d_ff/32 blocks)
 *   y = MMVQ_Q6K(down_e, hq)                                   (fp64, d_model)
 *   out[t] = sum_{k ascending} route_w[t][k] * y_tk            (fp64)
 * Weights: gate/up Q4_K [E][d_ff][d_model/256], down Q6_K (GGUF)
 * [E][d_model][d_ff/256]; xq Q8_1 [T][d_model/32].
 * If hq_in is non-NULL the down product uses hq_in (slot-major,
 * [T*topk][d_ff/32] blocks) instead of this function's own hq; this is the
 * staged comparison against a GPU's own requantized hidden state.
 * Optional outputs (any may be NULL): g, u [T*topk][d_ff] fp64; h fp32;
 * hq; y [T*topk][d_model] fp64 and its absum; out [T][d_model] fp64 and
 * out_absum = sum_k |w_tk| * absum(y_tk).
 * Returns 0, or -1 when an id is out of [0, E).
 */
int orc_grouped_expert(const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                       const uint8_t *xq, const int32_t *ids, const float *route_w,
                       int E, int T, int topk, int64_t d_model, int64_t d_ff,
                       const uint8_t *hq_in,
                       double *g_out, double *u_out, float *h_out, uint8_t *hq_out,
                       double *y_out, double *y_absum, double *out, double *out_absum) {
    int64_t gu_bytes = d_ff * (d_model / QK) * Q4K_BYTES;      /* per expert */
    int64_t dn_bytes = d_model * (d_ff / QK) * Q6K_BYTES;
    int64_t xq_row = (d_model / QB) * Q81_BYTES, hq_row = (d_ff / QB) * Q81_BYTES;
    double *g = malloc(sizeof(double) * d_ff), *u = malloc(sizeof(double) * d_ff);
    float *h = malloc(sizeof(float) * d_ff);
    uint8_t *hq = malloc(hq_row);
    double *y = malloc(sizeof(double) * d_model), *ya = malloc(sizeof(double) * d_model);
    int rc = 0;
    for (int t = 0; t < T; t++) {
        if (out)
            for (int64_t i = 0; i < d_model; i++) out[t * d_model + i] = 0.0;
        if (out_absum)
            for (int64_t i = 0; i < d_model; i++) out_absum[t * d_model + i] = 0.0;
        for (int k = 0; k < topk; k++) {
            int slot = t * topk + k;
            int e = ids[slot];
            if (e < 0 || e >= E) { rc = -1; goto done; }
            orc_mmvq_q4k(w_gate + e * gu_bytes, xq + t * xq_row, g, NULL, d_ff, d_model, 1, 0, d_ff);
            orc_mmvq_q4k(w_up + e * gu_bytes, xq + t * xq_row, u, NULL, d_ff, d_model, 1, 0, d_ff);
            for (int64_t i = 0; i < d_ff; i++) {
                double silu = g[i] / (1.0 + exp(-g[i]));
                h[i] = (float)(silu * u[i]);
            }
            orc_quantize_q8_1(h, hq, d_ff, 1);
            const uint8_t *hq_use = hq_in ? hq_in + slot * hq_row : hq;
            orc_mmvq_q6k(w_down + e * dn_bytes, hq_use, y, ya, d_model, d_ff, 1, 0, d_model);
            double wt = (double)route_w[slot];
            for (int64_t i = 0; i < d_model; i++) {
                if (out) out[t * d_model + i] += wt * y[i];
                if (out_absum) out_absum[t * d_model + i] += fabs(wt) * ya[i];
            }
            if (g_out) memcpy(g_out + slot * d_ff, g, sizeof(double) * d_ff);
            if (u_out) memcpy(u_out + slot * d_ff, u, sizeof(double) * d_ff);
            if (h_out) memcpy(h_out + slot * d_ff, h, sizeof(float) * d_ff);
            if (hq_out) memcpy(hq_out + slot * hq_row, hq, hq_row);
            if (y_out) memcpy(y_out + slot * d_model, y, sizeof(double) * d_model);
            if (y_absum) memcpy(y_absum + slot * d_model, ya, sizeof(double) * d_model);
        }
    }
done:
    free(g); free(u); free(h); free(hq); free(y); free(ya);
    return rc;
}
