/*
 * sage_oracle.c -- plain, slow, step-by-step CPU reference for SageAttention-
 * style quantized attention.  TEST INFRASTRUCTURE ONLY (see sage_oracle.h):
 * nothing in the product path may load or call it.
 *
 * Each function follows one step of the method in the order the pages give it;
 * there is no tiling, fusion or reordering beyond what the method itself
 * states.  The one blocking that IS part of the method -- FlashAttention-style
 * key blocks with an online softmax [SA2, 相关工作] -- is kept, because the
 * FP8 quantisation of P~ is taken relative to the running maximum.
 *
 * Build: gcc -O2 -std=c99 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include "sage_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of OpenMP threads the parallel loops below use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ===================================================================== */
/* Number formats                                                         */
/* ===================================================================== */

/*
 * Nearest value, ties to even, of a binary floating-point format that has
 * `mbits` stored fraction bits and smallest normal exponent `emin` (values
 * below 2^emin are subnormal with the fixed quantum 2^(emin-mbits)).
 * `a` must be finite and >= 0.  Exponent range at the top is NOT limited here;
 * the callers handle overflow.  All arithmetic is exact in binary64 (a / q and
 * m * q only shift exponents), so the single rounding is nearbyint's, which is
 * round-half-to-even in the default rounding mode.
 */
static double round_to_format(double a, int mbits, int emin) {
    if (a == 0.0) return 0.0;
    int e = ilogb(a);
    if (e < emin) e = emin;
    double q = ldexp(1.0, e - mbits);
    return nearbyint(a / q) * q;
}

/* IEEE binary16: 5 exponent bits (bias 15), 10 fraction bits. */
static float f16_bits_to_float(uint16_t h) {
    int sign = h >> 15, ex = (h >> 10) & 31, fr = h & 1023;
    double v;
    if (ex == 31) v = fr ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)fr, -24);
    else v = ldexp(1.0 + fr / 1024.0, ex - 15);
    return (float)(sign ? -v : v);
}

static uint16_t float_to_f16_bits(float x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double v = round_to_format(fabs((double)x), 10, -14);
    if (v >= 65536.0) return sign | 0x7c00; /* overflow -> inf */
    if (v < ldexp(1.0, -14)) return sign | (uint16_t)(v / ldexp(1.0, -24));
    int e = ilogb(v);
    uint16_t fr = (uint16_t)(ldexp(v, -e) * 1024.0 - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | fr;
}

/* bfloat16: the upper half of an IEEE binary32 (8 exponent bits, 7 fraction bits). */
static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t float_to_bf16_bits(float x) {
    if (isnan(x)) return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double v = round_to_format(fabs((double)x), 7, -126);
    if (v >= ldexp(1.0, 128)) return sign | 0x7f80;
    if (v < ldexp(1.0, -126)) return sign | (uint16_t)(v / ldexp(1.0, -133));
    int e = ilogb(v);
    uint16_t fr = (uint16_t)(ldexp(v, -e) * 128.0 - 128.0);
    return sign | (uint16_t)((e + 127) << 7) | fr;
}

void orc_decode16(const uint16_t *x, size_t n, int dtype, float *out) {
    for (size_t i = 0; i < n; ++i)
        out[i] = dtype == ORC_BF16 ? bf16_bits_to_float(x[i]) : f16_bits_to_float(x[i]);
}

void orc_encode16(const float *x, size_t n, int dtype, uint16_t *out) {
    for (size_t i = 0; i < n; ++i)
        out[i] = dtype == ORC_BF16 ? float_to_bf16_bits(x[i]) : float_to_f16_bits(x[i]);
}

/* fp32 -> nearest fp16 value, returned as fp32 (used for P and V in pv fp16 mode). */
static float round_f16(float x) { return f16_bits_to_float(float_to_f16_bits(x)); }

/*
 * FP8 E4M3 as in [OCP] "E4M3FN": 1 sign bit, 4 exponent bits (bias 7), 3
 * fraction bits; exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN;
 * there is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448.
 * [SA2, SageAttention2方法] names E4M3 for P~ and V.
 */
float orc_e4m3_decode(uint8_t c) {
    int sign = c >> 7, ex = (c >> 3) & 15, fr = c & 7;
    if (ex == 15 && fr == 7) return NAN;
    double v = ex == 0 ? ldexp((double)fr, -9) : ldexp(1.0 + fr / 8.0, ex - 7);
    return (float)(sign ? -v : v);
}

/* Round to nearest, ties to even; magnitudes beyond 448 saturate to 448. */
uint8_t orc_e4m3_encode(float x) {
    if (isnan(x)) return 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double v = round_to_format(fabs((double)x), 3, -6);
    if (v >= 448.0) return sign | 0x7e; /* 0x7e = 1.75 * 2^8 */
    if (v < ldexp(1.0, -6)) return sign | (uint8_t)(v / ldexp(1.0, -9));
    int e = ilogb(v);
    uint8_t fr = (uint8_t)(ldexp(v, -e) * 8.0 - 8.0);
    return sign | (uint8_t)((e + 7) << 3) | fr;
}

void orc_e4m3_encode_n(const float *x, size_t n, uint8_t *out) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

/*
 * FP4 E2M1 as in [OCP-MX] (the element format of MXFP4): 1 sign bit, 2 exponent
 * bits (bias 1), 1 fraction bit; exponent field 0 holds the subnormal 0.5; no
 * infinity or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Encoding rounds to
 * nearest, ties to even, saturates at 6; the sign bit is set iff x < 0.
 */
float orc_e2m1_decode(uint8_t c) {
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    return (c & 8) ? -mag[c & 7] : mag[c & 7];
}

uint8_t orc_e2m1_encode(float x) {
    uint8_t sign = x < 0.0f ? 8 : 0;
    double v = round_to_format(fabs((double)x), 1, 0);
    if (v >= 6.0) return sign | 7;
    if (v < 1.0) return sign | (uint8_t)(v / 0.5); /* 0 or the subnormal 0.5 */
    int e = ilogb(v);
    uint8_t fr = (uint8_t)(ldexp(v, -e) * 2.0 - 2.0);
    return sign | (uint8_t)((e + 1) << 1) | fr;
}

/* ===================================================================== */
/* Quantisation                                                           */
/* ===================================================================== */

/*
 * Symmetric INT8 quantisation of one block with one fp32 scale
 * ([KAI, 2.2] per-block INT8 for QK^T; [SA2, 相关工作] Q and K to INT8).
 * Reading of the unstated details: range +-127, scale = amax / 127,
 * code = round-half-even(x * (127 / amax)), an all-zero block gets scale 0 and
 * codes 0.  Every step is one correctly rounded fp32 operation.
 */
void orc_int8_quant_block(const float *x, size_t n, int8_t *codes, float *scale) {
    float amax = 0.0f;
    for (size_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale = 0.0f;
        memset(codes, 0, n);
        return;
    }
    float inv = 127.0f / amax;
    *scale = amax / 127.0f;
    for (size_t i = 0; i < n; ++i) {
        float t = rintf(x[i] * inv);
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        codes[i] = (int8_t)t;
    }
}

/*
 * K smoothing statistic: the mean of each channel over all S tokens of the
 * head ([SA2, 相关工作] K is pre-processed; [SA2, SageAttention2方法] K smoothing).
 * Sum in binary64 over tokens in order, divide by S in binary64, round once
 * to fp32.  A head with no tokens (an empty sequence of a packed batch) has
 * mean 0.
 */
void orc_channel_mean(const float *x, int S, int D, float *mean) {
    for (int d = 0; d < D; ++d) {
        double s = 0.0;
        for (int t = 0; t < S; ++t) s += (double)x[(size_t)t * D + d];
        mean[d] = S > 0 ? (float)(s / (double)S) : 0.0f;
    }
}

/* Q: INT8 blocks of `blk` consecutive tokens (all D channels share a scale). */
void orc_quant_q_head(const float *q, int S, int D, int blk, int8_t *codes, float *scales) {
    int nb = (S + blk - 1) / blk;
#pragma omp parallel for schedule(static)
    for (int b = 0; b < nb; ++b) {
        int r0 = b * blk, r1 = r0 + blk < S ? r0 + blk : S;
        size_t off = (size_t)r0 * D;
        orc_int8_quant_block(q + off, (size_t)(r1 - r0) * D, codes + off, &scales[b]);
    }
}

/*
 * K: optionally subtract the channel mean (one fp32 subtraction per element),
 * then INT8 blocks of `blk` tokens.  `mean` receives the channel means (zeros
 * when smooth == 0).
 */
void orc_quant_k_head(const float *k, int S, int D, int blk, int smooth, int8_t *codes,
                      float *scales, float *mean) {
    size_t n = (size_t)S * D;
    float *ks = (float *)malloc(n * sizeof(float));
    if (smooth) orc_channel_mean(k, S, D, mean);
    else memset(mean, 0, (size_t)D * sizeof(float));
    for (size_t i = 0; i < n; ++i) ks[i] = k[i] - mean[i % D];
    orc_quant_q_head(ks, S, D, blk, codes, scales);
    free(ks);
}

/*
 * Thread-level granularity ([SA2, SageAttention2方法]: quantise at the
 * granularity of the GPU threads' share of the matrix-multiply layout, so that
 * dequantisation costs nothing extra).  On the 32 x 32 INT8 matrix core of
 * gfx950 the score tile of 32 keys x 32 queries leaves each lane one query and
 * 16 keys: the keys whose offset in the 32-key sub-tile has bit 2 equal to the
 * lane's half of the wavefront.  Reading: Q gets one scale per token and K one
 * scale per such 16-key group; group of key n = 2 * (n / 32) + bit 2 of n.
 */
int orc_lane_group(int n) { return 2 * (n >> 5) + ((n >> 2) & 1); }

/*
 * Smoothed Q ([SA2, SageAttention2方法]: subtract the mean of each block of Q;
 * together with K smoothing the product splits into a pre-processing stage and
 * the attention stage).  Reading: the block is the INT8 scale block of `blk`
 * tokens; its channel means are summed in binary64 over the block's tokens,
 * divided by their number and rounded once to fp32; the block's values minus
 * its means (one fp32 subtraction each) are quantised by orc_quant_q_head's
 * rule with the same blocks (or per token, blk_scale = 1).  qmean: [nb][D].
 */
void orc_quant_q_head_smooth(const float *q, int S, int D, int blk, int blk_scale, int8_t *codes,
                             float *scales, float *qmean) {
    size_t n = (size_t)S * D;
    int nb = (S + blk - 1) / blk;
    float *qs = (float *)malloc((n ? n : 1) * sizeof(float));
    for (int b = 0; b < nb; ++b) {
        int r0 = b * blk, r1 = r0 + blk < S ? r0 + blk : S;
        orc_channel_mean(q + (size_t)r0 * D, r1 - r0, D, qmean + (size_t)b * D);
        for (int t = r0; t < r1; ++t)
            for (int d = 0; d < D; ++d) qs[(size_t)t * D + d] = q[(size_t)t * D + d] - qmean[(size_t)b * D + d];
    }
    orc_quant_q_head(qs, S, D, blk_scale, codes, scales);
    free(qs);
}

/*
 * The pre-processing stage of smoothed Q: delta[b][n] = fp32( sum_d qmean[b][d] * kc[n][d] )
 * in binary64, kc = K minus its channel mean kmean (one fp32 subtraction per element,
 * as orc_quant_k_head forms it).  The attention adds delta[query block][n] * sm_scale
 * to the dequantised score.
 */
void orc_qk_delta_head(const float *qmean, int nb, const float *k, const float *kmean, int S, int D,
                       float *delta) {
    size_t n = (size_t)S * D;
    float *kc = (float *)malloc((n ? n : 1) * sizeof(float));
    for (size_t i = 0; i < n; ++i) kc[i] = k[i] - kmean[i % D];
#pragma omp parallel for schedule(static)
    for (int b = 0; b < nb; ++b)
        for (int t = 0; t < S; ++t) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += (double)qmean[(size_t)b * D + d] * (double)kc[(size_t)t * D + d];
            delta[(size_t)b * S + t] = (float)acc;
        }
    free(kc);
}

/*
 * K with thread-level granularity: optional mean subtraction as in
 * orc_quant_k_head, then one INT8 scale per key group of orc_lane_group
 * (2 * ceil(S / 32) groups; a group without keys gets scale 0).
 */
void orc_quant_k_head_lane(const float *k, int S, int D, int smooth, int8_t *codes,
                           float *scales, float *mean) {
    size_t n = (size_t)S * D;
    int ng = 2 * ((S + 31) / 32);
    float *ks = (float *)malloc((n ? n : 1) * sizeof(float));
    float *grp = (float *)malloc((size_t)16 * D * sizeof(float));
    int8_t *gc = (int8_t *)malloc((size_t)16 * D);
    int *rows = (int *)malloc(16 * sizeof(int));
    if (smooth) orc_channel_mean(k, S, D, mean);
    else memset(mean, 0, (size_t)D * sizeof(float));
    for (size_t i = 0; i < n; ++i) ks[i] = k[i] - mean[i % D];
    for (int g = 0; g < ng; ++g) {
        int cnt = 0;
        for (int t = 32 * (g / 2); t < S && t < 32 * (g / 2 + 1); ++t)
            if (orc_lane_group(t) == g) rows[cnt++] = t;
        for (int r = 0; r < cnt; ++r) memcpy(grp + (size_t)r * D, ks + (size_t)rows[r] * D, (size_t)D * sizeof(float));
        orc_int8_quant_block(grp, (size_t)cnt * D, gc, &scales[g]);
        for (int r = 0; r < cnt; ++r) memcpy(codes + (size_t)rows[r] * D, gc + (size_t)r * D, (size_t)D);
    }
    free(ks);
    free(grp);
    free(gc);
    free(rows);
}

/*
 * V: per-channel FP8 E4M3 ([SA2, SageAttention2方法]: V to FP8 with per-channel
 * quantisation).  scale[d] = amax_d / 448, code = E4M3(v * (448 / amax_d));
 * an all-zero channel gets scale 0 and codes 0.
 */
void orc_quant_v_head(const float *v, int S, int D, uint8_t *codes, float *scales) {
    for (int d = 0; d < D; ++d) {
        float amax = 0.0f;
        for (int t = 0; t < S; ++t) {
            float a = fabsf(v[(size_t)t * D + d]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            scales[d] = 0.0f;
            for (int t = 0; t < S; ++t) codes[(size_t)t * D + d] = 0;
            continue;
        }
        float inv = 448.0f / amax;
        scales[d] = amax / 448.0f;
        for (int t = 0; t < S; ++t)
            codes[(size_t)t * D + d] = orc_e4m3_encode(v[(size_t)t * D + d] * inv);
    }
}

/*
 * MX micro-scaled FP4 ("Kairos" guide 2.2 and the full guide's 下一步 section:
 * FP4 micro-scaled attention; scale rule of [OCP-MX]): each block of 32
 * consecutive channels of a token shares an E8M0 scale 2^e,
 *   e = floor(log2(amax)) - 2        (2 = the largest exponent of E2M1),
 * clamped to [-127, 127] (an all-zero block gets -127); the elements are
 * E2M1(x / 2^e), which saturates the few values in (6, 8) * 2^e to 6 * 2^e.
 * codes: one E2M1 code per element (low 4 bits); e8m0: e + 127 per block.
 */
static int mx_shared_exp(float amax) {
    int e = -127;
    if (amax > 0.0f) {
        int fe;
        frexp((double)amax, &fe); /* amax = m * 2^fe, m in [0.5, 1): floor(log2) = fe - 1 */
        e = fe - 1 - 2;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    return e;
}

void orc_mxfp4_quant_rows(const float *x, int S, int D, uint8_t *codes, uint8_t *e8m0) {
    int nb = D / 32;
    for (int t = 0; t < S; ++t)
        for (int b = 0; b < nb; ++b) {
            const float *xb = x + (size_t)t * D + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(xb[i]) > amax) amax = fabsf(xb[i]);
            int e = mx_shared_exp(amax);
            e8m0[(size_t)t * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i)
                codes[(size_t)t * D + 32 * b + i] = orc_e2m1_encode((float)ldexp((double)xb[i], -e));
        }
}

/* K for the FP4 product: optional mean subtraction as in orc_quant_k_head, then MXFP4. */
void orc_quant_k_head_mxfp4(const float *k, int S, int D, int smooth, uint8_t *codes, uint8_t *e8m0,
                            float *mean) {
    size_t n = (size_t)S * D;
    float *ks = (float *)malloc((n ? n : 1) * sizeof(float));
    if (smooth) orc_channel_mean(k, S, D, mean);
    else memset(mean, 0, (size_t)D * sizeof(float));
    for (size_t i = 0; i < n; ++i) ks[i] = k[i] - mean[i % D];
    orc_mxfp4_quant_rows(ks, S, D, codes, e8m0);
    free(ks);
}

/*
 * Smoothed Q for the FP4 product: the block means of orc_quant_q_head_smooth
 * (blocks of `blk` tokens) are subtracted, one fp32 subtraction per element,
 * and the result is quantised by the MXFP4 rule of orc_mxfp4_quant_rows.
 */
void orc_quant_q_head_mxfp4_smooth(const float *q, int S, int D, int blk, uint8_t *codes, uint8_t *e8m0,
                                   float *qmean) {
    size_t n = (size_t)S * D;
    int nb = (S + blk - 1) / blk;
    float *qs = (float *)malloc((n ? n : 1) * sizeof(float));
    for (int b = 0; b < nb; ++b) {
        int r0 = b * blk, r1 = r0 + blk < S ? r0 + blk : S;
        orc_channel_mean(q + (size_t)r0 * D, r1 - r0, D, qmean + (size_t)b * D);
        for (int t = r0; t < r1; ++t)
            for (int d = 0; d < D; ++d) qs[(size_t)t * D + d] = q[(size_t)t * D + d] - qmean[(size_t)b * D + d];
    }
    orc_mxfp4_quant_rows(qs, S, D, codes, e8m0);
    free(qs);
}

/*
 * Key groups of the micro-scaled FP4 P~ V product.  The FP4 micro-scaling
 * ([KAI, 2.2]; the full guide's 性能调优实战 section) shares one scale per 32
 * elements along the contraction, which for P~ V runs over keys.  Reading: the
 * 32 keys are those one lane of gfx950's 32 x 32 x 64 matrix core holds of a
 * 64-key block -- the keys whose offset has bit 2 equal to the lane's half of
 * the wavefront (the score layout of the Q K^T product leaves each lane exactly
 * these) -- so group of key n = 2 * (n / 64) + bit 2 of n.
 */
int orc_pv_group(int n) { return 2 * (n >> 6) + ((n >> 2) & 1); }

/*
 * V for the FP4 P~ V product: optionally minus its channel mean (as
 * orc_quant_v_head_smooth), then MXFP4 along the keys: each channel of each
 * key group of orc_pv_group shares an E8M0 scale from the group's largest
 * magnitude (the rule of orc_mxfp4_quant_rows); keys past S count as 0.
 * codes [S][D] (one E2M1 code per byte), e8m0 [2 ceil(S / 64)][D], mean [D].
 */
void orc_quant_v_head_mxfp4(const float *v, int S, int D, int smooth, uint8_t *codes, uint8_t *e8m0,
                            float *mean) {
    size_t n = (size_t)S * D;
    int ng = 2 * ((S + 63) / 64);
    float *vs = (float *)malloc((n ? n : 1) * sizeof(float));
    if (smooth) orc_channel_mean(v, S, D, mean);
    else memset(mean, 0, (size_t)D * sizeof(float));
    for (size_t i = 0; i < n; ++i) vs[i] = v[i] - mean[i % D];
    for (int g = 0; g < ng; ++g)
        for (int d = 0; d < D; ++d) {
            float amax = 0.0f;
            for (int t = 64 * (g / 2); t < S && t < 64 * (g / 2 + 1); ++t)
                if (orc_pv_group(t) == g && fabsf(vs[(size_t)t * D + d]) > amax) amax = fabsf(vs[(size_t)t * D + d]);
            int e = mx_shared_exp(amax);
            e8m0[(size_t)g * D + d] = (uint8_t)(e + 127);
            for (int t = 64 * (g / 2); t < S && t < 64 * (g / 2 + 1); ++t)
                if (orc_pv_group(t) == g)
                    codes[(size_t)t * D + d] = orc_e2m1_encode((float)ldexp((double)vs[(size_t)t * D + d], -e));
        }
    free(vs);
}

/*
 * Q K^T of MXFP4 rows: out[r][n] = fp32( sum_d dec(q[rows[r]][d]) dec(k[n][d]) ), with
 * dec(x) = E2M1 value * 2^(e8m0 - 127) of x's block.  Every product is exact and
 * the sum is exact in binary64, so the only rounding is the final one to fp32.
 */
void orc_qk_mxfp4_rows(const uint8_t *q4, const uint8_t *qe, const uint8_t *k4, const uint8_t *ke, int S,
                       int D, const int *rows, int nrows, float *out) {
    int nb = D / 32;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < nrows; ++r) {
        int i = rows[r];
        for (int n = 0; n < S; ++n) {
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                double blk = 0.0;
                for (int d = 32 * b; d < 32 * b + 32; ++d)
                    blk += (double)orc_e2m1_decode(q4[(size_t)i * D + d]) * (double)orc_e2m1_decode(k4[(size_t)n * D + d]);
                acc += ldexp(blk, (int)qe[(size_t)i * nb + b] - 127 + (int)ke[(size_t)n * nb + b] - 127);
            }
            out[(size_t)r * S + n] = (float)acc;
        }
    }
}

/*
 * Smoothed V ([SA2, SageAttention2方法]: an optional V smoothing for the FP8 PV
 * product).  Reading: the same statistic as K smoothing -- the channel mean of V
 * over the head's S tokens (orc_channel_mean) -- is subtracted, one fp32
 * subtraction per element, and the result quantised per channel as above; the
 * attention adds the mean back after normalising (softmax weights sum to 1).
 */
void orc_quant_v_head_smooth(const float *v, int S, int D, uint8_t *codes, float *scales, float *mean) {
    size_t n = (size_t)S * D;
    float *vs = (float *)malloc((n ? n : 1) * sizeof(float));
    orc_channel_mean(v, S, D, mean);
    for (size_t i = 0; i < n; ++i) vs[i] = v[i] - mean[i % D];
    orc_quant_v_head(vs, S, D, codes, scales);
    free(vs);
}

/* ===================================================================== */
/* Attention                                                              */
/* ===================================================================== */

static int32_t dot_i8(const int8_t *a, const int8_t *b, int D) {
    int32_t s = 0;
    for (int d = 0; d < D; ++d) s += (int32_t)a[d] * (int32_t)b[d];
    return s;
}

/* Integer Q K^T of one head: out[i][n] = sum_d q8[i][d] * k8[n][d] (exact). */
void orc_qk_int32_head(const int8_t *q8, const int8_t *k8, int S, int D, int32_t *out) {
#pragma omp parallel for schedule(static)
    for (int i = 0; i < S; ++i)
        for (int n = 0; n < S; ++n)
            out[(size_t)i * S + n] = dot_i8(q8 + (size_t)i * D, k8 + (size_t)n * D, D);
}

/*
 * Quantized attention for selected query rows of one head over its S keys
 * (query rows index q8; the number of query rows may differ from S).
 *
 * Key tiles of `tile_k` tokens are visited in order with an online softmax
 * whose running max m and running sum l are fp32 ([SA2, 相关工作]: token-dim
 * blocking of FlashAttention; SageAttention builds on that blocking).  The tile
 * size is a free parameter of that blocking; it is independent of the INT8
 * scale blocks of K (`blk_k` tokens each, key n uses k_scale[n / blk_k]; with
 * k_lane, key n uses k_scale[orc_lane_group(n)]).  Query i uses q_scale[i / blk_q].
 * Per key tile:
 *   s_n   = float(q8_i . k8_n) * ((dq_i * dk_blk(n)) * sm_scale)     (dequantise)
 *           or, with the FP4 product (qk != NULL): s_n = qk[r][n] * sm_scale, qk from
 *           orc_qk_mxfp4_rows (already dequantised by the micro-scales);
 *           smoothed Q (delta != NULL): s_n += delta[i / blk_d][n] * sm_scale (blk_d: the
 *           tokens of a Q smoothing block)
 *   s_n   = -inf for keys n >= S, and for n > i when causal ([GUIDE, 性能调优实战] is_causal;
 *           key n and query i count from the start of their sequences)
 *   m'    = max(m, max_n s_n);  alpha = exp(m - m') (0 on the first tile)
 *   p_n   = exp(s_n - m')                                            (fp32)
 *   P_n   = p_n rounded to the format of the P~ V product (below)
 *   l     = alpha * l + sum_n P_n     (tile sum in binary64, rounded once to fp32)
 * The softmax denominator sums the same rounded weights P_n that multiply V, so
 * the normalised weights sum to one (the pages fix the fp32 online softmax and
 * the P~ quantisation, not which of the two values the row sum adds up).
 * pv fp8 ([SA2, SageAttention2方法]: P~ to E4M3 with a static scale, V per channel;
 *         FP32 buffer for the two-level accumulation):
 *   P_n   = dec(E4M3(p_n * 448))            (static scale 1/448: p = 1 -> 448)
 *   inner = sum_n P_n * dec(v8_n,d)         (fresh per key tile, rounded once to fp32)
 *   O_d   = alpha * O_d + inner_d                                    (fp32 buffer)
 *   out   = O_d * (dv_d / l)  (+ v_mean_d when V was smoothed, v_mean != NULL)
 * pv fp16 ([KAI, 2.1] sm80 row: INT8 QK^T, FP16 PV, fp32 accumulation):
 *   P_n   = fp16(p_n), V in fp16 (bf16 inputs rounded to fp16),
 *   O_d   = alpha * O_d + sum_n P_n * V_n,d;   out = O_d / l
 * pv fp4 (micro-scaled FP4 P~ V, [KAI, 2.2]; [GUIDE, 性能调优实战] FP4 micro-scaling):
 *   the tile's keys fall into the 32-key groups of orc_pv_group; a group's p_n
 *   share the E8M0 scale 2^e of its largest p_n (the MXFP4 rule), and
 *   P_n   = dec(E2M1(p_n / 2^e)) * 2^e;  V from orc_quant_v_head_mxfp4 (`v8` holds
 *   its E2M1 codes, `v_e8m0` its scales), dec(v)_n,d = dec(E2M1) * 2^(e8m0 - 127),
 *   inner and O as in pv fp8;  out = O_d / l  (+ v_mean_d).  tile_k must be a
 *   multiple of 64 so that no group spans two tiles.
 * `v` (fp32 values of the original V) is read only in pv fp16 mode; `v8` in pv
 * fp8 and fp4 modes, `v_scale` in pv fp8 mode, `v_e8m0` in pv fp4 mode.  out is
 * [nrows][D] fp32 (before the final rounding to the input dtype).  A row that
 * sees no key at all (S = 0) is 0.
 */
void orc_attn_head_rows(const int8_t *q8, const float *q_scale, int blk_q,
                        const int8_t *k8, const float *k_scale, int blk_k, int k_lane, int tile_k,
                        const uint8_t *v8, const float *v_scale, const uint8_t *v_e8m0, const float *v_mean,
                        const float *v, int in_dtype, int S, int D, int is_causal, float sm_scale,
                        int pv_mode, const int *rows, int nrows, const float *qk, const float *delta,
                        int blk_d, float *out) {
    int ntile = (S + tile_k - 1) / tile_k;
#pragma omp parallel
    {
        float *s = (float *)malloc((size_t)tile_k * sizeof(float));
        float *p = (float *)malloc((size_t)tile_k * sizeof(float));
        float *pq = (float *)malloc((size_t)tile_k * sizeof(float));
        float *O = (float *)malloc((size_t)D * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            int i = rows[r];
            float m = -INFINITY, l = 0.0f;
            for (int d = 0; d < D; ++d) O[d] = 0.0f;
            float dq = qk ? 0.0f : q_scale[i / blk_q];
            for (int j = 0; j < ntile; ++j) {
                int n0 = j * tile_k;
                if (is_causal && n0 > i) break; /* tile entirely in the future */
                float mt = -INFINITY;
                for (int t = 0; t < tile_k; ++t) {
                    int n = n0 + t;
                    if (n >= S || (is_causal && n > i)) {
                        s[t] = -INFINITY;
                    } else if (qk) {
                        s[t] = qk[(size_t)r * S + n] * sm_scale;
                    } else {
                        int kg = k_lane ? orc_lane_group(n) : n / blk_k;
                        float c = (dq * k_scale[kg]) * sm_scale;
                        s[t] = (float)dot_i8(q8 + (size_t)i * D, k8 + (size_t)n * D, D) * c;
                    }
                    if (delta && s[t] != -INFINITY) s[t] = s[t] + delta[(size_t)(i / blk_d) * S + n] * sm_scale;
                    if (s[t] > mt) mt = s[t];
                }
                float mnew = m > mt ? m : mt;
                float alpha = (m == -INFINITY) ? 0.0f : expf(m - mnew);
                for (int t = 0; t < tile_k; ++t) p[t] = (s[t] == -INFINITY) ? 0.0f : expf(s[t] - mnew);
                if (pv_mode == ORC_PV_FP8) {
                    for (int t = 0; t < tile_k; ++t) pq[t] = orc_e4m3_decode(orc_e4m3_encode(p[t] * 448.0f));
                } else if (pv_mode == ORC_PV_FP4) {
                    int g0 = orc_pv_group(n0);
                    for (int g = 0; g < 2 * tile_k / 64; ++g) {
                        float amax = 0.0f;
                        for (int t = 0; t < tile_k; ++t)
                            if (orc_pv_group(n0 + t) - g0 == g && p[t] > amax) amax = p[t];
                        int e = mx_shared_exp(amax);
                        for (int t = 0; t < tile_k; ++t)
                            if (orc_pv_group(n0 + t) - g0 == g)
                                pq[t] = (float)ldexp((double)orc_e2m1_decode(orc_e2m1_encode((float)ldexp((double)p[t], -e))), e);
                    }
                } else {
                    for (int t = 0; t < tile_k; ++t) pq[t] = round_f16(p[t]);
                }
                double psum = 0.0;
                for (int t = 0; t < tile_k; ++t) psum += (double)pq[t];
                l = alpha * l + (float)psum;
                if (pv_mode == ORC_PV_FP8) {
                    for (int d = 0; d < D; ++d) {
                        double acc = 0.0;
                        for (int t = 0; t < tile_k && n0 + t < S; ++t)
                            acc += (double)pq[t] * (double)orc_e4m3_decode(v8[(size_t)(n0 + t) * D + d]);
                        O[d] = alpha * O[d] + (float)acc;
                    }
                } else if (pv_mode == ORC_PV_FP4) {
                    for (int d = 0; d < D; ++d) {
                        double acc = 0.0;
                        for (int t = 0; t < tile_k && n0 + t < S; ++t) {
                            int n = n0 + t;
                            acc += (double)pq[t] * ldexp((double)orc_e2m1_decode(v8[(size_t)n * D + d]),
                                                         (int)v_e8m0[(size_t)orc_pv_group(n) * D + d] - 127);
                        }
                        O[d] = alpha * O[d] + (float)acc;
                    }
                } else {
                    for (int d = 0; d < D; ++d) {
                        double acc = 0.0;
                        for (int t = 0; t < tile_k && n0 + t < S; ++t) {
                            float vv = v[(size_t)(n0 + t) * D + d];
                            if (in_dtype == ORC_BF16) vv = round_f16(vv);
                            acc += (double)pq[t] * (double)vv;
                        }
                        O[d] = alpha * O[d] + (float)acc;
                    }
                }
                m = mnew;
            }
            float *o = out + (size_t)r * D;
            if (l == 0.0f) {
                for (int d = 0; d < D; ++d) o[d] = 0.0f;
            } else if (pv_mode == ORC_PV_FP8) {
                for (int d = 0; d < D; ++d) o[d] = O[d] * (v_scale[d] / l);
                if (v_mean)
                    for (int d = 0; d < D; ++d) o[d] = o[d] + v_mean[d];
            } else {
                for (int d = 0; d < D; ++d) o[d] = O[d] / l;
                if (v_mean && pv_mode == ORC_PV_FP4)
                    for (int d = 0; d < D; ++d) o[d] = o[d] + v_mean[d];
            }
        }
        free(s);
        free(p);
        free(pq);
        free(O);
    }
}

/*
 * Exact attention in binary64, no smoothing and no quantisation:
 * out_i = sum_n softmax_n(sm_scale * q_i . k_n) v_n over the S keys, keys n > i
 * excluded when causal; a row with no visible key is 0.
 */
void orc_attn_exact_head(const float *q, const float *k, const float *v, int S, int D,
                         int is_causal, double sm_scale, const int *rows, int nrows,
                         double *out) {
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)S * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            int i = rows[r];
            int nvis = is_causal ? (i + 1 < S ? i + 1 : S) : S;
            double mx = -INFINITY;
            for (int n = 0; n < nvis; ++n) {
                double a = 0.0;
                for (int d = 0; d < D; ++d) a += (double)q[(size_t)i * D + d] * (double)k[(size_t)n * D + d];
                s[n] = a * sm_scale;
                if (s[n] > mx) mx = s[n];
            }
            double den = 0.0;
            for (int n = 0; n < nvis; ++n) {
                s[n] = exp(s[n] - mx);
                den += s[n];
            }
            double *o = out + (size_t)r * D;
            for (int d = 0; d < D; ++d) {
                double a = 0.0;
                for (int n = 0; n < nvis; ++n) a += s[n] * (double)v[(size_t)n * D + d];
                o[d] = nvis > 0 ? a / den : 0.0;
            }
        }
        free(s);
    }
}
