/*
 * Drives every entry point of the CPU oracle (oracle/sage_oracle.c) on small
 * synthetic heads of awkward sizes -- a single token, ragged blocks and tiles,
 * keys past the last full block, empty heads, every pv format and Q/K format --
 * so that a build with AddressSanitizer and UndefinedBehaviorSanitizer sees
 * every buffer the oracle reads and writes.  It checks no values (the pins do
 * that); it exits non-zero only through the sanitizers or a non-finite output.
 *
 * Test infrastructure: built and run by tests/test_oracle_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "sage_oracle.h"

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* splitmix64 (Steele, Lea, Flood 2014), mapped to a float in [-2, 2) */
static float rnd(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (float)((double)(z >> 11) * (1.0 / 9007199254740992.0) * 4.0 - 2.0);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static int finite_all(const float *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static int run_head(int S, int D, int tile_k) {
    size_t n = (size_t)S * D;
    int nq32 = (S + 31) / 32, nk64 = (S + 63) / 64, ng = 2 * nk64, nl = 2 * ((S + 31) / 32);
    float *q = xmalloc(n * sizeof(float)), *k = xmalloc(n * sizeof(float)), *v = xmalloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) {
        q[i] = rnd();
        k[i] = rnd() + 1.5f;
        v[i] = rnd();
    }
    int8_t *q8 = xmalloc(n), *k8 = xmalloc(n), *kl8 = xmalloc(n);
    float *qs = xmalloc((size_t)(nq32 > 0 ? nq32 : 1) * sizeof(float));
    float *qts = xmalloc((size_t)(S > 0 ? S : 1) * sizeof(float));
    float *ks = xmalloc((size_t)(nk64 > 0 ? nk64 : 1) * sizeof(float));
    float *kls = xmalloc((size_t)(nl > 0 ? nl : 1) * sizeof(float));
    float *km = xmalloc((size_t)D * sizeof(float)), *vm = xmalloc((size_t)D * sizeof(float));
    float *qm = xmalloc((size_t)(nq32 > 0 ? nq32 : 1) * D * sizeof(float));
    uint8_t *v8 = xmalloc(n), *v4 = xmalloc(n), *q4 = xmalloc(n), *k4 = xmalloc(n);
    uint8_t *ve = xmalloc((size_t)(ng > 0 ? ng : 1) * D);
    uint8_t *qe = xmalloc((size_t)(S > 0 ? S : 1) * (D / 32)), *ke = xmalloc((size_t)(S > 0 ? S : 1) * (D / 32));
    float *vs = xmalloc((size_t)D * sizeof(float));
    float *delta = xmalloc((size_t)(nq32 > 0 ? nq32 : 1) * (S > 0 ? S : 1) * sizeof(float));
    int32_t *qk32 = xmalloc((size_t)(S > 0 ? S : 1) * (S > 0 ? S : 1) * sizeof(int32_t));
    float *qkf = xmalloc((size_t)(S > 0 ? S : 1) * (S > 0 ? S : 1) * sizeof(float));
    int *rows = xmalloc((size_t)(S > 0 ? S : 1) * sizeof(int));
    float *out = xmalloc(n * sizeof(float));
    double *outd = xmalloc(n * sizeof(double));
    uint16_t *c16 = xmalloc(n * sizeof(uint16_t));
    int ok = 1;
    for (int i = 0; i < S; ++i) rows[i] = S - 1 - i;

    orc_encode16(q, n, ORC_F16, c16);
    orc_decode16(c16, n, ORC_F16, q);
    orc_encode16(k, n, ORC_BF16, c16);
    orc_decode16(c16, n, ORC_BF16, k);
    orc_quant_q_head(q, S, D, 32, q8, qs);
    orc_quant_q_head(q, S, D, 1, q8, qts);
    orc_quant_k_head(k, S, D, 64, 1, k8, ks, km);
    orc_quant_k_head_lane(k, S, D, 1, kl8, kls, km);
    orc_quant_v_head(v, S, D, v8, vs);
    orc_quant_v_head_smooth(v, S, D, v8, vs, vm);
    orc_quant_v_head_mxfp4(v, S, D, 1, v4, ve, vm);
    orc_quant_q_head_smooth(q, S, D, 32, 32, q8, qs, qm);
    orc_qk_delta_head(qm, nq32, k, km, S, D, delta);
    orc_qk_int32_head(q8, k8, S, D, qk32);
    orc_mxfp4_quant_rows(q, S, D, q4, qe);
    orc_quant_q_head_mxfp4_smooth(q, S, D, 32, q4, qe, qm);
    orc_quant_k_head_mxfp4(k, S, D, 1, k4, ke, km);
    orc_qk_mxfp4_rows(q4, qe, k4, ke, S, D, rows, S, qkf);
    orc_quant_k_head(k, S, D, 64, 1, k8, ks, km);
    orc_quant_q_head(q, S, D, 32, q8, qs);
    for (int causal = 0; causal < 2; ++causal) {
        orc_attn_head_rows(q8, qs, 32, k8, ks, 64, 0, tile_k, v8, vs, ve, NULL, v, ORC_F16, S, D, causal, 0.125f,
                           ORC_PV_FP8, rows, S, NULL, NULL, 32, out);
        ok &= finite_all(out, n);
        orc_attn_head_rows(q8, qs, 32, k8, ks, 64, 0, tile_k, v8, vs, ve, vm, v, ORC_BF16, S, D, causal, 0.125f,
                           ORC_PV_FP16, rows, S, NULL, delta, 32, out);
        ok &= finite_all(out, n);
        orc_attn_head_rows(q8, qts, 1, kl8, kls, 64, 1, tile_k, v4, vs, ve, vm, v, ORC_F16, S, D, causal, 0.125f,
                           ORC_PV_FP4, rows, S, NULL, NULL, 32, out);
        ok &= finite_all(out, n);
        orc_attn_head_rows(q8, qs, 32, k8, ks, 64, 0, tile_k, v4, vs, ve, NULL, v, ORC_F16, S, D, causal, 0.125f,
                           ORC_PV_FP4, rows, S, qkf, delta, 32, out);
        ok &= finite_all(out, n);
        orc_attn_exact_head(q, k, v, S, D, causal, 0.125, rows, S, outd);
    }
    free(q), free(k), free(v), free(q8), free(k8), free(kl8), free(qs), free(qts), free(ks), free(kls);
    free(km), free(vm), free(qm), free(v8), free(v4), free(q4), free(k4), free(ve), free(qe), free(ke);
    free(vs), free(delta), free(qk32), free(qkf), free(rows), free(out), free(outd), free(c16);
    return ok;
}

int main(void) {
    static const int shapes[][3] = {{1, 64, 64}, {31, 64, 128}, {64, 128, 64}, {100, 64, 128},
                                    {129, 128, 128}, {257, 64, 64}, {0, 64, 128}};
    int ok = 1;
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        ok &= run_head(shapes[i][0], shapes[i][1], shapes[i][2]);
        for (uint8_t c = 0;; ++c) {
            volatile float a = orc_e4m3_decode(c), b = orc_e2m1_decode((uint8_t)(c & 15));
            (void)orc_e4m3_encode(a * 1.37f);
            (void)orc_e2m1_encode(b * 0.61f);
            if (c == 255) break;
        }
    }
    for (int t = 0; t < 300; ++t) ok &= orc_lane_group(t) >= 0 && orc_pv_group(t) >= 0;
    printf("%s\n", ok ? "oracle sanitizer run: all outputs finite" : "non-finite output");
    return ok ? 0 : 1;
}
