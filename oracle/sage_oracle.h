/*
 * sage_oracle.h -- plain CPU reference ("oracle") for SageAttention-style
 * quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this code.  The product
 * library (include/sage.h) never links, loads or calls it, and it shares no
 * source, header, table or helper with that library.
 *
 * Everything here works on ONE attention head at a time, on host memory, with
 * row-major [S][D] arrays (token s, channel d).  The callers do the
 * head/layout bookkeeping.  Floating point is IEEE binary32 where the method
 * fixes fp32 (quantisation decisions, the online softmax, the accumulation
 * buffer) and binary64 elsewhere; the library is built without fast-math and
 * without FMA contraction so every fp32 step rounds exactly once.
 *
 * Sources (web pages describing SageAttention; cited by page title and section):
 *   [SA2]   "SageAttention2" paper summary -- sections 相关工作 and SageAttention2方法.
 *   [KAI]   "Kairos的注意力加速利器：SageAttention INT8/FP8量化内核与FLA线性注意力解析指南",
 *           section 二 (2.1 dispatch table, 2.2 why quantisation is near-lossless).
 *   [GUIDE] "SageAttention量化加速框架完整指南：从安装配置到性能调优的实战之路",
 *           sections 五分钟跑通第一个加速样例 and 性能调优实战.
 *   [OCP]   OCP 8-bit floating point specification (E4M3 encoding), the format
 *           named by [SA2] for P~ and V.
 *   [OCP-MX] OCP Microscaling (MX) formats specification: the E2M1 element format
 *           and the E8M0 shared-scale rule of MXFP4, the micro-scaled FP4 that
 *           [KAI] 2.2 names for the next-generation kernels.
 */
#ifndef SAGE_ORACLE_H
#define SAGE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes for 16-bit inputs */
#define ORC_F16 0
#define ORC_BF16 1

/* pv modes */
#define ORC_PV_FP8 0
#define ORC_PV_FP16 1
#define ORC_PV_FP4 2

int orc_num_threads(void);

/* ---- number formats --------------------------------------------------- */
void orc_decode16(const uint16_t *x, size_t n, int dtype, float *out);
void orc_encode16(const float *x, size_t n, int dtype, uint16_t *out);
float orc_e4m3_decode(uint8_t code);
uint8_t orc_e4m3_encode(float x);
void orc_e4m3_encode_n(const float *x, size_t n, uint8_t *out);
float orc_e2m1_decode(uint8_t code);
uint8_t orc_e2m1_encode(float x);

/* ---- quantisation (per head) ----------------------------------------- */
void orc_int8_quant_block(const float *x, size_t n, int8_t *codes, float *scale);
void orc_channel_mean(const float *x, int S, int D, float *mean);
void orc_quant_q_head(const float *q, int S, int D, int blk, int8_t *codes, float *scales);
void orc_quant_k_head(const float *k, int S, int D, int blk, int smooth,
                      int8_t *codes, float *scales, float *mean);
int orc_lane_group(int n);
void orc_quant_q_head_smooth(const float *q, int S, int D, int blk, int blk_scale, int8_t *codes,
                             float *scales, float *qmean);
void orc_qk_delta_head(const float *qmean, int nb, const float *k, const float *kmean, int S, int D,
                       float *delta);
void orc_quant_k_head_lane(const float *k, int S, int D, int smooth,
                           int8_t *codes, float *scales, float *mean);
void orc_quant_v_head(const float *v, int S, int D, uint8_t *codes, float *scales);
void orc_mxfp4_quant_rows(const float *x, int S, int D, uint8_t *codes, uint8_t *e8m0);
void orc_quant_k_head_mxfp4(const float *k, int S, int D, int smooth, uint8_t *codes, uint8_t *e8m0,
                            float *mean);
void orc_qk_mxfp4_rows(const uint8_t *q4, const uint8_t *qe, const uint8_t *k4, const uint8_t *ke, int S,
                       int D, const int *rows, int nrows, float *out);
void orc_quant_v_head_smooth(const float *v, int S, int D, uint8_t *codes, float *scales, float *mean);
void orc_quant_q_head_mxfp4_smooth(const float *q, int S, int D, int blk, uint8_t *codes, uint8_t *e8m0,
                                   float *qmean);
int orc_pv_group(int n);
void orc_quant_v_head_mxfp4(const float *v, int S, int D, int smooth, uint8_t *codes, uint8_t *e8m0,
                            float *mean);

/* ---- attention (per head) ---------------------------------------------- */
void orc_qk_int32_head(const int8_t *q8, const int8_t *k8, int S, int D, int32_t *out);
void orc_attn_head_rows(const int8_t *q8, const float *q_scale, int blk_q,
                        const int8_t *k8, const float *k_scale, int blk_k, int k_lane, int tile_k,
                        const uint8_t *v8, const float *v_scale, const uint8_t *v_e8m0, const float *v_mean,
                        const float *v, int in_dtype, int S, int D, int is_causal, float sm_scale,
                        int pv_mode, const int *rows, int nrows, const float *qk, const float *delta,
                        int blk_d, float *out);
void orc_attn_exact_head(const float *q, const float *k, const float *v, int S, int D,
                         int is_causal, double sm_scale, const int *rows, int nrows,
                         double *out);

#ifdef __cplusplus
}
#endif
#endif
