// api.cpp -- the C ABI of libsage (declared in include/sage.h): argument
// checks, the gfx950 check, buffer geometry and kernel launches.  No compute
// happens here; every step of the method runs in the HIP kernels.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/sage.h"
#include "sage_impl.h"

using namespace sage;

static_assert(SAGE_BLK_Q == kBlkQ && SAGE_BLK_K == kBlkK && SAGE_KV_PAD == kKvPad, "granularity constants disagree");

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned(const void *p, size_t n) { return ((uintptr_t)p % n) == 0; }

int roundup(int x, int m) { return (x + m - 1) / m * m; }

constexpr int kMaxTotal = 1 << 30;  // tokens of a packed batch

int check_shape(int B, int H, int S, int D) {
  if (B < 1 || H < 1 || S < 1 || S > SAGE_MAX_S) return SAGE_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SAGE_ERR_INVALID_ARG;
  if ((long long)B * H > SAGE_MAX_BH) return SAGE_ERR_INVALID_ARG;
  // grid sizes: B*H*(S_q / 32) must fit in a 32-bit launch dimension
  if ((long long)B * H * (roundup(S, kBlkQ) / kBlkQ + 8) >= (1LL << 31)) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

// grouped-query attention: H_kv K/V heads, each shared by H / H_kv query heads
int check_kv_heads(int H, int H_kv) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

int check_qk_quant(int qk_quant) {
  return (qk_quant == SAGE_QK_INT8_BLOCK || qk_quant == SAGE_QK_INT8_LANE || qk_quant == SAGE_QK_MXFP4 ||
          qk_quant == SAGE_QK_INT8_TOKEN || qk_quant == SAGE_QK_INT8_HEAD)
             ? SAGE_OK
             : SAGE_ERR_INVALID_ARG;
}

// scale entries per head: Q per block of kBlkQ rows or per row; K per kBlkK-row block, 16-row group or row
// bytes per head of the Q / K codes and scales for `rows` buffer rows of D channels
size_t code_bytes(size_t rows, int D, int qk) { return qk == SAGE_QK_MXFP4 ? rows * D / 2 : rows * D; }
size_t q_scale_bytes(size_t rows, int D, int qk) {
  if (qk == SAGE_QK_MXFP4) return rows * (D / 32);  // E8M0 bytes
  return (qk == SAGE_QK_INT8_LANE || qk == SAGE_QK_INT8_TOKEN ? rows : rows / kBlkQ) * sizeof(float);
}
size_t k_scale_bytes(size_t rows, int D, int qk) {
  if (qk == SAGE_QK_MXFP4) return rows * (D / 32);
  if (qk == SAGE_QK_INT8_TOKEN) return rows * sizeof(float);
  return (qk == SAGE_QK_INT8_LANE ? rows / 16 : rows / kBlkK) * sizeof(float);
}

int check_enums(int dtype, int layout) {
  if (dtype != SAGE_DTYPE_F16 && dtype != SAGE_DTYPE_BF16) return SAGE_ERR_INVALID_ARG;
  if (layout != SAGE_LAYOUT_HND && layout != SAGE_LAYOUT_NHD) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

// pv mode and its V side buffers: pv fp8 needs the channel scales and pv fp4
// the E8M0 bytes (both through v_scale); V smoothing (v_mean) is for the
// quantised V codes, not for pv fp16, which reads the caller's V.
int check_pv(int pv_mode, const float *v_scale, const float *v_mean) {
  if (pv_mode != SAGE_PV_FP8 && pv_mode != SAGE_PV_FP16 && pv_mode != SAGE_PV_FP4) return SAGE_ERR_INVALID_ARG;
  if (pv_mode != SAGE_PV_FP16 && !v_scale) return SAGE_ERR_INVALID_ARG;
  if (pv_mode == SAGE_PV_FP16 && v_mean) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

// The current device must be gfx950.  Cached per device.
int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return SAGE_ERR_NO_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_NO_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return SAGE_ERR_NO_DEVICE;
    }
    st = sage_check_arch(prop.gcnArchName) == SAGE_OK ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? SAGE_OK : SAGE_ERR_UNSUPPORTED;
}

int launch_status(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_LAUNCH; }

// q16: the 16-bit Q, quantised in the kernel (then q_codes = q_scale = NULL)
int attn_common(const void *q16, const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale,
                const void *v, const float *v_scale, const float *v_mean, const float *q_mean, const float *delta_s,
                void *out, int dtype, int B, int H, int H_kv, int S, int D, int layout, int is_causal, float sm_scale,
                int pv_mode, int qk_quant, int dump_b, int dump_h, int32_t *qk, bool dump, void *stream) {
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if ((rc = check_kv_heads(H, H_kv))) return rc;
  if ((rc = check_qk_quant(qk_quant))) return rc;
  if ((rc = check_enums(dtype, layout))) return rc;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARG;
  if ((rc = check_pv(pv_mode, v_scale, v_mean))) return rc;
  if (!(sm_scale > 0.0f) || !isfinite(sm_scale)) return SAGE_ERR_INVALID_ARG;
  if (q16 && (q_codes || q_scale || qk_quant != SAGE_QK_INT8_BLOCK || delta_s || dump || !aligned(q16, 16)))
    return SAGE_ERR_INVALID_ARG;
  if ((!q16 && (!q_codes || !q_scale)) || !k_codes || !k_scale || !v || !out) return SAGE_ERR_INVALID_ARG;
  if (v_mean && !aligned(v_mean, 4)) return SAGE_ERR_INVALID_ARG;
  // smoothed Q: 4-byte aligned, not with the debug dump, not with per-head scales
  if (delta_s && (!aligned(delta_s, 4) || dump || qk_quant == SAGE_QK_INT8_HEAD)) return SAGE_ERR_INVALID_ARG;
  // INT8 per-block scales: the term is in score units, which the block means fix
  if (delta_s && qk_quant == SAGE_QK_INT8_BLOCK && (!q_mean || !aligned(q_mean, 4))) return SAGE_ERR_INVALID_ARG;
  // pv fp16 reads 128-token slices of the caller's V through a 32-bit byte range
  if (pv_mode == SAGE_PV_FP16 && layout == SAGE_LAYOUT_NHD && (long long)H_kv * D * 2 * kKvPad >= (1LL << 31))
    return SAGE_ERR_INVALID_ARG;
  if ((q_codes && !aligned(q_codes, 16)) || !aligned(k_codes, 16) || !aligned(v, 16) || !aligned(out, 16))
    return SAGE_ERR_INVALID_ARG;
  if ((q_scale && !aligned(q_scale, 4)) || !aligned(k_scale, 4) || (v_scale && !aligned(v_scale, 4)))
    return SAGE_ERR_INVALID_ARG;
  if (dump) {
    if (qk_quant == SAGE_QK_MXFP4) return SAGE_ERR_INVALID_ARG;  // the dump holds INT8 sums
    if (!qk || !aligned(qk, 16)) return SAGE_ERR_INVALID_ARG;
    if (dump_b < 0 || dump_b >= B || dump_h < 0 || dump_h >= H) return SAGE_ERR_INVALID_ARG;
  }
  if ((rc = check_device())) return rc;

  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q_i8 = (const int8_t *)q_codes;
  a.k_i8 = (const int8_t *)k_codes;
  a.q_scale = (const float *)q_scale;
  a.k_scale = (const float *)k_scale;
  a.q = q16;
  a.v = v;
  a.v_scale = v_scale;
  a.v_mean = v_mean;
  a.delta_s = delta_s;
  a.q_mean = delta_s ? q_mean : nullptr;
  a.out = out;
  a.dump = qk;
  a.dump_bh = dump ? dump_b * H + dump_h : -1;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = S;
  a.D = D;
  a.layout = layout;
  a.dtype = dtype;
  a.causal = is_causal;
  a.pv = pv_mode;
  a.S_q = roundup(S, kBlkQ);
  a.S_k = roundup(S, kKvPad);
  a.nq = a.S_q / kBlkQ;
  a.nk = a.S_k / kBlkK;
  a.nmblk = (S + 127) / 128;
  a.sm2 = sm_scale * 1.4426950408889634f;
  a.qk = qk_quant;
  return launch_status(launch_attn(a, dump, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int sage_get_config(int *blk_q, int *blk_k, int *tile_k_fp8, int *tile_k_fp16) {
  if (!blk_q || !blk_k || !tile_k_fp8 || !tile_k_fp16) return SAGE_ERR_INVALID_ARG;
  *blk_q = SAGE_BLK_Q;
  *blk_k = SAGE_BLK_K;
  *tile_k_fp8 = attn_tile_keys(SAGE_PV_FP8);
  *tile_k_fp16 = attn_tile_keys(SAGE_PV_FP16);
  return SAGE_OK;
}

int sage_buffer_sizes(int B, int H, int H_kv, int S, int D, int qk_quant, size_t *q_codes, size_t *q_scale,
                      size_t *k_codes, size_t *k_scale, size_t *k_mean, size_t *v_fp8, size_t *v_scale,
                      size_t *q_mean, size_t *delta_s) {
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if ((rc = check_kv_heads(H, H_kv))) return rc;
  if ((rc = check_qk_quant(qk_quant))) return rc;
  const size_t bh = (size_t)B * H, bhk = (size_t)B * H_kv;
  const size_t S_q = roundup(S, kBlkQ), S_k = roundup(S, kKvPad);
  if (q_codes) *q_codes = bh * code_bytes(S_q, D, qk_quant);
  if (q_scale) *q_scale = bh * q_scale_bytes(S_q, D, qk_quant);
  if (k_codes) *k_codes = bhk * code_bytes(S_k, D, qk_quant);
  if (k_scale) *k_scale = bhk * k_scale_bytes(S_k, D, qk_quant);
  if (k_mean) *k_mean = bhk * D * sizeof(float);
  if (v_fp8) *v_fp8 = bhk * S_k * D;
  if (v_scale) *v_scale = bhk * D * sizeof(float);
  if (q_mean) *q_mean = bh * (S_q / kBlkQ) * D * sizeof(float);
  if (delta_s) *delta_s = bh * (S_q / kBlkQ) * S_k * sizeof(float);
  return SAGE_OK;
}

int sage_v_fp4_buffer_sizes(int B, int H_kv, int S, int D, size_t *v_codes, size_t *v_e8m0) {
  int rc = check_shape(B, H_kv, S, D);
  if (rc) return rc;
  const size_t bhk = (size_t)B * H_kv, S_k = roundup(S, kKvPad);
  if (v_codes) *v_codes = bhk * S_k * D / 2;
  if (v_e8m0) *v_e8m0 = bhk * (S_k / kBlkK) * D * 2;
  return SAGE_OK;
}

// Argument checks and kernel arguments of the Q/K pass (no device check).
static int qk_args(QuantQKArgs &a, const void *q, const void *k, int dtype, int B, int H, int H_kv, int S, int D,
                   int layout, int qk_quant, void *q_codes, void *q_scale, void *k_codes, void *k_scale,
                   float *k_mean, float *q_mean) {
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if ((rc = check_kv_heads(H, H_kv))) return rc;
  if ((rc = check_qk_quant(qk_quant))) return rc;
  if (q_mean && !aligned(q_mean, 4)) return SAGE_ERR_INVALID_ARG;
  if (q_mean && qk_quant == SAGE_QK_INT8_HEAD) return SAGE_ERR_INVALID_ARG;  // per-head scales: unsmoothed Q only
  if ((rc = check_enums(dtype, layout))) return rc;
  // Q omitted (q, q_codes and q_scale all NULL): K alone, for the attention entry
  // points that quantise Q themselves (INT8 per block, unsmoothed Q)
  const bool no_q = !q && !q_codes && !q_scale;
  if (no_q && (qk_quant != SAGE_QK_INT8_BLOCK || q_mean)) return SAGE_ERR_INVALID_ARG;
  if ((!no_q && (!q || !q_codes || !q_scale)) || !k || !k_codes || !k_scale || !k_mean) return SAGE_ERR_INVALID_ARG;
  if (!no_q && (!aligned(q, 16) || !aligned(q_codes, 16) || !aligned(q_scale, 4))) return SAGE_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(k_codes, 16) || !aligned(k_scale, 4) || !aligned(k_mean, 4))
    return SAGE_ERR_INVALID_ARG;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.q_i8 = (int8_t *)q_codes;
  a.k_i8 = (int8_t *)k_codes;
  a.q_scale = (float *)q_scale;
  a.k_scale = (float *)k_scale;
  a.k_mean = k_mean;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = S;
  a.D = D;
  a.layout = layout;
  a.dtype = dtype;
  a.S_q = roundup(S, kBlkQ);
  a.S_k = roundup(S, kKvPad);
  a.nq = a.S_q / kBlkQ;
  a.nk = a.S_k / kBlkK;
  a.qk = qk_quant;
  a.q_mean = q_mean;
  return SAGE_OK;
}

// Argument checks and kernel arguments of the V pass (H: V heads; no device check).
static int v_args(QuantVArgs &a, const void *v, int dtype, int B, int H, int S, int D, int layout, uint8_t *v_fp8,
                  float *v_scale, float *v_mean) {
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if ((rc = check_enums(dtype, layout))) return rc;
  if (!v || !v_fp8 || !v_scale) return SAGE_ERR_INVALID_ARG;
  if (!aligned(v, 16) || !aligned(v_fp8, 16) || !aligned(v_scale, 4) || (v_mean && !aligned(v_mean, 4)))
    return SAGE_ERR_INVALID_ARG;
  memset(&a, 0, sizeof a);
  a.v = v;
  a.v_fp8 = v_fp8;
  a.v_scale = v_scale;
  a.v_mean = v_mean;
  a.B = B;
  a.H = H;
  a.S = S;
  a.D = D;
  a.layout = layout;
  a.dtype = dtype;
  a.nk = roundup(S, kKvPad) / kBlkK;
  return SAGE_OK;
}

int sage_smooth_quant_qk(const void *q, const void *k, int dtype, int B, int H, int H_kv, int S, int D,
                         int layout, int qk_quant, void *q_codes, void *q_scale, void *k_codes, void *k_scale,
                         float *k_mean, float *q_mean, void *stream) {
  QuantQKArgs a;
  int rc = qk_args(a, q, k, dtype, B, H, H_kv, S, D, layout, qk_quant, q_codes, q_scale, k_codes, k_scale, k_mean,
                   q_mean);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  return launch_status(launch_smooth_quant_qk(a, (hipStream_t)stream));
}

int sage_quantize_qkv(const void *q, const void *k, const void *v, int dtype, int B, int H, int H_kv, int S, int D,
                      int layout, int qk_quant, void *q_codes, void *q_scale, void *k_codes, void *k_scale,
                      float *k_mean, float *q_mean, uint8_t *v_fp8, float *v_scale, float *v_mean, void *stream) {
  QuantQKArgs a;
  QuantVArgs va;
  int rc = qk_args(a, q, k, dtype, B, H, H_kv, S, D, layout, qk_quant, q_codes, q_scale, k_codes, k_scale, k_mean,
                   q_mean);
  if (rc) return rc;
  if ((rc = v_args(va, v, dtype, B, H_kv, S, D, layout, v_fp8, v_scale, v_mean))) return rc;
  if ((rc = check_device())) return rc;
  return launch_status(launch_quantize_qkv(a, va, (hipStream_t)stream));
}

int sage_qk_delta(const void *k, int dtype, int B, int H, int H_kv, int S, int D, int layout, int qk_quant,
                  int is_causal, const float *q_mean, const float *k_mean, const void *q_scale, const void *k_scale,
                  float *delta_s, void *stream) {
  int rc = check_shape(B, H, S, D);
  if (rc) return rc;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARG;
  if ((rc = check_kv_heads(H, H_kv))) return rc;
  if ((rc = check_enums(dtype, layout))) return rc;
  if ((rc = check_qk_quant(qk_quant)) || qk_quant == SAGE_QK_INT8_HEAD) return SAGE_ERR_INVALID_ARG;
  if (!k || !q_mean || !k_mean || !delta_s) return SAGE_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(q_mean, 16) || !aligned(k_mean, 4) || !aligned(delta_s, 16))
    return SAGE_ERR_INVALID_ARG;
  // INT8 per-block scales: the term is written in score units (the scales are read)
  if (qk_quant == SAGE_QK_INT8_BLOCK && (!q_scale || !k_scale || !aligned(q_scale, 4) || !aligned(k_scale, 4)))
    return SAGE_ERR_INVALID_ARG;
  if ((rc = check_device())) return rc;
  QuantQKArgs a;
  memset(&a, 0, sizeof a);
  a.k = k;
  a.k_mean = const_cast<float *>(k_mean);
  a.q_mean = const_cast<float *>(q_mean);
  a.q_scale = (float *)const_cast<void *>(q_scale);
  a.k_scale = (float *)const_cast<void *>(k_scale);
  a.qk = qk_quant;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = S;
  a.D = D;
  a.layout = layout;
  a.dtype = dtype;
  a.S_q = roundup(S, kBlkQ);
  a.S_k = roundup(S, kKvPad);
  a.nq = a.S_q / kBlkQ;
  a.nk = a.S_k / kBlkK;
  a.causal = is_causal;
  return launch_status(launch_qk_delta(a, delta_s, (hipStream_t)stream));
}

int sage_quant_v(const void *v, int dtype, int B, int H, int S, int D, int layout, uint8_t *v_fp8, float *v_scale,
                 float *v_mean, void *stream) {
  QuantVArgs a;
  int rc = v_args(a, v, dtype, B, H, S, D, layout, v_fp8, v_scale, v_mean);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  return launch_status(launch_quant_v(a, (hipStream_t)stream));
}

int sage_quant_v_fp4(const void *v, int dtype, int B, int H, int S, int D, int layout, uint8_t *v_codes,
                     uint8_t *v_e8m0, float *v_mean, void *stream) {
  QuantVArgs a;
  if (!v_e8m0 || !aligned(v_e8m0, 4)) return SAGE_ERR_INVALID_ARG;
  // v_args checks the codes buffer and takes v_e8m0 as the (unused) scale slot
  int rc = v_args(a, v, dtype, B, H, S, D, layout, v_codes, reinterpret_cast<float *>(v_e8m0), v_mean);
  if (rc) return rc;
  if ((rc = check_device())) return rc;
  a.v_scale = nullptr;
  a.v_e8m0 = v_e8m0;
  a.code_shift = 1;
  return launch_status(launch_quant_v_fp4(a, (hipStream_t)stream));
}

int sage_attn_fwd(const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale, const void *v,
                  const float *v_scale, const float *v_mean, const float *q_mean, const float *delta_s, void *out,
                  int dtype, int B, int H, int H_kv, int S, int D, int layout, int is_causal, float sm_scale,
                  int pv_mode, int qk_quant, void *stream) {
  return attn_common(nullptr, q_codes, q_scale, k_codes, k_scale, v, v_scale, v_mean, q_mean, delta_s, out, dtype, B,
                     H, H_kv, S, D, layout, is_causal, sm_scale, pv_mode, qk_quant, 0, 0, nullptr, false, stream);
}

int sage_attn_fwd_q16(const void *q, const void *k_codes, const void *k_scale, const void *v, const float *v_scale,
                      const float *v_mean, void *out, int dtype, int B, int H, int H_kv, int S, int D, int layout,
                      int is_causal, float sm_scale, int pv_mode, void *stream) {
  if (!q) return SAGE_ERR_INVALID_ARG;
  return attn_common(q, nullptr, nullptr, k_codes, k_scale, v, v_scale, v_mean, nullptr, nullptr, out, dtype, B, H,
                     H_kv, S, D, layout, is_causal, sm_scale, pv_mode, SAGE_QK_INT8_BLOCK, 0, 0, nullptr, false,
                     stream);
}

int sage_attn_fwd_dump_qk(const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale,
                          const void *v, const float *v_scale, const float *v_mean, void *out, int dtype, int B,
                          int H, int H_kv, int S, int D, int layout, int is_causal, float sm_scale, int pv_mode,
                          int qk_quant, int b, int h, int32_t *qk, void *stream) {
  return attn_common(nullptr, q_codes, q_scale, k_codes, k_scale, v, v_scale, v_mean, nullptr, nullptr, out, dtype, B,
                     H, H_kv, S, D, layout, is_causal, sm_scale, pv_mode, qk_quant, b, h, qk, true, stream);
}

// ---- packed variable-length batches
static int check_varlen(int B, int H, int H_kv, int total_q, int total_k, int max_q, int max_k, int D,
                        int qk_quant) {
  if (B < 1 || total_q < 0 || total_k < 0 || total_q > kMaxTotal || total_k > kMaxTotal) return SAGE_ERR_INVALID_ARG;
  int rc = check_shape(B, H, max_q, D);  // max_q in 1 .. SAGE_MAX_S, launch sizes
  if (rc) return rc;
  if ((rc = check_shape(B, H, max_k, D))) return rc;
  if ((rc = check_qk_quant(qk_quant))) return rc;
  // the per-block passes launch one work-group per block of each head's buffer
  if ((long long)H * (varlen_rows(total_q, B, kBlkQ) / kBlkQ) >= (1LL << 31) ||
      (long long)H * (varlen_rows(total_k, B, kKvPad) / kBlkK) >= (1LL << 31))
    return SAGE_ERR_INVALID_ARG;
  return check_kv_heads(H, H_kv);
}

int sage_varlen_buffer_sizes(int B, int H, int H_kv, int total_q, int total_k, int D, int qk_quant,
                             size_t *q_codes, size_t *q_scale, size_t *k_codes, size_t *k_scale, size_t *k_mean,
                             size_t *v_fp8, size_t *v_scale) {
  int rc = check_varlen(B, H, H_kv, total_q, total_k, 1, 1, D, qk_quant);
  if (rc) return rc;
  const size_t rq = (size_t)varlen_rows(total_q, B, kBlkQ), rk = (size_t)varlen_rows(total_k, B, kKvPad);
  if (q_codes) *q_codes = (size_t)H * code_bytes(rq, D, qk_quant);
  if (q_scale) *q_scale = (size_t)H * q_scale_bytes(rq, D, qk_quant);
  if (k_codes) *k_codes = (size_t)H_kv * code_bytes(rk, D, qk_quant);
  if (k_scale) *k_scale = (size_t)H_kv * k_scale_bytes(rk, D, qk_quant);
  if (k_mean) *k_mean = (size_t)B * H_kv * D * sizeof(float);
  if (v_fp8) *v_fp8 = (size_t)H_kv * rk * D;
  if (v_scale) *v_scale = (size_t)B * H_kv * D * sizeof(float);
  return SAGE_OK;
}

int sage_smooth_quant_qk_varlen(const void *q, const void *k, int dtype, const int32_t *cu_seqlens_q,
                                const int32_t *cu_seqlens_k, int B, int H, int H_kv, int total_q, int total_k,
                                int max_seqlen_q, int max_seqlen_k, int D, int qk_quant, void *q_codes,
                                void *q_scale, void *k_codes, void *k_scale, float *k_mean, float *q_mean,
                                void *stream) {
  int rc = check_varlen(B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D, qk_quant);
  if (rc) return rc;
  if (q_mean && (!aligned(q_mean, 4) || qk_quant == SAGE_QK_INT8_HEAD)) return SAGE_ERR_INVALID_ARG;
  if ((rc = check_enums(dtype, SAGE_LAYOUT_NHD))) return rc;
  // Q omitted: as in the fixed-length call
  const bool no_q = !q && !q_codes && !q_scale;
  if (no_q && (qk_quant != SAGE_QK_INT8_BLOCK || q_mean)) return SAGE_ERR_INVALID_ARG;
  if ((!no_q && (!q || !q_codes || !q_scale)) || !k || !cu_seqlens_q || !cu_seqlens_k || !k_codes || !k_scale ||
      !k_mean)
    return SAGE_ERR_INVALID_ARG;
  if (!no_q && (!aligned(q, 16) || !aligned(q_codes, 16) || !aligned(q_scale, 4))) return SAGE_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(k_codes, 16) || !aligned(k_scale, 4) || !aligned(k_mean, 4) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return SAGE_ERR_INVALID_ARG;
  if ((rc = check_device())) return rc;
  QuantQKArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.q_i8 = (int8_t *)q_codes;
  a.k_i8 = (int8_t *)k_codes;
  a.q_scale = (float *)q_scale;
  a.k_scale = (float *)k_scale;
  a.k_mean = k_mean;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = max_seqlen_k;
  a.D = D;
  a.layout = SAGE_LAYOUT_NHD;
  a.dtype = dtype;
  a.nq = roundup(max_seqlen_q, kBlkQ) / kBlkQ;
  a.nk = roundup(max_seqlen_k, kKvPad) / kBlkK;
  a.varlen = 1;
  a.sq = SeqTable{cu_seqlens_q, total_q, max_seqlen_q};
  a.sk = SeqTable{cu_seqlens_k, total_k, max_seqlen_k};
  a.rows_q = varlen_rows(total_q, B, kBlkQ);
  a.rows_k = varlen_rows(total_k, B, kKvPad);
  a.qk = qk_quant;
  a.q_mean = q_mean;
  return launch_status(launch_smooth_quant_qk(a, (hipStream_t)stream));
}

int sage_varlen_smooth_q_sizes(int B, int H, int total_q, int total_k, int max_seqlen_q, int D, size_t *q_mean,
                               size_t *delta_s) {
  int rc = check_varlen(B, H, H, total_q, total_k, max_seqlen_q, 1, D, SAGE_QK_INT8_BLOCK);
  if (rc) return rc;
  const size_t rq = (size_t)varlen_rows(total_q, B, kBlkQ), rk = (size_t)varlen_rows(total_k, B, kKvPad);
  const size_t mqb = (size_t)roundup(max_seqlen_q, kBlkQ) / kBlkQ;
  if (q_mean) *q_mean = (size_t)H * (rq / kBlkQ) * D * sizeof(float);
  if (delta_s) *delta_s = (size_t)H * (rk / kKvPad) * mqb * kKvPad * sizeof(float);
  return SAGE_OK;
}

int sage_qk_delta_varlen(const void *k, int dtype, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int B,
                         int H, int H_kv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D,
                         int qk_quant, int is_causal, const float *q_mean, const float *k_mean, const void *q_scale,
                         const void *k_scale, float *delta_s, void *stream) {
  int rc = check_varlen(B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D, qk_quant);
  if (rc) return rc;
  if (qk_quant == SAGE_QK_INT8_HEAD || (is_causal != 0 && is_causal != 1)) return SAGE_ERR_INVALID_ARG;
  if ((rc = check_enums(dtype, SAGE_LAYOUT_NHD))) return rc;
  if (!k || !q_mean || !k_mean || !delta_s || !cu_seqlens_q || !cu_seqlens_k) return SAGE_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(q_mean, 16) || !aligned(k_mean, 4) || !aligned(delta_s, 16) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return SAGE_ERR_INVALID_ARG;
  if (qk_quant == SAGE_QK_INT8_BLOCK && (!q_scale || !k_scale || !aligned(q_scale, 4) || !aligned(k_scale, 4)))
    return SAGE_ERR_INVALID_ARG;
  if ((rc = check_device())) return rc;
  QuantQKArgs a;
  memset(&a, 0, sizeof a);
  a.k = k;
  a.k_mean = const_cast<float *>(k_mean);
  a.q_mean = const_cast<float *>(q_mean);
  a.q_scale = (float *)const_cast<void *>(q_scale);
  a.k_scale = (float *)const_cast<void *>(k_scale);
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = max_seqlen_k;
  a.D = D;
  a.layout = SAGE_LAYOUT_NHD;
  a.dtype = dtype;
  a.nq = roundup(max_seqlen_q, kBlkQ) / kBlkQ;  // delta rows per key tile
  a.varlen = 1;
  a.sq = SeqTable{cu_seqlens_q, total_q, max_seqlen_q};
  a.sk = SeqTable{cu_seqlens_k, total_k, max_seqlen_k};
  a.rows_q = varlen_rows(total_q, B, kBlkQ);
  a.rows_k = varlen_rows(total_k, B, kKvPad);
  a.qk = qk_quant;
  a.causal = is_causal;
  return launch_status(launch_qk_delta(a, delta_s, (hipStream_t)stream));
}

int sage_quant_v_varlen(const void *v, int dtype, const int32_t *cu_seqlens_k, int B, int H_kv, int total_k,
                        int max_seqlen_k, int D, uint8_t *v_fp8, float *v_scale, float *v_mean, void *stream) {
  int rc = check_varlen(B, H_kv, H_kv, 0, total_k, 1, max_seqlen_k, D, SAGE_QK_INT8_BLOCK);
  if (rc) return rc;
  if ((rc = check_enums(dtype, SAGE_LAYOUT_NHD))) return rc;
  if (!v || !cu_seqlens_k || !v_fp8 || !v_scale) return SAGE_ERR_INVALID_ARG;
  if (!aligned(v, 16) || !aligned(v_fp8, 16) || !aligned(v_scale, 4) || !aligned(cu_seqlens_k, 4) ||
      (v_mean && !aligned(v_mean, 4)))
    return SAGE_ERR_INVALID_ARG;
  if ((rc = check_device())) return rc;
  QuantVArgs a;
  memset(&a, 0, sizeof a);
  a.v = v;
  a.v_fp8 = v_fp8;
  a.v_scale = v_scale;
  a.v_mean = v_mean;
  a.B = B;
  a.H = H_kv;
  a.S = max_seqlen_k;
  a.D = D;
  a.layout = SAGE_LAYOUT_NHD;
  a.dtype = dtype;
  a.nk = roundup(max_seqlen_k, kKvPad) / kBlkK;
  a.varlen = 1;
  a.sk = SeqTable{cu_seqlens_k, total_k, max_seqlen_k};
  a.rows_k = varlen_rows(total_k, B, kKvPad);
  return launch_status(launch_quant_v(a, (hipStream_t)stream));
}

int sage_varlen_v_fp4_buffer_sizes(int B, int H_kv, int total_k, int D, size_t *v_codes, size_t *v_e8m0) {
  int rc = check_varlen(B, H_kv, H_kv, 0, total_k, 1, 1, D, SAGE_QK_INT8_BLOCK);
  if (rc) return rc;
  const size_t rk = (size_t)varlen_rows(total_k, B, kKvPad);
  if (v_codes) *v_codes = (size_t)H_kv * rk * D / 2;
  if (v_e8m0) *v_e8m0 = (size_t)H_kv * (rk / kBlkK) * D * 2;
  return SAGE_OK;
}

int sage_quant_v_fp4_varlen(const void *v, int dtype, const int32_t *cu_seqlens_k, int B, int H_kv, int total_k,
                            int max_seqlen_k, int D, uint8_t *v_codes, uint8_t *v_e8m0, float *v_mean,
                            void *stream) {
  int rc = check_varlen(B, H_kv, H_kv, 0, total_k, 1, max_seqlen_k, D, SAGE_QK_INT8_BLOCK);
  if (rc) return rc;
  if ((rc = check_enums(dtype, SAGE_LAYOUT_NHD))) return rc;
  if (!v || !cu_seqlens_k || !v_codes || !v_e8m0) return SAGE_ERR_INVALID_ARG;
  if (!aligned(v, 16) || !aligned(v_codes, 16) || !aligned(v_e8m0, 4) || !aligned(cu_seqlens_k, 4) ||
      (v_mean && !aligned(v_mean, 4)))
    return SAGE_ERR_INVALID_ARG;
  if ((rc = check_device())) return rc;
  QuantVArgs a;
  memset(&a, 0, sizeof a);
  a.v = v;
  a.v_fp8 = v_codes;
  a.v_e8m0 = v_e8m0;
  a.v_mean = v_mean;
  a.B = B;
  a.H = H_kv;
  a.S = max_seqlen_k;
  a.D = D;
  a.layout = SAGE_LAYOUT_NHD;
  a.dtype = dtype;
  a.nk = roundup(max_seqlen_k, kKvPad) / kBlkK;
  a.code_shift = 1;
  a.varlen = 1;
  a.sk = SeqTable{cu_seqlens_k, total_k, max_seqlen_k};
  a.rows_k = varlen_rows(total_k, B, kKvPad);
  return launch_status(launch_quant_v_fp4(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {
// the packed-batch attention; q16 as in attn_common
int attn_varlen(const void *q16, const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale,
                const void *v, const float *v_scale, const float *v_mean, const float *q_mean, const float *delta_s,
                void *out, int dtype, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int B, int H,
                int H_kv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D, int is_causal,
                float sm_scale, int pv_mode, int qk_quant, void *stream) {
  int rc = check_varlen(B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D, qk_quant);
  if (rc) return rc;
  if ((rc = check_enums(dtype, SAGE_LAYOUT_NHD))) return rc;
  if (is_causal != 0 && is_causal != 1) return SAGE_ERR_INVALID_ARG;
  if ((rc = check_pv(pv_mode, v_scale, v_mean))) return rc;
  if (!(sm_scale > 0.0f) || !isfinite(sm_scale)) return SAGE_ERR_INVALID_ARG;
  if (q16 && (q_codes || q_scale || qk_quant != SAGE_QK_INT8_BLOCK || delta_s || !aligned(q16, 16)))
    return SAGE_ERR_INVALID_ARG;
  if ((!q16 && (!q_codes || !q_scale)) || !k_codes || !k_scale || !v || !out || !cu_seqlens_q || !cu_seqlens_k)
    return SAGE_ERR_INVALID_ARG;
  if (v_mean && !aligned(v_mean, 4)) return SAGE_ERR_INVALID_ARG;
  // smoothed Q: as in the fixed-length call
  if (delta_s && (!aligned(delta_s, 4) || qk_quant == SAGE_QK_INT8_HEAD)) return SAGE_ERR_INVALID_ARG;
  if (delta_s && qk_quant == SAGE_QK_INT8_BLOCK && (!q_mean || !aligned(q_mean, 4))) return SAGE_ERR_INVALID_ARG;
  // pv fp16 reads 128-token slices of the caller's V through a 32-bit byte range
  if (pv_mode == SAGE_PV_FP16 && (long long)H_kv * D * 2 * kKvPad >= (1LL << 31)) return SAGE_ERR_INVALID_ARG;
  if ((q_codes && !aligned(q_codes, 16)) || !aligned(k_codes, 16) || !aligned(v, 16) || !aligned(out, 16))
    return SAGE_ERR_INVALID_ARG;
  if ((q_scale && !aligned(q_scale, 4)) || !aligned(k_scale, 4) || (v_scale && !aligned(v_scale, 4)) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return SAGE_ERR_INVALID_ARG;
  if ((rc = check_device())) return rc;
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q_i8 = (const int8_t *)q_codes;
  a.k_i8 = (const int8_t *)k_codes;
  a.q_scale = (const float *)q_scale;
  a.k_scale = (const float *)k_scale;
  a.v = v;
  a.v_scale = v_scale;
  a.v_mean = v_mean;
  a.delta_s = delta_s;
  a.q_mean = delta_s ? q_mean : nullptr;
  a.nq = roundup(max_seqlen_q, kBlkQ) / kBlkQ;  // smoothed Q: delta rows per key tile
  a.out = out;
  a.dump = nullptr;
  a.dump_bh = -1;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = max_seqlen_q;  // query blocks per (sequence, head) in the grid
  a.D = D;
  a.layout = SAGE_LAYOUT_NHD;
  a.dtype = dtype;
  a.causal = is_causal;
  a.pv = pv_mode;
  a.sm2 = sm_scale * 1.4426950408889634f;
  a.varlen = 1;
  a.sq = SeqTable{cu_seqlens_q, total_q, max_seqlen_q};
  a.sk = SeqTable{cu_seqlens_k, total_k, max_seqlen_k};
  a.rows_q = varlen_rows(total_q, B, kBlkQ);
  a.rows_k = varlen_rows(total_k, B, kKvPad);
  a.qk = qk_quant;
  a.q = q16;
  return launch_status(launch_attn(a, false, (hipStream_t)stream));
}
}  // namespace

extern "C" {

int sage_attn_fwd_varlen(const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale,
                         const void *v, const float *v_scale, const float *v_mean, const float *q_mean,
                         const float *delta_s, void *out, int dtype, const int32_t *cu_seqlens_q,
                         const int32_t *cu_seqlens_k, int B, int H, int H_kv, int total_q, int total_k,
                         int max_seqlen_q, int max_seqlen_k, int D, int is_causal, float sm_scale, int pv_mode,
                         int qk_quant, void *stream) {
  return attn_varlen(nullptr, q_codes, q_scale, k_codes, k_scale, v, v_scale, v_mean, q_mean, delta_s, out, dtype,
                     cu_seqlens_q, cu_seqlens_k, B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D,
                     is_causal, sm_scale, pv_mode, qk_quant, stream);
}

int sage_attn_fwd_varlen_q16(const void *q, const void *k_codes, const void *k_scale, const void *v,
                             const float *v_scale, const float *v_mean, void *out, int dtype,
                             const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int B, int H, int H_kv,
                             int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D, int is_causal,
                             float sm_scale, int pv_mode, void *stream) {
  if (!q) return SAGE_ERR_INVALID_ARG;
  return attn_varlen(q, nullptr, nullptr, k_codes, k_scale, v, v_scale, v_mean, nullptr, nullptr, out, dtype,
                     cu_seqlens_q, cu_seqlens_k, B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D,
                     is_causal, sm_scale, pv_mode, SAGE_QK_INT8_BLOCK, stream);
}

const char *sage_status_str(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_INVALID_ARG: return "invalid argument";
    case SAGE_ERR_UNSUPPORTED: return "unsupported device (gfx950 required)";
    case SAGE_ERR_NO_DEVICE: return "no HIP device";
    case SAGE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int sage_check_arch(const char *name) {
  if (!name) return SAGE_ERR_INVALID_ARG;
  if (strncmp(name, "gfx950", 6) != 0) return SAGE_ERR_UNSUPPORTED;
  const char c = name[6];
  return (c == '\0' || c == ':') ? SAGE_OK : SAGE_ERR_UNSUPPORTED;
}

}  // extern "C"
