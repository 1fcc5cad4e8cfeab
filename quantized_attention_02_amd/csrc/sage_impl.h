// sage_impl.h -- internals shared by the libsage kernels and the C ABI layer.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sage {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBlkQ = 32;  // Q tokens per INT8 scale (one wavefront's MFMA row tile)
constexpr int kBlkK = 64;  // K tokens per INT8 scale (one 64-key block)
constexpr int kKvPad = 128;  // K / V buffers hold roundup(S, 128) keys: whole 128-key tiles

// Geometry of one attention head inside a physical HND / NHD tensor:
// element (s, d) of head (b, h) lives at base + s * tok_stride + d.
struct HeadView {
  long long base;
  long long tok_stride;
};

__host__ __device__ inline HeadView head_view(int layout, int b, int h, int H, int S, int D) {
  HeadView v;
  if (layout == 0) {  // HND [B][H][S][D]
    v.base = ((long long)b * H + h) * S * D;
    v.tok_stride = D;
  } else {  // NHD [B][S][H][D]
    v.base = ((long long)b * S * H + h) * D;
    v.tok_stride = (long long)H * D;
  }
  return v;
}

// 16-bit input codes -> fp32 (exact for both formats).
__device__ inline float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
template <int DT>
__device__ inline float in_to_f32(uint32_t bits16) {
  return DT == 0 ? f16_to_f32(bits16) : bf16_to_f32(bits16);
}

// fp32 -> 16-bit codes, round to nearest even (hardware conversion for fp16;
// carry-propagating rounding on the bit pattern for bf16, finite inputs).
__device__ inline uint32_t f32_to_f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ inline uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
template <int DT>
__device__ inline uint32_t f32_to_out_bits(float x) {
  return DT == 0 ? f32_to_f16_bits(x) : f32_to_bf16_bits(x);
}

// Byte p (0..63) of a V tile row holds key vpos_key(p) of the tile; the inverse
// maps a key to its byte.  This is the key order in which the attention kernel
// holds P~ in registers after the K.Q^T MFMA (see attn.hip).
__host__ __device__ constexpr int vpos_key(int p) {
  return 32 * ((p & 31) >> 4) + 8 * ((p & 15) >> 2) + 4 * (p >> 5) + (p & 3);
}
__host__ __device__ constexpr int key_vpos(int n) {
  return 32 * ((n >> 2) & 1) + 16 * (n >> 5) + 4 * ((n & 31) >> 3) + (n & 3);
}

// ---- packed variable-length batches
// Sequence b owns tokens cu[b] .. cu[b+1] of a token-major [T][H][D] tensor.
// In the quantised buffers each (sequence, head) gets its own run of rows:
// a head's buffer has varlen_rows(T, B, pad) rows and sequence b starts at row
// seq_row0(cu[b], b, pad), a multiple of pad (32 for Q, 128 for K and V), so
// runs hold roundup(length, pad) rows without overlapping.
struct SeqTable {
  const int *cu;  // device, B + 1 entries
  int total;      // tokens in the packed tensor
  int max_len;    // upper bound of every length (host-side)
};

// Sequence b's first token and length, clamped to [0, total] and max_len so
// that every access stays inside the buffers whatever the table holds.
__device__ inline void seq_span(const SeqTable &t, int b, int &start, int &len) {
  int c0 = t.cu[b], c1 = t.cu[b + 1];
  c0 = min(max(c0, 0), t.total);
  c1 = min(max(c1, c0), t.total);
  start = c0;
  len = min(c1 - c0, t.max_len);
}
__host__ __device__ inline long long seq_row0(int start, int b, int pad) {
  return (long long)pad * (start / pad + b);
}
__host__ __device__ inline long long varlen_rows(int total, int B, int pad) {
  return (long long)pad * (total / pad + B + 1);
}

// One (sequence or batch entry, head) of an input tensor and its rows in a
// quantised buffer: element (s, d), s < S, is at base + s * stride + d of the
// input; its buffer row is row0 + s.
// Buffer resource for `bytes` bytes at `base` (raw buffer: stride 0, 32-bit
// data format).  Loads through it past `bytes` return zeros; stores past it
// are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

struct Seg {
  int S;
  long long base, stride, row0;
};

// fixed-length: head (b, h) of [B][H][S][D] / [B][S][H][D], buffers [B][H][S_pad][D]
__host__ __device__ inline Seg fixed_seg(int layout, int b, int h, int H, int S, int S_pad, int D) {
  const HeadView v = head_view(layout, b, h, H, S, D);
  return Seg{S, v.base, v.tok_stride, ((long long)b * H + h) * S_pad};
}
// packed: head h of sequence b in [T][H][D], buffers [H][rows][D]
__device__ inline Seg varlen_seg(const SeqTable &t, int b, int h, int H, int D, long long rows, int pad) {
  int start, len;
  seq_span(t, b, start, len);
  return Seg{len, ((long long)start * H + h) * D, (long long)H * D, h * rows + seq_row0(start, b, pad)};
}

// Smoothed Q with INT8 per-block scales: the pre-processing term delta enters
// the attention's INT8 accumulator as rint(delta / (u dk)), so the score scale u
// of a Q block must keep |delta| / (u dk) within int32 next to the INT8 sum
// (|sum| <= 127^2 D < 2^22).  |delta| <= sum_d |qbar_d| * 127 dk, so a scale of at
// least 127 sum_d |qbar_d| 2^-30 suffices; a block whose own scale dq is smaller
// (its residual Q - qbar is at or below fp32 resolution of qbar, or zero) takes
// that bound and drops its INT8 codes.  sum_abs: sum_d |qbar_d| in fp32 (the
// pre-processing pass and the attention kernel may sum in different orders; u
// then differs by a few ulps, well inside the term's rounding to units).
__device__ inline float smooth_q_unit(float dq, float sum_abs) { return fmaxf(dq, 127.0f * sum_abs * 0x1p-30f); }

struct QuantQKArgs {
  const void *q, *k;
  int8_t *q_i8, *k_i8;
  float *q_scale, *k_scale, *k_mean;
  int B, H, H_kv, S, D, layout, dtype;  // K has H_kv heads
  int S_q, S_k, nq, nk;                 // nq / nk: Q / K scale blocks per head (grid extent)
  int varlen;                           // packed batch: tables below, S unused
  SeqTable sq, sk;
  long long rows_q, rows_k;  // buffer rows per head (packed batch)
  int qk;                    // Q/K quantisation: 0 INT8 per block, 1 INT8 per lane, 2 MXFP4
  float *q_mean;             // smoothed Q: block means [B][H][nq][D] (nullptr: no Q smoothing)
  int causal;                // pre-processing term: only what a causal attention reads
};

struct QuantVArgs {
  const void *v;
  uint8_t *v_fp8;   // E4M3 codes (pv fp8) or packed E2M1 codes (pv fp4)
  uint8_t *v_e8m0;  // pv fp4: E8M0 scale per (64-key block, channel, key group)
  float *v_scale;
  float *v_mean;  // V smoothing: channel means out (nullptr: no smoothing)
  int B, H, S, D, layout, dtype;
  int nk;  // 64-key tiles per head (grid extent)
  int code_shift;  // log2(codes per byte) of v_fp8: 0 E4M3, 1 packed E2M1
  int varlen;
  SeqTable sk;
  long long rows_k;
};

struct AttnArgs {
  const int8_t *q_i8, *k_i8;
  const float *q_scale, *k_scale;
  const void *v;
  const float *v_scale;  // pv fp8: per-channel scales; pv fp4: the E8M0 bytes (reinterpreted)
  const float *v_mean;  // smoothed V: channel means added to the output (nullptr: none)
  const float *delta_s;  // smoothed Q: pre-processing term [B][H][nq][S_k] (nullptr: none)
  const float *q_mean;   // smoothed Q with INT8 per-block scales: the block means (score units)
  const void *q;         // the 16-bit Q itself, quantised in the attention kernel (q_i8, q_scale unused)
  void *out;
  int32_t *dump;
  int dump_bh;
  int B, H, H_kv, S, D, layout, dtype, causal, pv;  // K and V have H_kv heads
  int S_q, S_k, nq, nk, nmblk;
  float sm2;  // sm_scale * log2(e)
  int varlen;  // packed batch: tables below, S = the longest query sequence
  SeqTable sq, sk;
  long long rows_q, rows_k;
  int qk;  // Q/K quantisation of q_codes / k_codes (as QuantQKArgs::qk)
};

hipError_t launch_smooth_quant_qk(const QuantQKArgs &a, hipStream_t stream);
hipError_t launch_quant_v(const QuantVArgs &a, hipStream_t stream);
hipError_t launch_quant_v_fp4(const QuantVArgs &a, hipStream_t stream);
// pre-processing term of smoothed Q, delta[B][H][nq][S_k] (a.q_mean and a.k_mean read)
hipError_t launch_quantize_qkv(const QuantQKArgs &a, const QuantVArgs &v, hipStream_t stream);
hipError_t launch_qk_delta(const QuantQKArgs &a, float *delta, hipStream_t stream);
hipError_t launch_attn(const AttnArgs &a, bool dump, hipStream_t stream);
int attn_tile_keys(int pv_mode);  // keys per online-softmax tile of the attention kernel

}  // namespace sage
