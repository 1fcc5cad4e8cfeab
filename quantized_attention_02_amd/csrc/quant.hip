// quant.hip -- the two quantisation passes in front of the attention kernel.
//
//  * K smoothing: per-channel mean of K over the S tokens of each head,
//    subtracted before INT8 quantisation ("SageAttention2" summary, section
//    相关工作: K is pre-processed to keep INT8 accurate; section SageAttention2方法:
//    K smoothing).
//  * Per-block symmetric INT8 for Q and K ("Kairos" guide, section 2.2).
//  * Per-channel FP8 E4M3 for V ("SageAttention2" summary, SageAttention2方法).
//
// All three are HBM-bound streaming passes.  Every work-group reads whole
// 16-byte vectors of consecutive channels, so loads are coalesced in both the
// HND and the NHD layout.  Quantisation decisions are single, correctly
// rounded fp32 operations (no contraction), so codes are reproducible
// bit for bit on any IEEE machine.
#include <type_traits>

#include "sage_impl.h"

#pragma clang fp contract(off)

namespace sage {

static_assert(vpos_key(key_vpos(0)) == 0 && vpos_key(key_vpos(37)) == 37 && vpos_key(key_vpos(63)) == 63,
              "V tile key order must be a bijection");

constexpr int kThreads = 256;

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Block-wide max of a non-negative value; every thread receives the result.
__device__ inline float block_max(float x, float *red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// Load 8 consecutive 16-bit values (one 16-byte vector) and widen to fp32.
template <int DT>
__device__ inline void load8(const uint16_t *p, float *x) {
  const v4i u = *reinterpret_cast<const v4i *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = in_to_f32<DT>((uint32_t)u[i] & 0xffffu);
    x[2 * i + 1] = in_to_f32<DT>((uint32_t)u[i] >> 16);
  }
}

__device__ inline int8_t to_i8(float x, float inv) {
  float t = __builtin_rintf(x * inv);
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return (int8_t)(int)t;
}

// ---------------------------------------------------------------------------
// Per-channel reductions over the tokens of a head (the K channel sums and the
// V channel abs-max) run as a two-level reduction: one work-group per
// (head, chunk of tokens) writes per-chunk partials, and a small kernel
// combines a head's partials.  The partials live in the head's region of the
// output buffer that the next pass overwrites (k_i8 for K, v_fp8 for V), so
// the entry points need no workspace: a chunk has at least 256 tokens, and
// its 256 * D bytes of codes hold its D partials (8 bytes each) with room to
// spare.
// ---------------------------------------------------------------------------
constexpr int kMaxChunks = 32;

// Tokens per chunk: a multiple of 256 such that a head has at most kMaxChunks
// chunks (256 up to S = 8192).
__host__ __device__ inline int chunk_tokens(int S) {
  const int per = (S + kMaxChunks - 1) / kMaxChunks;
  return max(256, ((per + 255) / 256) * 256);
}
__host__ __device__ inline int n_chunks(int S) {
  const int c = chunk_tokens(S);
  return (S + c - 1) / c;
}
// Chunk work-groups launched per head when heads have at most max_len tokens:
// n_chunks(S) <= chunk_grid(max_len) for every S <= max_len.
__host__ __device__ inline int chunk_grid(int max_len) { return min(kMaxChunks, (max_len + 255) / 256); }

// The head (or sequence-head) of each pass: fixed-length batches or packed ones.
template <int D>
__device__ inline Seg q_seg(const QuantQKArgs &a, int b, int h) {
  return a.varlen ? varlen_seg(a.sq, b, h, a.H, D, a.rows_q, kBlkQ) : fixed_seg(a.layout, b, h, a.H, a.S, a.S_q, D);
}
template <int D>
__device__ inline Seg k_seg(const QuantQKArgs &a, int b, int h) {
  return a.varlen ? varlen_seg(a.sk, b, h, a.H_kv, D, a.rows_k, kKvPad)
                  : fixed_seg(a.layout, b, h, a.H_kv, a.S, a.S_k, D);
}
template <int D>
__device__ inline Seg v_seg(const QuantVArgs &a, int b, int h) {
  return a.varlen ? varlen_seg(a.sk, b, h, a.H, D, a.rows_k, kKvPad)
                  : fixed_seg(a.layout, b, h, a.H, a.S, a.nk * kBlkK, D);
}
// The chunk partials of one V head sit at the start of the head's run of the
// code buffer: roundup(S, 128) * D bytes for E4M3 codes, half that for E2M1.
__device__ inline uint8_t *v_partials(const QuantVArgs &a, const Seg &sg, int D) {
  return a.v_fp8 + ((sg.row0 * D) >> a.code_shift);
}
__device__ inline int ceil_div(int x, int m) { return (x + m - 1) / m; }

// Work-group -> (batch entry or sequence b, head h, block blk) of a per-block
// pass.  Fixed-length batches: wg = (b H + h) nblk + blk.  Packed batches: the
// grid covers each head's whole buffer, wg = h (rows / brows) + kb in blocks of
// brows rows; sequence b's run starts at row seq_row0(start_b, b, pad), which
// strictly increases with b, so b is found by binary search over the table
// (wave-uniform loads).  Callers compare blk with the sequence's block count: a
// block in the gap after a run has none (and a malformed table only moves the
// block to another clamped sequence).
__device__ inline void block_of(bool varlen, const SeqTable &t, int B, int H, int nblk, long long rows, int pad,
                                int brows, int wg, int &b, int &h, int &blk) {
  if (!varlen) {
    const int bh = wg / nblk;
    b = bh / H;
    h = bh % H;
    blk = wg % nblk;
    return;
  }
  const int nb = (int)(rows / brows);
  h = wg / nb;
  const long long r = (long long)(wg % nb) * brows;  // the block's first row in the head's buffer
  int lo = 0, hi = B - 1, start, len;
  while (lo < hi) {  // the last sequence whose run starts at or before row r
    const int mid = (lo + hi + 1) >> 1;
    seq_span(t, mid, start, len);
    if (seq_row0(start, mid, pad) <= r) lo = mid;
    else hi = mid - 1;
  }
  b = lo;
  seq_span(t, b, start, len);
  const long long off = r - seq_row0(start, b, pad);
  blk = off < 0 ? INT_MAX : (int)(off / brows);
}
// bytes of one quantised Q/K row: INT8 codes, or packed E2M1 pairs (MXFP4)
template <int D>
__device__ inline int code_row_bytes(const QuantQKArgs &a) { return a.qk == 2 ? D / 2 : D; }

// Thread layout of the chunk passes: G = D / 8 channel groups (16 bytes of a
// 16-bit row) x R = 256 / G rows; the chunk's rows are loaded kUnroll at a
// time, 256 rows (a minimum-size chunk) per round, so that a chunk of 256
// tokens is read with all of its loads in flight at once.
template <int D>
struct ChunkMap {
  static constexpr int G = D / 8;
  static constexpr int R = kThreads / G;
  static constexpr int kUnroll = 256 / R;
};

// K channel sums (binary64) of one chunk -> partials[chunk][D]; or, with
// ABSMAX, channel abs-max (fp32) of one chunk.  MINMAX (with the sums): also
// the chunk's channel max and min (fp32) -> minmax[chunk][2][D].
template <int DT, int D, bool ABSMAX, bool MINMAX = false>
__device__ inline void chunk_reduce(const uint16_t *x, const Seg &hv, int chunk, void *partials,
                                    float *minmax = nullptr) {
  static_assert(!(ABSMAX && MINMAX), "max / min ride along with the sums");
  const int S = hv.S;
  using M = ChunkMap<D>;
  typedef typename std::conditional<ABSMAX, float, double>::type acc_t;
  __shared__ acc_t part[M::R][D];
  __shared__ float pmx[MINMAX ? M::R : 1][MINMAX ? D : 1], pmn[MINMAX ? M::R : 1][MINMAX ? D : 1];
  const int tid = threadIdx.x, g = tid % M::G, r = tid / M::G;
  const int ct = chunk_tokens(S);
  const int s_end = min(S, (chunk + 1) * ct);
  acc_t acc[8];
  float mx[8], mn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i] = 0;
    mx[i] = -INFINITY;
    mn[i] = INFINITY;
  }
  for (int s0 = chunk * ct + r; s0 < s_end; s0 += M::R * M::kUnroll) {
    v4i raw[M::kUnroll];  // 16-bit pairs as loaded (zeros past the chunk)
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int s = s0 + u * M::R;
      raw[u] = s < s_end ? *reinterpret_cast<const v4i *>(x + hv.base + (long long)s * hv.stride + 8 * g)
                         : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = in_to_f32<DT>(i & 1 ? (uint32_t)raw[u][i >> 1] >> 16 : (uint32_t)raw[u][i >> 1] & 0xffffu);
        if (ABSMAX) acc[i] = fmaxf(acc[i], fabsf(v));
        else acc[i] += (double)v;
        if (MINMAX && s0 + u * M::R < s_end) {  // (rows past the chunk are not tokens)
          mx[i] = fmaxf(mx[i], v);
          mn[i] = fminf(mn[i], v);
        }
      }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    part[r][8 * g + i] = acc[i];
    if (MINMAX) {
      pmx[r][8 * g + i] = mx[i];
      pmn[r][8 * g + i] = mn[i];
    }
  }
  __syncthreads();
  if (tid < D) {
    acc_t t = part[0][tid];
    for (int rr = 1; rr < M::R; ++rr) {
      if (ABSMAX) t = fmaxf(t, part[rr][tid]);
      else t += part[rr][tid];
    }
    reinterpret_cast<acc_t *>(partials)[(long long)chunk * D + tid] = t;
    if (MINMAX) {
      float a = pmx[0][tid], b = pmn[0][tid];
      for (int rr = 1; rr < M::R; ++rr) {
        a = fmaxf(a, pmx[rr][tid]);
        b = fminf(b, pmn[rr][tid]);
      }
      minmax[((long long)chunk * 2) * D + tid] = a;
      minmax[((long long)chunk * 2 + 1) * D + tid] = b;
    }
  }
}

// ---------------------------------------------------------------------------
// K channel sums of one chunk of tokens -> partials (k_i8 region of the head).
// ---------------------------------------------------------------------------
// HEAD (per-head granularity): also each chunk's channel max and min, stored
// after the head's n_chunks(S) sums (2 D floats a chunk: the sums and these
// take 16 D bytes a chunk of at least 256 tokens, inside the head's codes).
template <int DT, int D, bool HEAD = false>
__device__ inline void ksum_wg(const QuantQKArgs &a, int wg) {
  const int nch = chunk_grid(a.varlen ? a.sk.max_len : a.S);
  const int bh = wg / nch, chunk = wg % nch;  // bh: K head (b, h_kv)
  const Seg sg = k_seg<D>(a, bh / a.H_kv, bh % a.H_kv);
  if (chunk >= n_chunks(sg.S)) return;
  int8_t *part = a.k_i8 + sg.row0 * code_row_bytes<D>(a);
  float *minmax = reinterpret_cast<float *>(reinterpret_cast<double *>(part) + (long long)n_chunks(sg.S) * D);
  chunk_reduce<DT, D, false, HEAD>((const uint16_t *)a.k, sg, chunk, part, minmax);
}
template <int DT, int D, bool HEAD>
__global__ __launch_bounds__(kThreads) void k_ksum(const QuantQKArgs a) { ksum_wg<DT, D, HEAD>(a, blockIdx.x); }

// ---------------------------------------------------------------------------
// Per-head granularity of Q: channel abs-max of one chunk of a Q head ->
// partials[chunk][D] (fp32) in the head's codes, which the Q pass overwrites
// later; then one work-group per head reduces them to the head's abs-max and
// leaves it in every block slot of q_scale, where each block's Q pass reads it
// before writing its scale there.
// ---------------------------------------------------------------------------
template <int DT, int D>
__device__ inline void qamax_part_wg(const QuantQKArgs &a, int wg) {
  const int nch = chunk_grid(a.varlen ? a.sq.max_len : a.S);
  const int bh = wg / nch, chunk = wg % nch;  // bh: Q head (b, h)
  const Seg sg = q_seg<D>(a, bh / a.H, bh % a.H);
  if (chunk >= n_chunks(sg.S)) return;
  chunk_reduce<DT, D, true>((const uint16_t *)a.q, sg, chunk, a.q_i8 + sg.row0 * D);
}
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void k_qamax_part(const QuantQKArgs a) { qamax_part_wg<DT, D>(a, blockIdx.x); }

template <int D>
__device__ inline void qhead_wg(const QuantQKArgs &a, int wg) {
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x;
  const Seg sg = q_seg<D>(a, wg / a.H, wg % a.H);  // (uniform across the work-group)
  const float *part = reinterpret_cast<const float *>(a.q_i8 + sg.row0 * D);
  const int n = n_chunks(sg.S) * D;  // <= kMaxChunks D
  float m = 0.0f;
  for (int i = tid; i < n; i += kThreads) m = fmaxf(m, part[i]);
  m = block_max(m, red);
  const int nblk = ceil_div(sg.S, kBlkQ);
  for (int blk = tid; blk < nblk; blk += kThreads) a.q_scale[(sg.row0 >> 5) + blk] = m;
}
template <int D>
__global__ __launch_bounds__(kThreads) void k_qhead(const QuantQKArgs a) { qhead_wg<D>(a, blockIdx.x); }

// ---------------------------------------------------------------------------
// Smoothed Q ("SageAttention2" summary, SageAttention2方法: subtract each block
// of Q's mean; with K smoothing, Q K^T splits into a pre-processing stage and
// the attention stage): the channel means of the block's valid tokens (binary64
// sums -- exact for 32 values of a 16-bit format -- divided by their number,
// rounded once) go to q_mean[block][D] and are subtracted from the block's
// valid rows (padding rows stay 0).  x: the thread's two row vectors as
// k_qquant loads them; nvalid: the block's valid rows; gblk: the block's index
// in q_mean.
// ---------------------------------------------------------------------------
template <int D>
__device__ inline void q_block_smooth(const QuantQKArgs &a, float (&x)[2][8], int nvalid, long long gblk) {
  constexpr int vec_per_row = D / 8;
  constexpr int RPP = kThreads / vec_per_row;  // rows a pass of the 256 threads covers
  __shared__ double part[RPP][D];
  __shared__ float mean[D];
  const int tid = threadIdx.x, c8 = (tid % vec_per_row) * 8, r = tid / vec_per_row;
#pragma unroll
  for (int i = 0; i < 8; ++i) part[r][c8 + i] = (double)x[0][i] + (double)x[1][i];  // rows r and r + RPP
  __syncthreads();
  if (tid < D) {
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < RPP; ++j) t += part[j][tid];
    const float m = nvalid > 0 ? (float)(t / (double)min(nvalid, kBlkQ)) : 0.0f;
    mean[tid] = m;
    a.q_mean[gblk * D + tid] = m;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = (tid + u * kThreads) / vec_per_row;
    if (tid + u * kThreads < kBlkQ * vec_per_row && row < nvalid)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = x[u][i] - mean[c8 + i];
  }
}

// ---------------------------------------------------------------------------
// The pre-processing stage of smoothed Q:
//   delta[bh][blk][n] = sum_d q_mean[bh][blk][d] * (K[n][d] - k_mean[d])
// for n < S (0 for the padding keys up to S_k): an [nq x D] . [D x S] product
// per head, run on the 16-bit MFMA as
//   delta = q_mean . K  -  q_mean . k_mean.
// K enters the MFMA exactly (it is fp16 / bf16 already).  q_mean is split into
// 16-bit pieces that sum to it: fp16 hi + lo (22 significant bits) for fp16
// inputs, three truncated bf16 pieces (all 24 bits, exact) for bf16.  Products
// of 16-bit values are exact in the fp32 accumulator, so the result carries fp32
// summation rounding only (and 2^-22 of q_mean with fp16 inputs).
// A work-group of four wavefronts owns 128 keys of one query head.  Each
// wavefront keeps its 32 keys' K rows in registers (the A operand) and walks the
// head's query blocks 32 at a time.  The split means of those 32 blocks and their
// dot products with k_mean are staged once per work-group in LDS (the B operand;
// rows padded by 16 bytes against bank conflicts; two buffers, so one barrier a
// chunk), and the means of the chunk after next load while a chunk is computed.  A
// lane ends with 16 results of one query block: 4 runs of 4 consecutive keys,
// stored as 4 float4.  delta is stored tile-major ([bh][key tile][block][128
// keys]), so a work-group writes one contiguous 16 KB region per chunk.  Packed
// batches: [query head][128-row tile of the K buffer][block][128 keys], with as
// many blocks as the longest query sequence has; a sequence's tiles hold its
// own query blocks and the rest of each tile is left as it was.
// INTU (INT8 per-block scales): each result is stored as the int32
// rint(delta / (dq dk)) in the score units of its Q block and 64-key K block
// (smooth_q_unit), the starting value of the attention's INT8 accumulator.
// ---------------------------------------------------------------------------
constexpr int kDeltaKeys = 128;
static_assert(kDeltaKeys == kKvPad, "a delta work-group covers one 128-key K tile");

template <int DT>
struct DeltaMfma;

template <>
struct DeltaMfma<0> {  // fp16 inputs
  typedef _Float16 T8 __attribute__((ext_vector_type(8)));
  static constexpr int kSplit = 2;
  __device__ static v16f mfma(T8 a, T8 b, v16f c) { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
  // x = hi + lo + r with |r| <= 2^-22 |x| (+ 2^-25 near the fp16 subnormal range)
  __device__ static void split(float x, uint16_t *p) {
    const _Float16 hi = (_Float16)x;
    const _Float16 lo = (_Float16)(x - (float)hi);  // x - hi is exact in fp32
    p[0] = __builtin_bit_cast(uint16_t, hi);
    p[1] = __builtin_bit_cast(uint16_t, lo);
  }
};

template <>
struct DeltaMfma<1> {  // bf16 inputs
  typedef __bf16 T8 __attribute__((ext_vector_type(8)));
  static constexpr int kSplit = 3;
  __device__ static v16f mfma(T8 a, T8 b, v16f c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
  // truncation to the top 8 significant bits, three times: the pieces hold all
  // 24 bits of x, and each remainder is an exact fp32 subtraction
  __device__ static void split(float x, uint16_t *p) {
    float r = x;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const uint32_t u = __float_as_uint(r) & 0xffff0000u;
      p[i] = (uint16_t)(u >> 16);
      r = r - __uint_as_float(u);
    }
  }
};

template <int DT, int D, bool INTU>
__global__ __launch_bounds__(kThreads) void k_qk_delta(const QuantQKArgs a, float *delta) {
  typedef DeltaMfma<DT> M;
  typedef typename M::T8 T8;
  constexpr int NS = M::kSplit;
  constexpr int KSTEPS = D / 16;  // MFMA k steps over the channels
  constexpr int RS = D + 8;       // LDS row stride (16-bit elements): 16 bytes of padding
  constexpr int CPT = D / 8;      // channels per staging thread (8 threads per query block)
  __shared__ __align__(16) uint16_t am[2][NS][32 * RS];  // double-buffered by chunk
  __shared__ float cs[2][32];
  __shared__ float cu[2][32];  // INTU: each block's score scale (smooth_q_unit)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  // fixed length: S_k / 128 key tiles per (batch, query head); packed batches:
  // rows_k / 128 per query head, each in one sequence's run (or between runs)
  const int nkt = a.varlen ? (int)(a.rows_k / kDeltaKeys) : a.S_k / kDeltaKeys;
  // work-group -> (query head, key tile); with a grid that divides evenly, each
  // XCD takes whole heads, so a head's block means are read through one L2
  int wg = blockIdx.x;
  if ((gridDim.x & 7) == 0) wg = (wg & 7) * (gridDim.x >> 3) + (wg >> 3);
  int b, h, kt;  // kt: the tile within the sequence (packed) or the head (fixed)
  block_of(a.varlen, a.sk, a.B, a.H, nkt, a.rows_k, kKvPad, kDeltaKeys, wg, b, h, kt);
  const int bh = b * a.H + h, hk = h / (a.H / a.H_kv);
  const Seg ks = a.varlen ? varlen_seg(a.sk, b, hk, a.H_kv, D, a.rows_k, kKvPad)
                          : fixed_seg(a.layout, b, hk, a.H_kv, a.S, a.S_k, D);
  if (kt >= ceil_div(ks.S, kDeltaKeys)) return;  // past this sequence's keys (packed batches)
  // the query blocks: the batch entry's, or the sequence's (its own run of Q rows)
  long long qblk0;  // the first block's index in q_mean / q_scale
  int nqb;          // blocks of this sequence (fixed length: of the head)
  long long drow0;  // this tile's first row of delta ([tile][block][128 keys])
  if (a.varlen) {
    const Seg qv = varlen_seg(a.sq, b, h, a.H, D, a.rows_q, kBlkQ);
    qblk0 = qv.row0 >> 5;
    nqb = ceil_div(qv.S, kBlkQ);
    drow0 = ((long long)h * nkt + ((ks.row0 - (long long)hk * a.rows_k) >> 7) + kt) * a.nq;
  } else {
    qblk0 = (long long)bh * a.nq;
    nqb = a.nq;
    drow0 = ((long long)bh * nkt + kt) * a.nq;
  }
  const int S = ks.S;                            // this sequence's keys
  const int key0 = kt * kDeltaKeys + 32 * wave;  // this wavefront's 32 keys (< S_k)
  const int n = key0 + (lane & 31);              // the key whose K row this lane holds
  // A operand: channels 16 s + 8 hh .. +7 of key n for each k step s
  const uint16_t *k = (const uint16_t *)a.k;
  T8 kf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    v4i u = {0, 0, 0, 0};
    if (n < S) u = *reinterpret_cast<const v4i *>(k + ks.base + (long long)n * ks.stride + 16 * s + 8 * hh);
    kf[s] = __builtin_bit_cast(T8, u);
  }
  // staging role: query block sb of a chunk, channels sc .. sc + CPT - 1
  const int sb = tid >> 3, sc = (tid & 7) * CPT;
  float km[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) km[i] = a.k_mean[((long long)b * a.H_kv + hk) * D + sc + i];
  // The head's block means and this work-group's 128-key tile of delta go
  // through buffer resources: loads past the last block return zeros and stores
  // past it are dropped, so neither needs a branch, and the wait for a chunk's
  // prefetched means leaves the previous chunk's stores in flight.
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q_mean + qblk0 * D, nqb * D * 4);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(delta + drow0 * kDeltaKeys, nqb * kDeltaKeys * 4);
  // this thread's means of block blk0 + sb
  auto load_means = [&](float (&x)[CPT], int blk0) {
#pragma unroll
    for (int i = 0; i < CPT; i += 4) {
      const v4i u = __builtin_amdgcn_raw_buffer_load_b128(qrs, ((blk0 + sb) * D + sc + i) * 4, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[i + e] = __int_as_float(u[e]);
    }
  };
  // stage the means in x (one chunk) into buffer buf: split pieces and dot
  // products with k_mean
  // causal attention reads tile kt only for query blocks whose last query can
  // see one of its keys (32 blk + 31 >= 128 kt, i.e. blk >= 4 kt); the tile's
  // other rows are left unwritten (chunks start at a multiple of 32 blocks)
  const int first = a.causal ? min(kt * (kDeltaKeys / kBlkQ), nqb) & ~31 : 0;
  int blk0_of_buf[2] = {first, first + 32};  // the first query block of the chunk staged in each buffer
  auto stage = [&](const float (&x)[CPT], int buf) {
    float c = 0.0f, sa = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      c = __builtin_fmaf(x[i], km[i], c);
      sa += fabsf(x[i]);
    }
    c += __shfl_xor(c, 1, 64);
    c += __shfl_xor(c, 2, 64);
    c += __shfl_xor(c, 4, 64);
    if constexpr (INTU) {
      sa += __shfl_xor(sa, 1, 64);
      sa += __shfl_xor(sa, 2, 64);
      sa += __shfl_xor(sa, 4, 64);
    }
    if ((tid & 7) == 0) {
      cs[buf][sb] = c;
      if constexpr (INTU) {
        const int blk = blk0_of_buf[buf] + sb;
        cu[buf][sb] = blk < nqb ? smooth_q_unit(a.q_scale[qblk0 + blk], sa) : 0.0f;
      }
    }
    uint16_t p[CPT][NS];
#pragma unroll
    for (int i = 0; i < CPT; ++i) M::split(x[i], p[i]);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp)
#pragma unroll
      for (int i = 0; i < CPT; i += 8) {
        v4i u;
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = (int)((uint32_t)p[i + 2 * j][sp] | ((uint32_t)p[i + 2 * j + 1][sp] << 16));
        *reinterpret_cast<v4i *>(&am[buf][sp][sb * RS + sc + i]) = u;
      }
  };
  // chunk blk0 from buffer buf: MFMAs and stores
  auto compute = [&](int blk0, int buf) {
    // D[key][block] = K rows (A) . split means (B): the lane's column is query
    // block blk0 + lane % 32, its rows the keys key0 + 8 g + 4 hh + 0..3 (g < 4)
    v16f acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) {
        const v4i u = *reinterpret_cast<const v4i *>(&am[buf][sp][(lane & 31) * RS + 16 * s + 8 * hh]);
        acc = M::mfma(kf[s], __builtin_bit_cast(T8, u), acc);
      }
    // row blk0 + lane % 32 of the tile (a store past the last block is dropped)
    const float c = cs[buf][lane & 31];
    float inv = 0.0f;
    if constexpr (INTU) {  // this wavefront's 32 keys lie in one 64-key K block
      const float unit = cu[buf][lane & 31] * a.k_scale[(ks.row0 + key0) >> 6];
      inv = unit > 0.0f ? 1.0f / unit : 0.0f;
    }
    const int row = (blk0 + (lane & 31)) * kDeltaKeys + 32 * wave + 4 * hh;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int k0 = key0 + 8 * g + 4 * hh;
      v4i o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = k0 + e < S ? acc[4 * g + e] - c : 0.0f;  // padding keys: 0
        o[e] = INTU ? (int)__builtin_rintf(d * inv) : __float_as_int(d);
      }
      __builtin_amdgcn_raw_buffer_store_b128(o, drs, (row + 8 * g) * 4, 0, 0);
    }
  };
  // Chunk c is computed from buffer c % 2 while the means of chunk c + 2 load
  // (two register sets, so a load has two chunks' time to arrive; past the last
  // chunk they read as zeros and are not used).  Chunk c + 1 is staged into the
  // other buffer after chunk c's stores; that buffer's last readers (chunk c - 1)
  // are past chunk c's barrier.
  float xa[CPT], xb[CPT];
  load_means(xa, first);
  load_means(xb, first + 32);
  stage(xa, 0);
  for (int blk0 = first; blk0 < nqb; blk0 += 64) {
    __syncthreads();
    load_means(xa, blk0 + 64);
    compute(blk0, 0);
    if (blk0 + 32 >= nqb) break;
    blk0_of_buf[1] = blk0 + 32;
    stage(xb, 1);
    __syncthreads();
    load_means(xb, blk0 + 96);
    compute(blk0 + 32, 1);
    blk0_of_buf[0] = blk0 + 64;
    if (blk0 + 64 < nqb) stage(xa, 0);
  }
}

// ---------------------------------------------------------------------------
// INT8 quantisation of one 32-token block of Q: one scale for the block, or
// (LANE) one scale per token -- the query a lane column holds in the 32 x 32
// INT8 MFMA layout of the attention kernel (per-token granularity of Q and K
// uses the same Q pass) -- or (HEAD) the head's one scale, from the abs-max
// that the per-head reduction left in the block's slot.
// ---------------------------------------------------------------------------
template <int DT, int D, bool LANE, bool HEAD = false>
__device__ inline void qquant_wg(const QuantQKArgs &a, int wg) {
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x;
  int b, h, blk;
  block_of(a.varlen, a.sq, a.B, a.H, a.nq, a.rows_q, kBlkQ, kBlkQ, wg, b, h, blk);
  const Seg hv = q_seg<D>(a, b, h);
  if (blk >= ceil_div(hv.S, kBlkQ)) return;  // past this sequence's blocks (packed batches)
  const uint16_t *q = (const uint16_t *)a.q;
  constexpr int vec_per_row = D / 8;
  constexpr int nvec = kBlkQ * vec_per_row;  // <= 512: at most 2 per thread
  float x[2][8];
  float amax = 0.0f, ramax[2] = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int vi = tid + u * kThreads;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    const int s = blk * kBlkQ + row;
    if (vi < nvec && s < hv.S) {
      load8<DT>(q + hv.base + (long long)s * hv.stride + c8, x[u]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
    }
  }
  if (a.q_mean) {  // smoothed Q: subtract the block's channel means
    q_block_smooth<D>(a, x, hv.S - blk * kBlkQ, (hv.row0 >> 5) + blk);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ramax[u] = fmaxf(ramax[u], fabsf(x[u][i]));
    amax = fmaxf(amax, ramax[u]);
  }
  float inv[2];
  if constexpr (LANE) {
    // a token's vec_per_row vectors sit in consecutive lanes of one wavefront
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int o = vec_per_row / 2; o >= 1; o >>= 1) ramax[u] = fmaxf(ramax[u], __shfl_xor(ramax[u], o, 64));
      inv[u] = ramax[u] > 0.0f ? 127.0f / ramax[u] : 0.0f;
      const int vi = tid + u * kThreads;
      if (vi < nvec && vi % vec_per_row == 0)
        a.q_scale[hv.row0 + blk * kBlkQ + vi / vec_per_row] = ramax[u] > 0.0f ? ramax[u] / 127.0f : 0.0f;
    }
  } else if constexpr (HEAD) {
    // the head's abs-max, left in this block's slot by the reduction pass; the
    // slot is overwritten with the scale once every thread has read it
    const long long slot = (hv.row0 >> 5) + blk;
    const float hm = a.q_scale[slot];
    inv[0] = inv[1] = hm > 0.0f ? 127.0f / hm : 0.0f;
    __syncthreads();
    if (tid == 0) a.q_scale[slot] = hm > 0.0f ? hm / 127.0f : 0.0f;
  } else {
    amax = block_max(amax, red);
    inv[0] = inv[1] = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (tid == 0) a.q_scale[(hv.row0 >> 5) + blk] = amax > 0.0f ? amax / 127.0f : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int vi = tid + u * kThreads;
    if (vi >= nvec) break;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= (uint32_t)(uint8_t)to_i8(x[u][i], inv[u]) << (8 * (i & 3));
    v2i out = {(int)w[0], (int)w[1]};
    *reinterpret_cast<v2i *>(a.q_i8 + (hv.row0 + blk * kBlkQ + row) * D + c8) = out;
  }
}
template <int DT, int D, bool LANE, bool HEAD = false>
__global__ __launch_bounds__(kThreads) void k_qquant(const QuantQKArgs a) {
  qquant_wg<DT, D, LANE, HEAD>(a, blockIdx.x);
}

// k_mean[bh][d] = fp32(sum over the head's chunk partials / S); thread = (K head bh, d).
// HEAD (per-head granularity): the head's max |K - k_mean| as well, formed
// from the chunks' channel max and min: fl(x - m) is monotone in x, so the
// largest |fl(K[s][d] - m)| over the tokens is fl(max_d - m) or fl(m - min_d);
// the D channels of a head are D consecutive threads of one work-group
// (256 = a multiple of D), and the head's value is left in each of its K
// block slots of k_scale for the K pass.
template <int D, bool HEAD = false>
__device__ inline void kmean_wg(const QuantQKArgs &a, int wg) {
  const long long i = (long long)wg * kThreads + threadIdx.x;
  const bool valid = i < (long long)a.B * a.H_kv * D;
  const int bh = (int)(i / D), d = (int)(i % D);
  float hmax = 0.0f;
  Seg sg{};
  if (valid) {
    sg = k_seg<D>(a, bh / a.H_kv, bh % a.H_kv);
    const double *part = reinterpret_cast<const double *>(a.k_i8 + sg.row0 * code_row_bytes<D>(a));
    const int nch = n_chunks(sg.S);
    double v[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) v[c] = c < nch ? part[(long long)c * D + d] : 0.0;  // all loads in flight
    double t = 0.0;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) t += v[c];
    const float m = sg.S > 0 ? (float)(t / (double)sg.S) : 0.0f;
    a.k_mean[i] = m;
    if (HEAD && sg.S > 0) {
      const float *mm = reinterpret_cast<const float *>(part + (long long)nch * D);
      float mx = -INFINITY, mn = INFINITY;
      for (int c = 0; c < nch; ++c) {
        mx = fmaxf(mx, mm[(2LL * c) * D + d]);
        mn = fminf(mn, mm[(2LL * c + 1) * D + d]);
      }
      hmax = fmaxf(mx - m, m - mn);
    }
  }
  if constexpr (HEAD) {
    __shared__ float hm[kThreads];
    const int tid = threadIdx.x;
    hm[tid] = hmax;
    __syncthreads();
    const int h0 = tid - d;  // the head's first thread in this work-group
    float r = 0.0f;
    for (int c = 0; c < D; ++c) r = fmaxf(r, hm[h0 + c]);
    if (valid) {
      const int nslot = ceil_div(sg.S, kKvPad) * (kKvPad / kBlkK);  // the K pass's blocks of this head
      for (int blk = d; blk < nslot; blk += D) a.k_scale[(sg.row0 >> 6) + blk] = r;
    }
  }
}
template <int D, bool HEAD>
__global__ __launch_bounds__(kThreads) void k_kmean(const QuantQKArgs a) { kmean_wg<D, HEAD>(a, blockIdx.x); }

// ---------------------------------------------------------------------------
// Pass 2: INT8 quantisation of one 64-token block of K - k_mean: one scale for
// the block (QK 0), or (QK 1, LANE) one per 16-key lane group -- the keys one
// half of a wavefront holds of each 32-key sub-tile in the attention kernel's
// 32 x 32 MFMA result, group 2 * (n / 32) + bit 2 of n (4 groups per block) --
// or (QK 3, TOKEN) one per token, or (QK 4, HEAD) the head's one scale, from
// the abs-max that the mean pass left in the block's slot.
// ---------------------------------------------------------------------------
__device__ inline int lane_group_in_block(int row) { return 2 * (row >> 5) + ((row >> 2) & 1); }

template <int DT, int D, int QK>
__device__ inline void kquant_wg(const QuantQKArgs &a, int wg) {
  constexpr bool LANE = QK == 1, TOKEN = QK == 3, HEAD = QK == 4;
  __shared__ float red[4][kThreads / 64];
  __shared__ float mean[D];
  const int tid = threadIdx.x;
  int b, h, blk;
  block_of(a.varlen, a.sk, a.B, a.H_kv, a.nk, a.rows_k, kKvPad, kBlkK, wg, b, h, blk);
  const int bh = b * a.H_kv + h;  // K head (b, h_kv)
  const Seg hv = k_seg<D>(a, b, h);
  if (blk >= ceil_div(hv.S, kKvPad) * (kKvPad / kBlkK)) return;  // past this sequence's rows
  const uint16_t *k = (const uint16_t *)a.k;
  if (tid < D) mean[tid] = a.k_mean[(long long)bh * D + tid];
  __syncthreads();
  constexpr int vec_per_row = D / 8;
  constexpr int nvec = kBlkK * vec_per_row;  // <= 1024: at most 4 per thread
  float x[4][8];
  float amax = 0.0f, gmax[4] = {0.0f, 0.0f, 0.0f, 0.0f}, rmax[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int vi = tid + u * kThreads;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    const int s = blk * kBlkK + row;
    if (vi < nvec && s < hv.S) {
      load8<DT>(k + hv.base + (long long)s * hv.stride + c8, x[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = x[u][i] - mean[c8 + i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[u][i]));
    amax = fmaxf(amax, m);
    rmax[u] = m;
    if (LANE && vi < nvec) {
      const int g = lane_group_in_block(row);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) gmax[gg] = g == gg ? fmaxf(gmax[gg], m) : gmax[gg];
    }
  }
  float inv[4];
  if constexpr (LANE) {
    const int w = tid >> 6;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float r = wave_max(gmax[g]);
      if ((tid & 63) == 0) red[g][w] = r;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float r = red[g][0];
#pragma unroll
      for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[g][i]);
      gmax[g] = r;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (tid + u * kThreads) / vec_per_row;
      const int g = lane_group_in_block(row & (kBlkK - 1));
      float m = gmax[0];
#pragma unroll
      for (int gg = 1; gg < 4; ++gg) m = g == gg ? gmax[gg] : m;
      inv[u] = m > 0.0f ? 127.0f / m : 0.0f;
    }
    if (tid < 4) {
      float m = gmax[0];
#pragma unroll
      for (int gg = 1; gg < 4; ++gg) m = tid == gg ? gmax[gg] : m;
      a.k_scale[(hv.row0 >> 4) + 4 * blk + tid] = m > 0.0f ? m / 127.0f : 0.0f;
    }
  } else if constexpr (TOKEN) {
    // a token's vec_per_row vectors sit in consecutive lanes of one wavefront
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int o = vec_per_row / 2; o >= 1; o >>= 1) rmax[u] = fmaxf(rmax[u], __shfl_xor(rmax[u], o, 64));
      inv[u] = rmax[u] > 0.0f ? 127.0f / rmax[u] : 0.0f;
      const int vi = tid + u * kThreads;
      if (vi < nvec && vi % vec_per_row == 0)
        a.k_scale[hv.row0 + blk * kBlkK + vi / vec_per_row] = rmax[u] > 0.0f ? rmax[u] / 127.0f : 0.0f;
    }
  } else if constexpr (HEAD) {
    // the head's abs-max, left in this block's slot by the mean pass; the slot
    // is overwritten with the scale once every thread has read it
    const long long slot = (hv.row0 >> 6) + blk;
    const float hm = a.k_scale[slot];
#pragma unroll
    for (int u = 0; u < 4; ++u) inv[u] = hm > 0.0f ? 127.0f / hm : 0.0f;
    __syncthreads();
    if (tid == 0) a.k_scale[slot] = hm > 0.0f ? hm / 127.0f : 0.0f;
  } else {
    amax = block_max(amax, red[0]);
#pragma unroll
    for (int u = 0; u < 4; ++u) inv[u] = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (tid == 0) a.k_scale[(hv.row0 >> 6) + blk] = amax > 0.0f ? amax / 127.0f : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int vi = tid + u * kThreads;
    if (vi >= nvec) break;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= (uint32_t)(uint8_t)to_i8(x[u][i], inv[u]) << (8 * (i & 3));
    v2i out = {(int)w[0], (int)w[1]};
    *reinterpret_cast<v2i *>(a.k_i8 + (hv.row0 + blk * kBlkK + row) * D + c8) = out;
  }
}
template <int DT, int D, int QK>
__global__ __launch_bounds__(kThreads) void k_kquant(const QuantQKArgs a) { kquant_wg<DT, D, QK>(a, blockIdx.x); }

// ---------------------------------------------------------------------------
// MXFP4 quantisation of one block of ROWS tokens (32 of Q, or 64 of K - k_mean):
// every 32-channel block of a token shares an E8M0 scale 2^e,
// e = floor(log2(amax)) - 2 clamped to [-127, 127] (-127 when amax = 0), and
// its values become E2M1(x / 2^e), round to nearest even, saturating at 6
// (the OCP Microscaling shared-exponent rule; the FP4 micro-scaling of the
// "Kairos" guide, section 2.2).  A thread converts 8 consecutive channels; the
// 4 threads of a 32-channel block are consecutive lanes.
// ---------------------------------------------------------------------------
__device__ inline uint32_t e2m1_code(float y) {  // y = x / 2^e, |y| < 8
  const float v = fabsf(y);
  const uint32_t m = v <= 0.25f ? 0u : v < 0.75f ? 1u : v <= 1.25f ? 2u : v < 1.75f ? 3u
                     : v <= 2.5f ? 4u : v < 3.5f ? 5u : v <= 5.0f ? 6u : 7u;  // ties to the even neighbour
  return m | (y < 0.0f ? 8u : 0u);
}

__device__ inline int mx_exponent(float amax) {  // floor(log2(amax)) - 2, clamped; amax >= 0
  if (amax == 0.0f) return -127;
  const uint32_t b = __float_as_uint(amax);
  const int ex = (int)(b >> 23);
  const int fl = ex ? ex - 127 : 31 - __builtin_clz(b & 0x7fffffu) - 149;  // subnormal: leading mantissa bit
  return min(max(fl - 2, -127), 127);
}

template <int DT, int D, bool IS_K>
__device__ inline void mxfp4_wg(const QuantQKArgs &a, int wg) {
  constexpr int ROWS = IS_K ? kBlkK : kBlkQ;
  constexpr int vec_per_row = D / 8;
  constexpr int nvec = ROWS * vec_per_row;
  constexpr int U = (nvec + kThreads - 1) / kThreads;
  __shared__ float mean[D];
  const int tid = threadIdx.x;
  const int hn = IS_K ? a.H_kv : a.H;
  int b, h, blk;
  if (IS_K) block_of(a.varlen, a.sk, a.B, hn, a.nk, a.rows_k, kKvPad, kBlkK, wg, b, h, blk);
  else block_of(a.varlen, a.sq, a.B, hn, a.nq, a.rows_q, kBlkQ, kBlkQ, wg, b, h, blk);
  const int bh = b * hn + h;
  const Seg hv = IS_K ? k_seg<D>(a, b, h) : q_seg<D>(a, b, h);
  if (IS_K ? blk >= ceil_div(hv.S, kKvPad) * (kKvPad / kBlkK) : blk >= ceil_div(hv.S, kBlkQ)) return;
  if (IS_K) {
    if (tid < D) mean[tid] = a.k_mean[(long long)bh * D + tid];
    __syncthreads();
  }
  const uint16_t *x = (const uint16_t *)(IS_K ? a.k : a.q);
  uint8_t *codes = reinterpret_cast<uint8_t *>(IS_K ? a.k_i8 : a.q_i8);
  uint8_t *scales = reinterpret_cast<uint8_t *>(IS_K ? a.k_scale : a.q_scale);
  // Q: both row vectors of the thread first (U <= 2), so that smoothed Q can
  // subtract the block's channel means before the E2M1 rule
  float xq[2][8];
  if constexpr (!IS_K) {
    static_assert(U <= 2, "a Q block is at most two vectors a thread");
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int vi = tid + u * kThreads;
      const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
      const int s = blk * ROWS + row;
      if (vi < nvec && s < hv.S) {
        load8<DT>(x + hv.base + (long long)s * hv.stride + c8, xq[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xq[u][i] = 0.0f;
      }
    }
    if (a.q_mean) q_block_smooth<D>(a, xq, hv.S - blk * kBlkQ, (hv.row0 >> 5) + blk);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = tid + u * kThreads;  // uniform over the wavefront: nvec is a multiple of 64
    if (vi >= nvec) break;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    const int s = blk * ROWS + row;
    float v[8];
    if constexpr (!IS_K) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = xq[u][i];
    } else if (s < hv.S) {
      load8<DT>(x + hv.base + (long long)s * hv.stride + c8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] - mean[c8 + i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int e = mx_exponent(amax);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= e2m1_code(__builtin_ldexpf(v[i], -e)) << (4 * i);
    const long long r = hv.row0 + (long long)blk * ROWS + row;
    *reinterpret_cast<uint32_t *>(codes + r * (D / 2) + c8 / 2) = w;
    if (c8 % 32 == 0) scales[r * (D / 32) + c8 / 32] = (uint8_t)(e + 127);
  }
}
template <int DT, int D, bool IS_K>
__global__ __launch_bounds__(kThreads) void k_mxfp4(const QuantQKArgs a) { mxfp4_wg<DT, D, IS_K>(a, blockIdx.x); }

// ---------------------------------------------------------------------------
// V, four short launches:
//   k_vamax_part   per (head, chunk): channel abs-max partials -> v_fp8 region
//                  (smoothing: k_vstats_part, channel sum, max and min)
//   k_vamax        per (head, channel): v_scale <- amax (held there until the end)
//                  (smoothing: v_mean <- mean, v_scale <- amax of V - mean)
//   k_vconvert     per (head, 64-key tile): E4M3 codes in the tiled key order
//   k_vscale       per (head, channel): v_scale <- amax / 448
// V smoothing ("SageAttention2" summary, SageAttention2方法: optional smooth V)
// quantises V - mean with mean = the channel mean over the head's tokens (the
// K-smoothing statistic).  Its abs-max needs no second pass over V: fp32
// subtraction is monotonic and symmetric, so max_s |fl(V[s] - mean)| =
// max(fl(max V - mean), fl(mean - min V)).
// ---------------------------------------------------------------------------
// Channel sum (binary64), max and min of one chunk -> partials at 16 D bytes
// per chunk: [D doubles | D floats | D floats].
template <int DT, int D>
__device__ inline void chunk_stats(const uint16_t *x, const Seg &hv, int chunk, uint8_t *partials) {
  using M = ChunkMap<D>;
  __shared__ double psum[M::R][D];
  __shared__ float pmax[M::R][D], pmin[M::R][D];
  const int tid = threadIdx.x, g = tid % M::G, r = tid / M::G;
  const int S = hv.S;
  const int ct = chunk_tokens(S);
  const int s_end = min(S, (chunk + 1) * ct);
  double sum[8];
  float mx[8], mn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sum[i] = 0.0;
    mx[i] = -INFINITY;
    mn[i] = INFINITY;
  }
  for (int s0 = chunk * ct + r; s0 < s_end; s0 += M::R * M::kUnroll) {
    v4i raw[M::kUnroll];  // 16-bit pairs as loaded
    bool ok[M::kUnroll];
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u) {
      const int s = s0 + u * M::R;
      ok[u] = s < s_end;
      raw[u] = ok[u] ? *reinterpret_cast<const v4i *>(x + hv.base + (long long)s * hv.stride + 8 * g)
                     : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < M::kUnroll; ++u)
      if (ok[u])
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = in_to_f32<DT>(i & 1 ? (uint32_t)raw[u][i >> 1] >> 16 : (uint32_t)raw[u][i >> 1] & 0xffffu);
          sum[i] += (double)v;
          mx[i] = fmaxf(mx[i], v);
          mn[i] = fminf(mn[i], v);
        }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    psum[r][8 * g + i] = sum[i];
    pmax[r][8 * g + i] = mx[i];
    pmin[r][8 * g + i] = mn[i];
  }
  __syncthreads();
  if (tid < D) {
    double t = psum[0][tid];
    float a = pmax[0][tid], b = pmin[0][tid];
    for (int rr = 1; rr < M::R; ++rr) {
      t += psum[rr][tid];
      a = fmaxf(a, pmax[rr][tid]);
      b = fminf(b, pmin[rr][tid]);
    }
    uint8_t *base = partials + (long long)chunk * 16 * D;
    reinterpret_cast<double *>(base)[tid] = t;
    reinterpret_cast<float *>(base + 8 * D)[tid] = a;
    reinterpret_cast<float *>(base + 12 * D)[tid] = b;
  }
}

template <int DT, int D>
__device__ inline void vstats_part_wg(const QuantVArgs &a, int wg) {
  const int nch = chunk_grid(a.varlen ? a.sk.max_len : a.S);
  const int bh = wg / nch, chunk = wg % nch;
  const Seg sg = v_seg<D>(a, bh / a.H, bh % a.H);
  if (chunk >= n_chunks(sg.S)) return;
  chunk_stats<DT, D>((const uint16_t *)a.v, sg, chunk, v_partials(a, sg, D));
}
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void k_vstats_part(const QuantVArgs a) { vstats_part_wg<DT, D>(a, blockIdx.x); }

template <int DT, int D>
__device__ inline void vamax_part_wg(const QuantVArgs &a, int wg) {
  const int nch = chunk_grid(a.varlen ? a.sk.max_len : a.S);
  const int bh = wg / nch, chunk = wg % nch;
  const Seg sg = v_seg<D>(a, bh / a.H, bh % a.H);
  if (chunk >= n_chunks(sg.S)) return;
  chunk_reduce<DT, D, true>((const uint16_t *)a.v, sg, chunk, v_partials(a, sg, D));
}
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void k_vamax_part(const QuantVArgs a) { vamax_part_wg<DT, D>(a, blockIdx.x); }

template <int D>
__device__ inline void vamax_wg(const QuantVArgs &a, int wg) {
  const long long i = (long long)wg * kThreads + threadIdx.x;
  if (i >= (long long)a.B * a.H * D) return;
  const int bh = (int)(i / D), d = (int)(i % D);
  const Seg sg = v_seg<D>(a, bh / a.H, bh % a.H);
  const int nch = n_chunks(sg.S);
  if (a.v_mean) {  // smoothing: combine sums, maxima and minima
    const uint8_t *base = v_partials(a, sg, D);
    double t = 0.0;
    float hi = -INFINITY, lo = INFINITY;
    for (int c = 0; c < nch; ++c) {
      const uint8_t *pc = base + (long long)c * 16 * D;
      t += reinterpret_cast<const double *>(pc)[d];
      hi = fmaxf(hi, reinterpret_cast<const float *>(pc + 8 * D)[d]);
      lo = fminf(lo, reinterpret_cast<const float *>(pc + 12 * D)[d]);
    }
    const float mean = sg.S > 0 ? (float)(t / (double)sg.S) : 0.0f;
    a.v_mean[i] = mean;
    a.v_scale[i] = sg.S > 0 ? fmaxf(hi - mean, mean - lo) : 0.0f;
    return;
  }
  const float *part = reinterpret_cast<const float *>(v_partials(a, sg, D));
  float v[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) v[c] = c < nch ? part[(long long)c * D + d] : 0.0f;
  float m = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) m = fmaxf(m, v[c]);
  a.v_scale[i] = m;
}
template <int D>
__global__ __launch_bounds__(kThreads) void k_vamax(const QuantVArgs a) { vamax_wg<D>(a, blockIdx.x); }

// One 64-key tile of one head: thread (q, g) converts keys 4q .. 4q + 3 of
// channels 8g .. 8g + 7.  The four keys are consecutive in the tile's key
// order (key_vpos(4q + i) = key_vpos(4q) + i), so each channel's four codes
// form one 32-bit word of the channel's 64-byte row; the 16 threads of a
// channel group together write whole rows.
template <int DT, int D>
__device__ inline void vconvert_wg(const QuantVArgs &a, int wg, int tid) {
  const int q = tid & 15, g = tid >> 4;
  int b, h, t;
  block_of(a.varlen, a.sk, a.B, a.H, a.nk, a.rows_k, kKvPad, kBlkK, wg, b, h, t);
  const int bh = b * a.H + h;
  const Seg hv = v_seg<D>(a, b, h);
  if (t >= ceil_div(hv.S, kKvPad) * (kKvPad / kBlkK)) return;  // past this sequence's tiles
  const uint16_t *v = (const uint16_t *)a.v;
  float inv[8], mean[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float m = a.v_scale[(long long)bh * D + 8 * g + i];  // the channel's amax at this point
    inv[i] = m > 0.0f ? 448.0f / m : 0.0f;
    mean[i] = a.v_mean ? a.v_mean[(long long)bh * D + 8 * g + i] : 0.0f;
  }
  float x[4][8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = t * kBlkK + 4 * q + k;
    if (s < hv.S) {
      load8<DT>(v + hv.base + (long long)s * hv.stride + 8 * g, x[k]);
      if (a.v_mean)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[k][i] = x[k][i] - mean[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[k][i] = 0.0f;
    }
  }
  uint8_t *dst = a.v_fp8 + (((hv.row0 >> 6) + t) * D + 8 * g) * kBlkK + key_vpos(4 * q);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = fminf(fmaxf(x[k][i] * inv[i], -448.0f), 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
    *reinterpret_cast<int *>(dst + i * kBlkK) = w;
  }
}
template <int DT, int D>
__global__ __launch_bounds__(2 * D) void k_vconvert(const QuantVArgs a) { vconvert_wg<DT, D>(a, blockIdx.x, threadIdx.x); }

// ---------------------------------------------------------------------------
// V for the micro-scaled FP4 P~ V product: one work-group per 64-key block of a
// head.  The block's 16-bit rows are staged in LDS (coalesced 16-byte loads);
// thread (d, half) then gathers channel d of the 32 keys of its key group --
// the keys SAGE_VPOS_KEY(32 half + i), i = 0..31, i.e. those whose offset has
// bit 2 equal to `half`, in the order the attention kernel holds P~ -- takes
// the group's MX exponent e = floor(log2 amax) - 2 (clamped to [-127, 127]),
// and writes the 32 E2M1 codes of x / 2^e as 16 bytes (code of position 2u in
// the low nibble of byte u) and the E8M0 byte e + 127.  Keys past the sequence
// count as 0.  With V smoothing the channel means (from the statistics passes)
// are subtracted first.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(2 * D) void k_v4convert(const QuantVArgs a) {
  constexpr int RS = D + 8;  // LDS row stride in 16-bit elements (16-byte aligned rows, banks offset)
  __shared__ __attribute__((aligned(16))) uint16_t tile[kBlkK][RS];
  const int tid = threadIdx.x;
  int b, h, t;
  block_of(a.varlen, a.sk, a.B, a.H, a.nk, a.rows_k, kKvPad, kBlkK, blockIdx.x, b, h, t);
  const int bh = b * a.H + h;
  const Seg hv = v_seg<D>(a, b, h);
  if (t >= ceil_div(hv.S, kKvPad) * (kKvPad / kBlkK)) return;  // past this sequence's blocks
  const uint16_t *v = (const uint16_t *)a.v;
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int ROUNDS = kBlkK * CPR / (2 * D);  // chunks a thread stages
#pragma unroll
  for (int u = 0; u < ROUNDS; ++u) {
    const int ci = tid + u * 2 * D, row = ci / CPR, c8 = (ci % CPR) * 8;
    const int s = t * kBlkK + row;
    const v4i x = s < hv.S ? *reinterpret_cast<const v4i *>(v + hv.base + (long long)s * hv.stride + c8)
                           : v4i{0, 0, 0, 0};
    *reinterpret_cast<v4i *>(&tile[row][c8]) = x;
  }
  __syncthreads();
  const int d = tid >> 1, half = tid & 1;
  const float mean = a.v_mean ? a.v_mean[(long long)bh * D + d] : 0.0f;
  float x[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int key = vpos_key(32 * half + i);
    const bool valid = t * kBlkK + key < hv.S;
    x[i] = valid ? in_to_f32<DT>(tile[key][d]) - mean : 0.0f;
    amax = fmaxf(amax, fabsf(x[i]));
  }
  const int e = mx_exponent(amax);
  v4i w = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i)
    w[i >> 3] |= (int)(e2m1_code(__builtin_ldexpf(x[i], -e)) << (4 * (i & 7)));
  const long long blk = (hv.row0 >> 6) + t;  // 64-key block of the head's buffer
  *reinterpret_cast<v4i *>(a.v_fp8 + (blk * D + d) * 32 + 16 * half) = w;
  a.v_e8m0[(blk * D + d) * 2 + half] = (uint8_t)(e + 127);
}

template <int D>
__device__ inline void vscale_wg(const QuantVArgs &a, int wg) {
  const long long i = (long long)wg * kThreads + threadIdx.x;
  if (i >= (long long)a.B * a.H * D) return;
  const float m = a.v_scale[i];
  a.v_scale[i] = m > 0.0f ? m / 448.0f : 0.0f;
}
template <int D>
__global__ __launch_bounds__(kThreads) void k_vscale(const QuantVArgs a) { vscale_wg<D>(a, blockIdx.x); }

template <int DT, int D>
static void launch_qk(const QuantQKArgs &a, hipStream_t stream) {
  const int bhk = a.B * a.H_kv;
  const int gd = (bhk * D + kThreads - 1) / kThreads;
  // per-block passes: every block of every (entry, head), or of each head's packed buffer
  const dim3 gq(a.varlen ? a.H * (int)(a.rows_q / kBlkQ) : a.B * a.H * a.nq);
  const dim3 gk(a.varlen ? a.H_kv * (int)(a.rows_k / kBlkK) : bhk * a.nk);
  const dim3 gs(bhk * chunk_grid(a.varlen ? a.sk.max_len : a.S));
  if (a.qk == 4) {  // per head: the heads' abs-max first, then the per-block passes
    hipLaunchKernelGGL((k_ksum<DT, D, true>), gs, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((k_qamax_part<DT, D>), dim3(a.B * a.H * chunk_grid(a.varlen ? a.sq.max_len : a.S)),
                       dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((k_qhead<D>), dim3(a.B * a.H), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((k_qquant<DT, D, false, true>), gq, dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((k_kmean<D, true>), dim3(gd), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((k_kquant<DT, D, 4>), gk, dim3(kThreads), 0, stream, a);
    return;
  }
  hipLaunchKernelGGL((k_ksum<DT, D, false>), gs, dim3(kThreads), 0, stream, a);
  if (a.qk == 2) hipLaunchKernelGGL((k_mxfp4<DT, D, false>), gq, dim3(kThreads), 0, stream, a);
  else if (a.qk == 1 || a.qk == 3) hipLaunchKernelGGL((k_qquant<DT, D, true>), gq, dim3(kThreads), 0, stream, a);
  else if (a.q_i8) hipLaunchKernelGGL((k_qquant<DT, D, false>), gq, dim3(kThreads), 0, stream, a);
  // (no Q codes: the attention kernel quantises Q itself)
  hipLaunchKernelGGL((k_kmean<D, false>), dim3(gd), dim3(kThreads), 0, stream, a);
  if (a.qk == 2) hipLaunchKernelGGL((k_mxfp4<DT, D, true>), gk, dim3(kThreads), 0, stream, a);
  else if (a.qk == 1) hipLaunchKernelGGL((k_kquant<DT, D, 1>), gk, dim3(kThreads), 0, stream, a);
  else if (a.qk == 3) hipLaunchKernelGGL((k_kquant<DT, D, 3>), gk, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL((k_kquant<DT, D, 0>), gk, dim3(kThreads), 0, stream, a);
}

template <int DT, int D>
static void launch_v(const QuantVArgs &a, hipStream_t stream) {
  const int bh = a.B * a.H;
  const int gd = (bh * D + kThreads - 1) / kThreads;
  const dim3 parts(bh * chunk_grid(a.varlen ? a.sk.max_len : a.S));
  if (a.v_mean) hipLaunchKernelGGL((k_vstats_part<DT, D>), parts, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL((k_vamax_part<DT, D>), parts, dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL((k_vamax<D>), dim3(gd), dim3(kThreads), 0, stream, a);
  const dim3 gv(a.varlen ? a.H * (int)(a.rows_k / kBlkK) : bh * a.nk);  // 64-key tiles, as the K blocks
  hipLaunchKernelGGL((k_vconvert<DT, D>), gv, dim3(2 * D), 0, stream, a);
  hipLaunchKernelGGL((k_vscale<D>), dim3(gd), dim3(kThreads), 0, stream, a);
}

// MXFP4 V: with smoothing, the channel statistics passes first (partials staged
// in the code buffer, the means written to v_mean, the abs-maxima -- unused
// here -- to the scale buffer, which the conversion then overwrites).
template <int DT, int D>
static void launch_v4(const QuantVArgs &a, hipStream_t stream) {
  const int bh = a.B * a.H;
  if (a.v_mean) {
    QuantVArgs s = a;
    s.v_scale = reinterpret_cast<float *>(a.v_e8m0);
    const int gd = (bh * D + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((k_vstats_part<DT, D>), dim3(bh * chunk_grid(a.varlen ? a.sk.max_len : a.S)), dim3(kThreads),
                       0, stream, s);
    hipLaunchKernelGGL((k_vamax<D>), dim3(gd), dim3(kThreads), 0, stream, s);
  }
  const dim3 gv(a.varlen ? a.H * (int)(a.rows_k / kBlkK) : bh * a.nk);
  hipLaunchKernelGGL((k_v4convert<DT, D>), gv, dim3(2 * D), 0, stream, a);
}

hipError_t launch_quant_v_fp4(const QuantVArgs &a, hipStream_t stream) {
  if (a.D == 64) {
    if (a.dtype == 0) launch_v4<0, 64>(a, stream);
    else launch_v4<1, 64>(a, stream);
  } else {
    if (a.dtype == 0) launch_v4<0, 128>(a, stream);
    else launch_v4<1, 128>(a, stream);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Q, K and V quantisation in four launches (sage_quantize_qkv): the passes of
// sage_smooth_quant_qk and sage_quant_v that do not depend on each other share
// a launch, each work-group taking one role by its index:
//   1. K chunk sums | V chunk statistics
//   2. Q quantisation | K means | V abs-max (and means) from the chunk partials
//   3. K quantisation | V FP8 conversion
//   4. V scales
// Per-head granularity moves Q: its chunk abs-max joins launch 1, the per-head
// reduction takes its place in launch 2, and Q quantisation joins launch 3.
// Every pass that overwrites a buffer holding chunk partials (K and V codes)
// runs in a later launch than the work-groups that read them.
// ---------------------------------------------------------------------------
template <int DT, int D, bool VSTATS, bool HEAD>
__global__ __launch_bounds__(kThreads) void k_qkv1(const QuantQKArgs a, const QuantVArgs v) {
  const int n_k = a.B * a.H_kv * chunk_grid(a.S);  // (V has as many chunks: H_kv heads)
  const int wg = blockIdx.x;
  if (wg < n_k) ksum_wg<DT, D, HEAD>(a, wg);
  else if (HEAD && wg >= 2 * n_k) qamax_part_wg<DT, D>(a, wg - 2 * n_k);
  else if constexpr (VSTATS) vstats_part_wg<DT, D>(v, wg - n_k);
  else vamax_part_wg<DT, D>(v, wg - n_k);
}

template <int DT, int D, int QK>
__global__ __launch_bounds__(kThreads) void k_qkv2(const QuantQKArgs a, const QuantVArgs v) {
  constexpr bool HEAD = QK == 4;
  // (no Q codes: the attention kernel quantises Q itself)
  const int n_q = !a.q_i8 ? 0 : HEAD ? a.B * a.H : a.B * a.H * a.nq, n_m = ceil_div(a.B * a.H_kv * D, kThreads);
  const int wg = blockIdx.x;
  if (wg < n_q) {
    if constexpr (QK == 2) mxfp4_wg<DT, D, false>(a, wg);
    else if constexpr (HEAD) qhead_wg<D>(a, wg);
    else qquant_wg<DT, D, QK == 1 || QK == 3>(a, wg);  // one scale per token (LANE, TOKEN)
  } else if (wg < n_q + n_m) {
    kmean_wg<D, HEAD>(a, wg - n_q);
  } else {
    vamax_wg<D>(v, wg - n_q - n_m);
  }
}

template <int DT, int D, int QK>
__global__ __launch_bounds__(kThreads) void k_qkv3(const QuantQKArgs a, const QuantVArgs v) {
  constexpr int TPW = kThreads / (2 * D);  // 64-key V tiles a work-group converts (2 D threads each)
  const int n_k = a.B * a.H_kv * a.nk, n_v = ceil_div(v.B * v.H * v.nk, TPW);
  const int wg = blockIdx.x;
  if (wg < n_k) {
    if constexpr (QK == 2) mxfp4_wg<DT, D, true>(a, wg);
    else kquant_wg<DT, D, QK>(a, wg);
  } else if (QK == 4 && wg >= n_k + n_v) {
    qquant_wg<DT, D, false, true>(a, wg - n_k - n_v);  // per head: Q after its reduction
  } else {
    const int t = (wg - n_k) * TPW + (int)threadIdx.x / (2 * D);
    if (t < v.B * v.H * v.nk) vconvert_wg<DT, D>(v, t, (int)threadIdx.x % (2 * D));
  }
}

template <int DT, int D, int QK>
static void launch_qkv3(const QuantQKArgs &a, const QuantVArgs &v, hipStream_t st) {
  const int bhk = a.B * a.H_kv, gm = (bhk * D + kThreads - 1) / kThreads;
  constexpr int TPW = kThreads / (2 * D);
  const int nq = a.q_i8 ? a.B * a.H * a.nq : 0;  // Q blocks (none: the attention kernel quantises Q)
  hipLaunchKernelGGL((k_qkv2<DT, D, QK>), dim3((QK == 4 ? a.B * a.H : nq) + 2 * gm), dim3(kThreads), 0, st, a, v);
  hipLaunchKernelGGL((k_qkv3<DT, D, QK>), dim3(bhk * a.nk + (bhk * v.nk + TPW - 1) / TPW + (QK == 4 ? nq : 0)),
                     dim3(kThreads), 0, st, a, v);
}

template <int DT, int D>
static void launch_qkv(const QuantQKArgs &a, const QuantVArgs &v, hipStream_t st) {
  const int bhk = a.B * a.H_kv, gm = (bhk * D + kThreads - 1) / kThreads;
  // K chunks, then as many V chunks (V has H_kv heads), then (per head) the Q chunks
  const dim3 g1(2 * bhk * chunk_grid(a.S) + (a.qk == 4 ? a.B * a.H * chunk_grid(a.S) : 0));
  if (a.qk == 4) {
    if (v.v_mean) hipLaunchKernelGGL((k_qkv1<DT, D, true, true>), g1, dim3(kThreads), 0, st, a, v);
    else hipLaunchKernelGGL((k_qkv1<DT, D, false, true>), g1, dim3(kThreads), 0, st, a, v);
  } else {
    if (v.v_mean) hipLaunchKernelGGL((k_qkv1<DT, D, true, false>), g1, dim3(kThreads), 0, st, a, v);
    else hipLaunchKernelGGL((k_qkv1<DT, D, false, false>), g1, dim3(kThreads), 0, st, a, v);
  }
  if (a.qk == 4) launch_qkv3<DT, D, 4>(a, v, st);
  else if (a.qk == 2) launch_qkv3<DT, D, 2>(a, v, st);
  else if (a.qk == 1) launch_qkv3<DT, D, 1>(a, v, st);
  else if (a.qk == 3) launch_qkv3<DT, D, 3>(a, v, st);
  else launch_qkv3<DT, D, 0>(a, v, st);
  hipLaunchKernelGGL((k_vscale<D>), dim3(gm), dim3(kThreads), 0, st, v);
}

hipError_t launch_quantize_qkv(const QuantQKArgs &a, const QuantVArgs &v, hipStream_t stream) {
  if (a.D == 64) {
    if (a.dtype == 0) launch_qkv<0, 64>(a, v, stream);
    else launch_qkv<1, 64>(a, v, stream);
  } else {
    if (a.dtype == 0) launch_qkv<0, 128>(a, v, stream);
    else launch_qkv<1, 128>(a, v, stream);
  }
  return hipGetLastError();
}

hipError_t launch_smooth_quant_qk(const QuantQKArgs &a, hipStream_t stream) {
  if (a.D == 64) {
    if (a.dtype == 0) launch_qk<0, 64>(a, stream);
    else launch_qk<1, 64>(a, stream);
  } else {
    if (a.dtype == 0) launch_qk<0, 128>(a, stream);
    else launch_qk<1, 128>(a, stream);
  }
  return hipGetLastError();
}

template <bool INTU>
static void launch_qk_delta_t(const QuantQKArgs &a, float *delta, hipStream_t stream) {
  // S_k, rows_k: multiples of 128
  const dim3 grid(a.varlen ? a.H * (int)(a.rows_k / kDeltaKeys) : a.B * a.H * (a.S_k / kDeltaKeys));
  if (a.D == 64) {
    if (a.dtype == 0) hipLaunchKernelGGL((k_qk_delta<0, 64, INTU>), grid, dim3(kThreads), 0, stream, a, delta);
    else hipLaunchKernelGGL((k_qk_delta<1, 64, INTU>), grid, dim3(kThreads), 0, stream, a, delta);
  } else {
    if (a.dtype == 0) hipLaunchKernelGGL((k_qk_delta<0, 128, INTU>), grid, dim3(kThreads), 0, stream, a, delta);
    else hipLaunchKernelGGL((k_qk_delta<1, 128, INTU>), grid, dim3(kThreads), 0, stream, a, delta);
  }
}

hipError_t launch_qk_delta(const QuantQKArgs &a, float *delta, hipStream_t stream) {
  if (a.qk == 0) launch_qk_delta_t<true>(a, delta, stream);
  else launch_qk_delta_t<false>(a, delta, stream);
  return hipGetLastError();
}

hipError_t launch_quant_v(const QuantVArgs &a, hipStream_t stream) {
  if (a.D == 64) {
    if (a.dtype == 0) launch_v<0, 64>(a, stream);
    else launch_v<1, 64>(a, stream);
  } else {
    if (a.dtype == 0) launch_v<0, 128>(a, stream);
    else launch_v<1, 128>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace sage
