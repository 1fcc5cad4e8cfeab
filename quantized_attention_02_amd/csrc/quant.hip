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
#include "sage_impl.h"

#pragma clang fp contract(off)

namespace sage {

static_assert(vpos_key(key_vpos(0)) == 0 && vpos_key(key_vpos(37)) == 37 && vpos_key(key_vpos(63)) == 63,
              "V tile key order must be a bijection");

constexpr int kThreads = 256;
constexpr int kSliceCh = 32;  // channels per work-group in the column passes (64 B of a 16-bit row)

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
// Pass 1 (one launch, two roles by blockIdx):
//   [0, B*H*D/32)        channel sums of K over all S tokens -> k_mean
//   [B*H*D/32, + B*H*nq) INT8 quantisation of one 32-token block of Q
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_kmean_qquant(const QuantQKArgs a) {
  __shared__ double part[kThreads][8];
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x;
  const int nslice = a.D / kSliceCh;
  const int nsum = a.B * a.H * nslice;
  const uint16_t *q = (const uint16_t *)a.q, *k = (const uint16_t *)a.k;

  if ((int)blockIdx.x < nsum) {
    // ---- K channel mean: thread = (row offset tid/4, 8-channel group tid%4)
    const int bh = blockIdx.x / nslice, slice = blockIdx.x % nslice;
    const int b = bh / a.H, h = bh % a.H;
    const HeadView hv = head_view(a.layout, b, h, a.H, a.S, a.D);
    const int grp = tid & 3, r0 = tid >> 2;
    const int d0 = slice * kSliceCh + grp * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s = r0; s < a.S; s += kThreads / 4) {
      float x[8];
      load8<DT>(k + hv.base + (long long)s * hv.tok_stride + d0, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += (double)x[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[tid][i] = acc[i];
    __syncthreads();
    if (tid < kSliceCh) {
      const int g = tid >> 3, i = tid & 7;
      double s = 0.0;
      for (int r = 0; r < kThreads / 4; ++r) s += part[r * 4 + g][i];
      a.k_mean[(long long)bh * a.D + slice * kSliceCh + tid] = (float)(s / (double)a.S);
    }
    return;
  }

  // ---- Q block quantisation
  const int idx = blockIdx.x - nsum;
  const int bh = idx / a.nq, blk = idx % a.nq;
  const int b = bh / a.H, h = bh % a.H;
  const HeadView hv = head_view(a.layout, b, h, a.H, a.S, a.D);
  const int vec_per_row = a.D / 8;
  const int nvec = kBlkQ * vec_per_row;  // <= 512: at most 2 per thread
  float x[2][8];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int vi = tid + u * kThreads;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    const int s = blk * kBlkQ + row;
    if (vi < nvec && s < a.S) {
      load8<DT>(q + hv.base + (long long)s * hv.tok_stride + c8, x[u]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[u][i]));
  }
  amax = block_max(amax, red);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (tid == 0) a.q_scale[(long long)bh * a.nq + blk] = amax > 0.0f ? amax / 127.0f : 0.0f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int vi = tid + u * kThreads;
    if (vi >= nvec) break;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= (uint32_t)(uint8_t)to_i8(x[u][i], inv) << (8 * (i & 3));
    v2i out = {(int)w[0], (int)w[1]};
    *reinterpret_cast<v2i *>(a.q_i8 + ((long long)bh * a.S_q + blk * kBlkQ + row) * a.D + c8) = out;
  }
}

// ---------------------------------------------------------------------------
// Pass 2: INT8 quantisation of one 64-token block of K - k_mean.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_kquant(const QuantQKArgs a) {
  __shared__ float red[kThreads / 64];
  __shared__ float mean[128];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / a.nk, blk = blockIdx.x % a.nk;
  const int b = bh / a.H, h = bh % a.H;
  const HeadView hv = head_view(a.layout, b, h, a.H, a.S, a.D);
  const uint16_t *k = (const uint16_t *)a.k;
  if (tid < a.D) mean[tid] = a.k_mean[(long long)bh * a.D + tid];
  __syncthreads();
  const int vec_per_row = a.D / 8;
  const int nvec = kBlkK * vec_per_row;  // <= 1024: at most 4 per thread
  float x[4][8];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int vi = tid + u * kThreads;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    const int s = blk * kBlkK + row;
    if (vi < nvec && s < a.S) {
      load8<DT>(k + hv.base + (long long)s * hv.tok_stride + c8, x[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = x[u][i] - mean[c8 + i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[u][i]));
  }
  amax = block_max(amax, red);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (tid == 0) a.k_scale[(long long)bh * a.nk + blk] = amax > 0.0f ? amax / 127.0f : 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int vi = tid + u * kThreads;
    if (vi >= nvec) break;
    const int row = vi / vec_per_row, c8 = (vi % vec_per_row) * 8;
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= (uint32_t)(uint8_t)to_i8(x[u][i], inv) << (8 * (i & 3));
    v2i out = {(int)w[0], (int)w[1]};
    *reinterpret_cast<v2i *>(a.k_i8 + ((long long)bh * a.S_k + blk * kBlkK + row) * a.D + c8) = out;
  }
}

// ---------------------------------------------------------------------------
// V: one work-group per (head, 32-channel slice).  Pass A: channel amax over S.
// Pass B: per 64-key tile, convert to E4M3, transpose through LDS into the
// channel-major tile layout with the attention kernel's key order, and store
// the slice's 32 x 64 bytes with 16-byte vector stores.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_vquant(const QuantVArgs a) {
  __shared__ float pmax[kThreads][8];
  __shared__ float inv_s[kSliceCh];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kSliceCh * kBlkK];
  const int tid = threadIdx.x;
  const int nslice = a.D / kSliceCh;
  const int bh = blockIdx.x / nslice, slice = blockIdx.x % nslice;
  const int b = bh / a.H, h = bh % a.H;
  const HeadView hv = head_view(a.layout, b, h, a.H, a.S, a.D);
  const uint16_t *v = (const uint16_t *)a.v;
  const int grp = tid & 3, r0 = tid >> 2;  // 64 rows x 4 groups of 8 channels
  const int d0 = slice * kSliceCh + grp * 8;

  float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = r0; s < a.S; s += kThreads / 4) {
    float x[8];
    load8<DT>(v + hv.base + (long long)s * hv.tok_stride + d0, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(x[i]));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) pmax[tid][i] = mx[i];
  __syncthreads();
  if (tid < kSliceCh) {
    const int g = tid >> 3, i = tid & 7;
    float m = 0.0f;
    for (int r = 0; r < kThreads / 4; ++r) m = fmaxf(m, pmax[r * 4 + g][i]);
    inv_s[tid] = m > 0.0f ? 448.0f / m : 0.0f;
    a.v_scale[(long long)bh * a.D + slice * kSliceCh + tid] = m > 0.0f ? m / 448.0f : 0.0f;
  }
  __syncthreads();
  float inv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) inv[i] = inv_s[grp * 8 + i];

  const int pos = key_vpos(r0);
  for (int t = 0; t < a.nk; ++t) {
    const int s = t * kBlkK + r0;
    float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (s < a.S) load8<DT>(v + hv.base + (long long)s * hv.tok_stride + d0, x);
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float y0 = fminf(fmaxf(x[i] * inv[i], -448.0f), 448.0f);
      const float y1 = fminf(fmaxf(x[i + 1] * inv[i + 1], -448.0f), 448.0f);
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      tile[(grp * 8 + i) * kBlkK + pos] = (uint8_t)(pk & 0xff);
      tile[(grp * 8 + i + 1) * kBlkK + pos] = (uint8_t)((pk >> 8) & 0xff);
    }
    __syncthreads();
    if (tid < kSliceCh * kBlkK / 16) {
      const v4i val = reinterpret_cast<const v4i *>(tile)[tid];
      uint8_t *dst = a.v_fp8 + (((long long)bh * a.nk + t) * a.D + slice * kSliceCh) * kBlkK;
      reinterpret_cast<v4i *>(dst)[tid] = val;
    }
    __syncthreads();
  }
}

hipError_t launch_smooth_quant_qk(const QuantQKArgs &a, hipStream_t stream) {
  const int nslice = a.D / kSliceCh;
  const int g1 = a.B * a.H * nslice + a.B * a.H * a.nq;
  const int g2 = a.B * a.H * a.nk;
  if (a.dtype == 0) {
    hipLaunchKernelGGL(k_kmean_qquant<0>, dim3(g1), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(k_kquant<0>, dim3(g2), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(k_kmean_qquant<1>, dim3(g1), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(k_kquant<1>, dim3(g2), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_quant_v(const QuantVArgs &a, hipStream_t stream) {
  const int g = a.B * a.H * (a.D / kSliceCh);
  if (a.dtype == 0) hipLaunchKernelGGL(k_vquant<0>, dim3(g), dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(k_vquant<1>, dim3(g), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sage
