// attn.hip -- fused quantized attention for gfx950.
//
// Method ("SageAttention2" summary, sections 相关工作 and SageAttention2方法;
// "Kairos" guide, sections 2.1 and 2.2): INT8 Q.K^T with int32 accumulation,
// dequantised by the product of the Q-block and K-block scales; an online
// fp32 softmax over 64-key tiles (FlashAttention blocking); P~ quantised to
// FP8 E4M3 with the static scale 448 and multiplied with per-channel FP8 V;
// the FP8 products of one tile are summed by the MFMA into a fresh accumulator
// and then folded into an fp32 output buffer (two-level accumulation).  A pv
// fp16 mode keeps P~ and V in fp16 with fp32 accumulation.
//
// Mapping onto CDNA4:
//  * one work-group = 4 wavefronts = 128 query rows; one wavefront owns 32
//    query rows for the whole key loop (Q fragments stay in VGPRs);
//  * per 64-key tile the work-group stages the INT8 K tile (64 x D) and the
//    FP8 V tile (D x 64, channel-major, produced in that form by the V
//    quantiser) in LDS, XOR-swizzled by 16-byte chunk against bank conflicts;
//  * the wavefront computes S^T = K . Q^T with v_mfma_i32_32x32x32_i8, so the
//    32x32 result holds one query per lane column: lane (q, half) owns 16 keys
//    of each 32-key half tile, the row max / sum need one exchange with the
//    other half-wave, and the running max, sum and rescale factor stay in the
//    lane that uses them;
//  * the same registers, converted to E4M3 (v_cvt_pk_fp8_f32), are directly
//    the B operand of O^T = V^T . P^T on v_mfma_f32_32x32x64_f8f6f4: the key
//    order they imply is the order the V tile is stored in (vpos_key), so no
//    LDS round trip is needed for P;
//  * work-groups are numbered so that each XCD (own L2) works through whole
//    heads, keeping one head's K/V tiles in one L2; causal work is issued
//    longest query blocks first.
#include <math.h>

#include "sage_impl.h"

namespace sage {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448): folds the static P~ scale into exp2

// XOR swizzle of the 16-byte chunks of an LDS row, so that the 8 (or 16)
// consecutive rows a ds_read_b128 serves in one pass hit distinct banks.
// CH = chunks per row: 8 for 128-byte rows, 4 for 64-byte rows.
template <int CH>
__device__ inline int swz(int chunk, int row) {
  if (CH == 8) return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
  return chunk ^ (((row >> 1) ^ (row >> 3)) & 3);
}

template <int DT>
__device__ inline void store4(void *out, long long off, float a, float b, float c, float d) {
  const uint32_t lo = f32_to_out_bits<DT>(a) | (f32_to_out_bits<DT>(b) << 16);
  const uint32_t hi = f32_to_out_bits<DT>(c) | (f32_to_out_bits<DT>(d) << 16);
  v2i w = {(int)lo, (int)hi};
  *reinterpret_cast<v2i *>(reinterpret_cast<uint16_t *>(out) + off) = w;
}

template <int D, int PV, int DT, bool CAUSAL, bool DUMP>
__global__ __launch_bounds__(kThreads) void k_attn(const AttnArgs a) {
  constexpr int NC = D / 32;                      // 32-channel chunks of the head dim
  constexpr int KCH = D / 16;                     // 16-byte chunks per K row
  constexpr int VROW = PV == 0 ? 64 : 128;        // bytes per V^T row in LDS
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[64 * D];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * VROW];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, qn = lane & 31;

  // ---- work-group -> (head, query block), XCD-aware
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int nbh = a.B * a.H;
  int bh, mrank;
  if ((nbh & 7) == 0) {
    const int heads_per_xcd = nbh >> 3;
    const int xcd = wg & 7, idx = wg >> 3;
    if (CAUSAL) {  // longest blocks first, heads of this XCD interleaved
      bh = xcd * heads_per_xcd + idx % heads_per_xcd;
      mrank = idx / heads_per_xcd;
    } else {  // one head after the other inside this XCD
      bh = xcd * heads_per_xcd + idx / a.nmblk;
      mrank = idx % a.nmblk;
    }
  } else {
    if (CAUSAL) {
      bh = wg % nbh;
      mrank = wg / nbh;
    } else {
      bh = wg / a.nmblk;
      mrank = wg % a.nmblk;
    }
  }
  (void)nwg;
  const int mblk = CAUSAL ? a.nmblk - 1 - mrank : mrank;
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = mblk * kBlockM;
  const int qw = q0 + 32 * wave;  // first query row of this wavefront
  const bool active = qw < a.S;
  const int qi = qw + qn;         // this lane's query row

  // ---- Q fragments: B operand of S^T = K.Q^T; lane (q, half) holds
  //      Q[q][32c + 16*half .. +16] for chunk c
  v4i qf[NC];
  float dq = 0.0f;
  if (active) {
    const int8_t *qrow = a.q_i8 + ((long long)bh * a.S_q + qi) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const v4i *>(qrow + 32 * c + 16 * hh);
    dq = a.q_scale[(long long)bh * a.nq + (qw >> 5)];
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = v4i{0, 0, 0, 0};
  }

  int ntiles = a.nk;
  if (CAUSAL) {
    const int last_q = min(q0 + kBlockM - 1, a.S - 1);
    ntiles = min(a.nk, last_q / 64 + 1);
  }

  float m = -INFINITY;  // running max (log2 domain, scaled scores)
  float l = 0.0f;       // running sum of this half-wave's keys
  v16f O[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[c][r] = 0.0f;

  const int8_t *kbase = a.k_i8 + (long long)bh * a.S_k * D;
  const float *kscale = a.k_scale + (long long)bh * a.nk;

  for (int j = 0; j < ntiles; ++j) {
    __syncthreads();  // every wave is done with the previous tile
    // ---- stage K tile (64 x D int8, contiguous in HBM)
    {
      const v4i *src = reinterpret_cast<const v4i *>(kbase + (long long)j * 64 * D);
#pragma unroll
      for (int u = tid; u < 64 * KCH; u += kThreads) {
        const int row = u / KCH, ch = u % KCH;
        *reinterpret_cast<v4i *>(k_lds + row * D + 16 * swz<KCH>(ch, row)) = src[u];
      }
    }
    // ---- stage V tile
    if (PV == 0) {
      const v4i *src = reinterpret_cast<const v4i *>(reinterpret_cast<const uint8_t *>(a.v) +
                                                     ((long long)bh * a.nk + j) * D * 64);
#pragma unroll
      for (int u = tid; u < D * 4; u += kThreads) {
        const int row = u >> 2, ch = u & 3;
        *reinterpret_cast<v4i *>(v_lds + row * 64 + 16 * swz<4>(ch, row)) = src[u];
      }
    } else {
      // original 16-bit V (key-major) -> fp16 V^T rows in the vpos_key order.
      // thread: key pair (2e, 2e+1) x 8 channels; writes 8 x (2 halves).
      const HeadView hv = head_view(a.layout, b, h, a.H, a.S, D);
      const uint16_t *vsrc = reinterpret_cast<const uint16_t *>(a.v);
      constexpr int NU = 32 * (D / 8);  // key pairs x channel groups
#pragma unroll
      for (int u = tid; u < NU; u += kThreads) {
        const int pair = u / (D / 8), c8 = (u % (D / 8)) * 8;
        const int n0 = j * 64 + 2 * pair;
        uint32_t w0[4] = {0, 0, 0, 0}, w1[4] = {0, 0, 0, 0};
        if (n0 < a.S) {
          const v4i t0 = *reinterpret_cast<const v4i *>(vsrc + hv.base + (long long)n0 * hv.tok_stride + c8);
#pragma unroll
          for (int i = 0; i < 4; ++i) w0[i] = (uint32_t)t0[i];
        }
        if (n0 + 1 < a.S) {
          const v4i t1 = *reinterpret_cast<const v4i *>(vsrc + hv.base + (long long)(n0 + 1) * hv.tok_stride + c8);
#pragma unroll
          for (int i = 0; i < 4; ++i) w1[i] = (uint32_t)t1[i];
        }
        const int pos = key_vpos(2 * pair);  // even key; its odd partner sits at pos + 1
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t e0 = (w0[i >> 1] >> (16 * (i & 1))) & 0xffffu;
          uint32_t e1 = (w1[i >> 1] >> (16 * (i & 1))) & 0xffffu;
          if (DT == 1) {  // bf16 -> fp16, round to nearest even
            e0 = f32_to_f16_bits(bf16_to_f32(e0));
            e1 = f32_to_f16_bits(bf16_to_f32(e1));
          }
          const int row = c8 + i;
          const int byte = 2 * pos;  // 16-bit element pos, within a 128-byte row
          const int ch = byte >> 4, within = byte & 15;
          *reinterpret_cast<uint32_t *>(v_lds + row * 128 + 16 * swz<8>(ch, row) + within) = e0 | (e1 << 16);
        }
      }
    }
    __syncthreads();

    if (!active) continue;
    if (CAUSAL && j * 64 > qw + 31) continue;  // every key of the tile is in this wave's future

    // ---- S^T = K . Q^T : two 32-key halves, int32 accumulators
    v16i st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      const int row = 32 * t + qn;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v4i kf = *reinterpret_cast<const v4i *>(k_lds + row * D + 16 * swz<KCH>(2 * c + hh, row));
        st[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[c], st[t], 0, 0, 0);
      }
    }

    if (DUMP && bh == a.dump_bh && qi < a.S) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * 64 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key < a.S) a.dump[(long long)qi * a.S + key] = st[t][r];
        }
    }

    // ---- dequantise (log2 domain), mask, online softmax
    const float c2 = (dq * kscale[j]) * a.sm2;
    const bool need_mask = (j * 64 + 64 > a.S) || (CAUSAL && j * 64 + 63 > qw);
    float x[32];
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = (float)st[t][r] * c2;
        if (need_mask) {
          const int key = j * 64 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= a.S || (CAUSAL && key > qi)) v = -INFINITY;
        }
        x[16 * t + r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    const float sub = PV == 0 ? mn - kLog2_448 : mn;
    float ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] = __builtin_amdgcn_exp2f(x[i] - sub);
      ps += x[i];
    }
    l = alpha * l + ps;
    m = mn;

    if (PV == 0) {
      // ---- P~ -> E4M3 (byte 16t + r = key of st[t][r]), then O^T += V^T . P^T
      v8i pk;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w], x[4 * w + 1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2], x[4 * w + 3], word, true);
        pk[w] = word;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int row = 32 * c + qn;
        const v4i lo = *reinterpret_cast<const v4i *>(v_lds + row * 64 + 16 * swz<4>(2 * hh, row));
        const v4i hi = *reinterpret_cast<const v4i *>(v_lds + row * 64 + 16 * swz<4>(2 * hh + 1, row));
        const v8i vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const v16f zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        const v16f inner = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pk, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) O[c][r] = alpha * O[c][r] + inner[r];
      }
    } else {
      // ---- P~ -> fp16, O^T += V^T . P^T with four K=16 steps per tile
      v8h ph[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) ph[s][i] = (_Float16)x[8 * s + i];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int row = 32 * c + qn;
        v16f inner = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v8h vf = *reinterpret_cast<const v8h *>(v_lds + row * 128 + 16 * swz<8>(4 * hh + s, row));
          inner = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, ph[s], inner, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) O[c][r] = alpha * O[c][r] + inner[r];
      }
    }
  }

  if (!active) return;
  // ---- epilogue: combine the two half-wave sums, normalise, store
  const float lt = l + __shfl_xor(l, 32, 64);
  if (qi >= a.S) return;
  const float rl = 1.0f / lt;
  long long off;
  if (a.layout == 0) off = (((long long)b * a.H + h) * a.S + qi) * D;
  else off = (((long long)b * a.S + qi) * a.H + h) * D;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * c + 8 * g + 4 * hh;
      float o[4];
      if (PV == 0) {
        const float *vs = a.v_scale + (long long)bh * D + d0;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = O[c][4 * g + i] * (vs[i] * rl);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = O[c][4 * g + i] * rl;
      }
      store4<DT>(a.out, off + d0, o[0], o[1], o[2], o[3]);
    }
}

template <int D, int PV, int DT, bool CAUSAL>
static hipError_t launch4(const AttnArgs &a, bool dump, dim3 grid, hipStream_t st) {
  if (dump) hipLaunchKernelGGL((k_attn<D, PV, DT, CAUSAL, true>), grid, dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((k_attn<D, PV, DT, CAUSAL, false>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, int PV, int DT>
static hipError_t launch3(const AttnArgs &a, bool dump, dim3 grid, hipStream_t st) {
  return a.causal ? launch4<D, PV, DT, true>(a, dump, grid, st) : launch4<D, PV, DT, false>(a, dump, grid, st);
}

template <int D, int PV>
static hipError_t launch2(const AttnArgs &a, bool dump, dim3 grid, hipStream_t st) {
  return a.dtype == 0 ? launch3<D, PV, 0>(a, dump, grid, st) : launch3<D, PV, 1>(a, dump, grid, st);
}

template <int D>
static hipError_t launch1(const AttnArgs &a, bool dump, dim3 grid, hipStream_t st) {
  return a.pv == 0 ? launch2<D, 0>(a, dump, grid, st) : launch2<D, 1>(a, dump, grid, st);
}

hipError_t launch_attn(const AttnArgs &a, bool dump, hipStream_t stream) {
  const dim3 grid(a.B * a.H * a.nmblk);
  return a.D == 64 ? launch1<64>(a, dump, grid, stream) : launch1<128>(a, dump, grid, stream);
}

}  // namespace sage
