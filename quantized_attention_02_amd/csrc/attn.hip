// attn.hip -- fused quantized attention for gfx950.
//
// Method ("SageAttention2" summary, sections 相关工作 and SageAttention2方法;
// "Kairos" guide, sections 2.1 and 2.2): INT8 Q.K^T with int32 accumulation,
// dequantised by the product of the Q-block and K-block scales; an online
// fp32 softmax over key tiles (FlashAttention blocking); P~ quantised to FP8
// E4M3 with the static scale 448 and multiplied with per-channel FP8 V; the
// FP8 products of one tile are summed by the MFMA into a fresh accumulator and
// then folded into an fp32 output buffer (two-level accumulation).  A pv fp16
// mode keeps P~ and V in fp16 with fp32 accumulation.
//
// Mapping onto CDNA4:
//  * one work-group = 4 wavefronts = 128 query rows; a wavefront owns 32 query
//    rows for the whole key loop (Q fragments stay in VGPRs);
//  * the key loop walks 128-key tiles (two 64-key INT8 scale blocks).  K and
//    FP8 V tiles are copied HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), double-buffered: the copy of tile j+1 is in flight while tile j
//    is computed, and one barrier per tile publishes it.  The 16-byte chunks
//    of each LDS row are XOR-swizzled (applied to the source address of the
//    copy) so that the MFMA operand reads are bank-conflict free;
//  * the wavefront computes S^T = K . Q^T with v_mfma_i32_32x32x32_i8: the
//    32x32 result holds one query per lane column, so lane (q, half) owns 16
//    keys of every 32-key sub-tile, the row max needs one exchange with the
//    other half-wave, and the running max, sum and rescale factor live in the
//    lane that uses them.  The row max is taken on the int32 sums (one scale
//    per 64-key block), so each score costs one convert, one FMA and one exp2;
//  * the exp2 results, converted to E4M3 (v_cvt_pk_fp8_f32), are directly the
//    B operand of O^T = V^T . P^T on v_mfma_f32_32x32x64_f8f6f4: the key order
//    they imply is the order the V quantiser stores each 64-key block in
//    (vpos_key), so P never goes through LDS;
//  * work-groups are numbered so that each XCD (own L2) works through whole
//    heads; causal work is issued longest query blocks first.
#include <math.h>

#include "sage_impl.h"

namespace sage {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;
constexpr int kTileN = 128;  // keys per loop iteration (two INT8 K blocks)
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448): folds the static P~ scale into exp2

// XOR swizzle of the 16-byte chunks of an LDS row (CH = chunks per row) so that
// the 16 lanes an LDS read serves together hit 16 distinct bank groups when
// they read the same logical chunk of consecutive rows.
template <int CH>
__device__ __forceinline__ int swz(int chunk, int row) {
  if (CH == 8) return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
  return chunk ^ ((row >> 2) & 3);
}

// One wavefront-wide LDS DMA: lane i copies 16 bytes from `src` to
// lds_base + 16 * i (lds_base is the same for the whole wavefront).
__device__ __forceinline__ void dma16(const void *src, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds(
      src, (__attribute__((address_space(3))) void *)(__attribute__((address_space(3))) uint8_t *)lds_base, 16, 0, 0);
}

// Two consecutive floats at a wave-uniform address, read with a scalar load
// (constant address space), which the vector-memory counter does not track.
__device__ __forceinline__ float2 load2_uniform(const float *p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  typedef const __attribute__((address_space(4))) float2 *cptr;
  return *(cptr)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

template <int DT>
__device__ __forceinline__ void store4(void *out, long long off, float a, float b, float c, float d) {
  const uint32_t lo = f32_to_out_bits<DT>(a) | (f32_to_out_bits<DT>(b) << 16);
  const uint32_t hi = f32_to_out_bits<DT>(c) | (f32_to_out_bits<DT>(d) << 16);
  v2i w = {(int)lo, (int)hi};
  *reinterpret_cast<v2i *>(reinterpret_cast<uint16_t *>(out) + off) = w;
}

// Copy a K tile (128 x D int8) and, in pv fp8 mode, its two FP8 V blocks
// (2 x D x 64, contiguous in HBM) into LDS, swizzled.  Each wavefront issues
// its share of the 1 KiB wave-copies.
template <int D, int PV>
__device__ __forceinline__ void issue_tile(const int8_t *kt, const uint8_t *vt, uint8_t *kbuf, uint8_t *vbuf,
                                           int wave, int lane) {
  constexpr int KCH = D / 16;
  constexpr int KLOADS = kTileN * D / 1024;
  constexpr int KROWS = 1024 / D;
#pragma unroll
  for (int i = 0; i < KLOADS / kWaves; ++i) {
    const int w = wave + kWaves * i;
    const int row = w * KROWS + lane / KCH;
    dma16(kt + row * D + 16 * swz<KCH>(lane % KCH, row), kbuf + w * 1024);
  }
  if (PV == 0) {
    constexpr int VLOADS = 2 * D * 64 / 1024;
#pragma unroll
    for (int i = 0; i < VLOADS / kWaves; ++i) {
      const int w = wave + kWaves * i;
      const int row = w * 16 + (lane >> 2);
      dma16(vt + row * 64 + 16 * swz<4>(lane & 3, row), vbuf + w * 1024);
    }
  }
}

// pv fp16: original 16-bit V rows [n0, n0 + 64) -> fp16 V^T rows (128 bytes,
// vpos_key order, swizzled) in `vb`.  Staged through VGPRs: the layout change
// and the bf16 -> fp16 rounding need the values in registers anyway.
template <int D, int DT>
__device__ __forceinline__ void stage_v16(const AttnArgs &a, const HeadView &hv, int n0, uint8_t *vb, int tid) {
  const uint16_t *vsrc = reinterpret_cast<const uint16_t *>(a.v);
  constexpr int NU = 32 * (D / 8);  // key pairs x 8-channel groups
#pragma unroll
  for (int u = tid; u < NU; u += kThreads) {
    const int pair = u / (D / 8), c8 = (u % (D / 8)) * 8;
    const int n = n0 + 2 * pair;
    v4i t0 = {0, 0, 0, 0}, t1 = {0, 0, 0, 0};
    if (n < a.S) t0 = *reinterpret_cast<const v4i *>(vsrc + hv.base + (long long)n * hv.tok_stride + c8);
    if (n + 1 < a.S) t1 = *reinterpret_cast<const v4i *>(vsrc + hv.base + (long long)(n + 1) * hv.tok_stride + c8);
    const int pos = key_vpos(2 * pair);  // even key; its odd partner sits at pos + 1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t e0 = ((uint32_t)t0[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      uint32_t e1 = ((uint32_t)t1[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      if (DT == 1) {  // bf16 -> fp16, round to nearest even
        e0 = f32_to_f16_bits(bf16_to_f32(e0));
        e1 = f32_to_f16_bits(bf16_to_f32(e1));
      }
      const int row = c8 + i, byte = 2 * pos;
      *reinterpret_cast<uint32_t *>(vb + row * 128 + 16 * swz<8>(byte >> 4, row) + (byte & 15)) = e0 | (e1 << 16);
    }
  }
}

template <int D, int PV, int DT, bool CAUSAL, bool DUMP>
__global__ __launch_bounds__(kThreads, 2) void k_attn(const AttnArgs a) {
  constexpr int NC = D / 32;
  constexpr int KCH = D / 16;
  constexpr int KBYTES = kTileN * D;                         // K tile
  constexpr int VBYTES = PV == 0 ? 2 * D * 64 : D * 128;     // fp8: two 64-key blocks; fp16: one block
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[PV == 0 ? VBYTES : 1024];
  __shared__ __attribute__((aligned(16))) float vsc[D];  // this head's V channel scales (pv fp8)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, qn = lane & 31;

  // ---- work-group -> (head, query block), XCD-aware
  const int wg = blockIdx.x;
  const int nbh = a.B * a.H;
  int bh, mrank;
  if ((nbh & 7) == 0) {
    const int heads_per_xcd = nbh >> 3;
    const int xcd = wg & 7, idx = wg >> 3;
    if (CAUSAL) {  // longest blocks first; the XCD's heads interleaved
      bh = xcd * heads_per_xcd + idx % heads_per_xcd;
      mrank = idx / heads_per_xcd;
    } else {  // one head after the other inside this XCD
      bh = xcd * heads_per_xcd + idx / a.nmblk;
      mrank = idx % a.nmblk;
    }
  } else if (CAUSAL) {
    bh = wg % nbh;
    mrank = wg / nbh;
  } else {
    bh = wg / a.nmblk;
    mrank = wg % a.nmblk;
  }
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

  int ntiles = a.S_k / kTileN;
  if (CAUSAL) ntiles = min(ntiles, min(q0 + kBlockM - 1, a.S - 1) / kTileN + 1);

  float m = -INFINITY;  // running max (log2 domain, scaled scores)
  float l = 0.0f;       // running sum over this half-wave's keys
  v16f O[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[c][r] = 0.0f;

  const int8_t *kbase = a.k_i8 + (long long)bh * a.S_k * D;
  const uint8_t *vbase = reinterpret_cast<const uint8_t *>(a.v) + (long long)bh * a.S_k * D;
  const float *kscale = a.k_scale + (long long)bh * a.nk;
  const HeadView hv = head_view(a.layout, b, h, a.H, a.S, D);

  // One 128-key tile: QK^T, online softmax, PV.  kb / vb: this tile's LDS.
  auto tile = [&](int j, const uint8_t *kb, uint8_t *vb) {
    const int key0 = j * kTileN;
    const bool work = active && !(CAUSAL && key0 > qw + 31);
    // the tile's two K-block scales, read through a wave-uniform address (scalar loads)
    const float2 ksv = load2_uniform(kscale + 2 * j);
    const float ks[2] = {ksv.x, ksv.y};
    float p[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) p[i] = 0.0f;
    float alpha = 1.0f;
    if (work) {
      // ---- S^T = K . Q^T for four 32-key sub-tiles; per 32-channel chunk the
      //      four K fragments are read together, then four MFMAs consume them
      v16i s[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        v4i kf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int row = 32 * t + qn;
          kf[t] = *reinterpret_cast<const v4i *>(kb + row * D + 16 * swz<KCH>(2 * c + hh, row));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) s[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[t], qf[c], s[t], 0, 0, 0);
      }
      if (DUMP && bh == a.dump_bh && qi < a.S) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key < a.S) a.dump[(long long)qi * a.S + key] = s[t][r];
          }
      }
      float c2[2];
      c2[0] = (dq * ks[0]) * a.sm2;
      c2[1] = (dq * ks[1]) * a.sm2;
      // ---- mask: only tiles that reach past S or cross the causal diagonal
      const bool need_mask = (key0 + kTileN > a.S) || (CAUSAL && key0 + kTileN - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= a.S || (CAUSAL && key > qi)) s[t][r] = INT_MIN;
          }
      }
      // ---- row max on the int32 sums (c2 > 0 per 64-key block)
      float mt = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        int mx = INT_MIN;
#pragma unroll
        for (int t = 2 * blk; t < 2 * blk + 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = max(mx, s[t][r]);
        if (mx != INT_MIN) mt = fmaxf(mt, (float)mx * c2[blk]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m, mt);
      alpha = __builtin_amdgcn_exp2f(m - mn);
      const float sub = PV == 0 ? mn - kLog2_448 : mn;
      m = mn;
      // ---- p = exp2(s * c2 - sub)  (= 448 p~ in fp8 mode), row sum
      float ps = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = __builtin_fmaf((float)s[t][r], c2[t >> 1], -sub);
          if (need_mask && s[t][r] == INT_MIN) x = -INFINITY;
          p[16 * t + r] = __builtin_amdgcn_exp2f(x);
          ps += p[16 * t + r];
        }
      l = alpha * l + ps;
    }

    if constexpr (PV == 0) {
      if (work) {
        // ---- P~ -> E4M3: byte 16t' + r of operand blk = key of s[2 blk + t'][r]
        v8i pk[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int i0 = 32 * blk + 4 * w;
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[i0], p[i0 + 1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p[i0 + 2], p[i0 + 3], word, true);
            pk[blk][w] = word;
          }
        // ---- O^T = alpha * O^T + V^T . P^T (inner sum over the tile's 128 keys)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          v16f inner = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            const int row = blk * D + 32 * c + qn;
            const v4i lo = *reinterpret_cast<const v4i *>(vb + row * 64 + 16 * swz<4>(2 * hh, row));
            const v4i hi = *reinterpret_cast<const v4i *>(vb + row * 64 + 16 * swz<4>(2 * hh + 1, row));
            const v8i vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            inner = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pk[blk], inner, 0, 0, 0, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) O[c][r] = alpha * O[c][r] + inner[r];
        }
      }
    } else {
      // ---- pv fp16: P~ -> fp16, O rescaled, then O^T += V^T . P^T with fp32
      //      accumulation in the MFMA; V is staged one 64-key block at a time
      //      by the whole work-group (every wavefront takes part in the barriers)
      v8h ph[8];
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
#pragma unroll
        for (int i = 0; i < 8; ++i) ph[s8][i] = (_Float16)p[8 * s8 + i];
      if (work) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[c][r] *= alpha;
      }
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        stage_v16<D, DT>(a, hv, key0 + 64 * blk, vb, tid);
        __syncthreads();
        if (work) {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int row = 32 * c + qn;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const v8h vf = *reinterpret_cast<const v8h *>(vb + row * 128 + 16 * swz<8>(4 * hh + s4, row));
              O[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, ph[4 * blk + s4], O[c], 0, 0, 0);
            }
          }
        }
        __syncthreads();
      }
    }
  };

  if (PV == 0 && tid < D) vsc[tid] = a.v_scale[(long long)bh * D + tid];

  // ---- main loop: tile j computed from buffer j % 2 while tile j + 1 lands in the other
  issue_tile<D, PV>(kbase, vbase, kbuf0, vbuf0, wave, lane);
  wait_dma();
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    if (j + 1 < ntiles)
      issue_tile<D, PV>(kbase + (long long)(j + 1) * kTileN * D, vbase + (long long)(j + 1) * kTileN * D, kbuf1,
                        vbuf1, wave, lane);
    tile(j, kbuf0, vbuf0);
    wait_dma();
    __syncthreads();
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles)
      issue_tile<D, PV>(kbase + (long long)(j + 2) * kTileN * D, vbase + (long long)(j + 2) * kTileN * D, kbuf0,
                        vbuf0, wave, lane);
    tile(j + 1, kbuf1, PV == 0 ? vbuf1 : vbuf0);
    wait_dma();
    __syncthreads();
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
        const float4 vs = *reinterpret_cast<const float4 *>(vsc + d0);
        o[0] = O[c][4 * g + 0] * (vs.x * rl);
        o[1] = O[c][4 * g + 1] * (vs.y * rl);
        o[2] = O[c][4 * g + 2] * (vs.z * rl);
        o[3] = O[c][4 * g + 3] * (vs.w * rl);
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
