// attn_common.h -- device helpers of the attention kernel (attn.hip): LDS
// swizzles, HBM -> LDS tile copies through buffer resources, wave-uniform
// scalar loads, half-wave reductions, the row-sum operand, the work-group
// order, and the output store.  gfx950 only.
#pragma once

#include <math.h>

#include <type_traits>

#include "sage_impl.h"

namespace sage {

constexpr float kLog2_448 = 8.807354922057604f;  // log2(448): folds the static P~ scale into exp2



// XOR swizzle of the 16-byte chunks of an LDS row (CH = chunks per row) so that
// the 16 lanes an LDS read serves together hit 16 distinct bank groups when
// they read the same logical chunk of consecutive rows.
template <int CH>
__device__ __forceinline__ int swz(int chunk, int row) {
  if (CH == 8) return chunk ^ ((row & 7) ^ ((row >> 3) & 1));
  if (CH == 2) return chunk ^ ((row >> 3) & 1);
  return chunk ^ ((row >> 2) & 3);
}

// One wavefront-wide buffer load into LDS: lane i copies 16 bytes from
// resource offset soff + voff (voff per lane, soff wave-uniform) to
// lds_base + 16 * i.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff, uint8_t *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void *)(__attribute__((address_space(3))) uint8_t *)lds_base, 16, voff,
      soff, 0, 0);
}

// As dma16_buf with 4 bytes a lane (lane i -> lds_base + 4 * i).
__device__ __forceinline__ void dma4_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff, uint8_t *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void *)(__attribute__((address_space(3))) uint8_t *)lds_base, 4, voff,
      soff, 0, 0);
}

// Two consecutive floats at a wave-uniform address, read with a scalar load
// (constant address space), which the vector-memory counter does not track.
__device__ __forceinline__ float load1_uniform(const float *p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  typedef const __attribute__((address_space(4))) float *cptr;
  return *(cptr)(((uint64_t)hi << 32) | lo);
}

// n consecutive floats through a wave-uniform address (scalar loads)
template <int N>
__device__ __forceinline__ void loadn_uniform(const float *p, float *out) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  typedef const __attribute__((address_space(4))) float *cptr;
  const cptr q = (cptr)(((uint64_t)hi << 32) | lo);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = q[i];
}

__device__ __forceinline__ float2 load2_uniform(const float *p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  typedef const __attribute__((address_space(4))) float *cptr;
  const cptr q = (cptr)(((uint64_t)hi << 32) | lo);
  float2 r;
  r.x = q[0];
  r.y = q[1];
  return r;
}

// s_waitcnt vmcnt(N) (expcnt / lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// wait_vm with a wave-uniform count known at run time (at most 8 kept in
// flight; a larger count waits for everything)
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    default: wait_vm<0>(); break;
  }
}

// Max / sum of a value over the two half-waves (lanes i and i ^ 32 hold the
// same query row).  v_permlane32_swap exchanges the halves between its two
// outputs; one output then holds the lane's own value and the other its
// partner's, so the pair's max and sum need no lane-dependent select.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DT>
__device__ __forceinline__ void store4(void *out, long long off, float a, float b, float c, float d) {
  const uint32_t lo = f32_to_out_bits<DT>(a) | (f32_to_out_bits<DT>(b) << 16);
  const uint32_t hi = f32_to_out_bits<DT>(c) | (f32_to_out_bits<DT>(d) << 16);
  v2i w = {(int)lo, (int)hi};
  *reinterpret_cast<v2i *>(reinterpret_cast<uint16_t *>(out) + off) = w;
}

// A operand of the row-sum product.  v_mfma_f32_16x16x128_f8f6f4 reads its B
// operand (the 32 E4M3 weights a lane holds for its query and half-wave) as
// column l % 16, k-group l / 16 of a 128 x 16 matrix, so B's column n mixes
// the weights of queries n and n + 16 of both half-waves.  A row m of ones over
// the k-groups whose parity equals that of m / 4 gives C[m][n] = the full row
// sum of query n (m / 4 even) or n + 16 (m / 4 odd); lane l receives rows
// 4 (l / 16) .. + 3 of column l % 16, i.e. the sum of its own query l % 32.
// (Lane l of A holds row l % 16, k-group l / 16.)
__device__ __forceinline__ v8i rowsum_ones(int lane) {
  const int w = ((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)) ? 0x38383838 : 0;  // E4M3 1.0 x 4
  return v8i{w, w, w, w, w, w, w, w};
}

// Copy a K tile (TN x D int8) and, in pv fp8 mode, its FP8 V blocks
// (TN/64 x D x 64, contiguous in HBM) into LDS, swizzled.  Each wavefront
// issues its share of the 1 KiB wave-copies as buffer loads: scalar resource,
// scalar offset (tile + copy), one per-lane offset computed once.  Copy
// w = wave + WAVES i covers rows w * rows-per-copy ..; the swizzle of a lane's
// chunk depends on its row only through bits the copy index does not change
// (row mod 8 and the parity of row / 8 with D = 128 -- the parity of w is that
// of `wave` -- row / 4 mod 4 otherwise), so copy i is copy 0 shifted by
// 1024 WAVES i bytes, in HBM and in LDS.
template <int D, int TN, int WAVES>
struct TileCopy {
  static constexpr int KCH = D / 16;
  static constexpr int NCOPY = TN * D / 1024;                 // 1 KiB wave-copies per K (or V) tile
  static constexpr int LOADS = (NCOPY + WAVES - 1) / WAVES;  // per wavefront (the last round may be partial)
  static_assert(WAVES % 2 == 0, "copy i keeps the parity of the wavefront's first copy");
  uint32_t koff, voff;  // this lane's source offsets in the wavefront's first K / V copy
  __device__ __forceinline__ TileCopy(int wave, int lane) {
    const int krow = wave * (1024 / D) + lane / KCH;
    koff = (uint32_t)(krow * D + 16 * swz<KCH>(lane % KCH, krow));
    const int vrow = wave * 16 + (lane >> 2);
    voff = (uint32_t)(vrow * 64 + 16 * swz<4>(lane & 3, vrow));
  }
  // K copies a wavefront issues per tile
  __device__ __forceinline__ static int k_loads(int wave) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) n += (NCOPY % WAVES == 0 || wave + WAVES * i < NCOPY) ? 1 : 0;
    return n;
  }
  template <bool WITH_V>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, int tile_off,
                                        uint8_t *kbuf, uint8_t *vbuf, int wave) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      if (NCOPY % WAVES == 0 || wave + WAVES * i < NCOPY)
        dma16_buf(krs, koff, tile_off + 1024 * WAVES * i, kbuf + (wave + WAVES * i) * 1024);
    if (WITH_V) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        if (NCOPY % WAVES == 0 || wave + WAVES * i < NCOPY)
          dma16_buf(vrs, voff, tile_off + 1024 * WAVES * i, vbuf + (wave + WAVES * i) * 1024);
    }
  }
};

// MXFP4 Q K^T: copy a K tile of packed E2M1 rows (TN x D/2 bytes, 16-byte
// chunks swizzled by swz<D/32> so that the 16 lanes an LDS read serves hit 16
// distinct bank groups), then its E8M0 scale bytes (TN x D/32, linear, 4 bytes
// a lane), and, in pv fp8 mode, the FP8 V blocks as TileCopy does.
template <int D, int TN, int WAVES>
struct TileCopy4 {
  static constexpr int ROWB = D / 2;                          // bytes of a packed K row
  static constexpr int CPR = ROWB / 16;                       // 16-byte chunks a row (4 or 2)
  static constexpr int NCOPY = TN * ROWB / 1024;              // 1 KiB wave-copies of codes
  static constexpr int LOADS = (NCOPY + WAVES - 1) / WAVES;
  static constexpr int SCB = TN * (D / 32);                   // scale bytes a tile
  static constexpr int NSC = SCB / 256;                       // 256-byte wave-copies of scales
  static constexpr int VCOPY = TN * D / 1024;                 // 1 KiB wave-copies of FP8 V
  static constexpr int VLOADS = (VCOPY + WAVES - 1) / WAVES;
  static_assert(NSC <= WAVES && SCB % 256 == 0, "scale copy split");
  uint32_t koff, voff;  // as in TileCopy: copy i is copy 0 shifted by 1024 WAVES i bytes
  __device__ __forceinline__ TileCopy4(int wave, int lane) {
    const int krow = wave * (1024 / ROWB) + lane / CPR;
    koff = (uint32_t)(krow * ROWB + 16 * swz<CPR>(lane % CPR, krow));
    const int vrow = wave * 16 + (lane >> 2);
    voff = (uint32_t)(vrow * 64 + 16 * swz<4>(lane & 3, vrow));
  }
  // code and scale copies a wavefront issues per tile (without V)
  __device__ __forceinline__ static int k_loads(int wave) {
    int n = wave < NSC ? 1 : 0;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) n += (NCOPY % WAVES == 0 || wave + WAVES * i < NCOPY) ? 1 : 0;
    return n;
  }
  // tile j of the head: codes at j TN ROWB, scales at j SCB, V at j TN D
  template <bool WITH_V>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t srs,
                                        __amdgpu_buffer_rsrc_t vrs, int j, uint8_t *kbuf, uint8_t *vbuf, int wave,
                                        int lane) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      if (NCOPY % WAVES == 0 || wave + WAVES * i < NCOPY)
        dma16_buf(krs, koff, j * TN * ROWB + 1024 * WAVES * i, kbuf + (wave + WAVES * i) * 1024);
    if (wave < NSC) dma4_buf(srs, (uint32_t)(4 * lane), j * SCB + 256 * wave, kbuf + TN * ROWB + 256 * wave);
    if (WITH_V) {
#pragma unroll
      for (int i = 0; i < VLOADS; ++i)
        if (VCOPY % WAVES == 0 || wave + WAVES * i < VCOPY)
          dma16_buf(vrs, voff, j * TN * D + 1024 * WAVES * i, vbuf + (wave + WAVES * i) * 1024);
    }
  }
};


// The same selector for the micro-scaled FP4 product (E2M1 1.0 = code 2, two a
// byte); the FP4 operand fills four of the eight registers.
__device__ __forceinline__ v8i rowsum_ones_fp4(int lane) {
  const int w = ((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)) ? 0x22222222 : 0;
  return v8i{w, w, w, w, 0, 0, 0, 0};
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = I .. N - 1 (for
// builtins whose arguments must be constants).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<I + 1, N>(f);
  }
}

// Work-group -> (batch-head pair, rank of its query block), XCD-aware: the
// eight XCDs (each with its own L2) take eighths of the work so that a head's
// K/V codes are read from one or two L2s.  Causal work is ranked longest query
// blocks first.
__device__ __forceinline__ void map_work(const AttnArgs &a, bool causal, int &bh, int &mrank) {
  const int wg = blockIdx.x;
  const int nbh = a.B * a.H;
  if (a.varlen && (a.H & 7) == 0) {
    // packed batches: sequences differ in length, so every XCD takes the same
    // share of every sequence: XCD x owns heads [x H/8, (x+1) H/8) of each one
    // (consecutive heads, so a grouped-query K/V head stays in one L2)
    const int hx = a.H >> 3, xcd = wg & 7, idx = wg >> 3;
    const int pairs = a.B * hx;  // (sequence, head) pairs of this XCD
    int pair;
    if (causal) {  // longest blocks first
      pair = idx % pairs;
      mrank = idx / pairs;
    } else {
      pair = idx / a.nmblk;
      mrank = idx % a.nmblk;
    }
    bh = (pair / hx) * a.H + xcd * hx + pair % hx;
  } else if (!a.varlen && (nbh & 7) == 0) {
    const int heads_per_xcd = nbh >> 3;
    const int xcd = wg & 7, idx = wg >> 3;
    if (causal && a.nmblk < 128) {  // longest blocks first; the XCD's heads interleaved
      bh = xcd * heads_per_xcd + idx % heads_per_xcd;
      mrank = idx / heads_per_xcd;
    } else {  // one head after the other inside this XCD (causal: longest blocks first)
      // A long causal head (128 query blocks or more) alone keeps an XCD's 64
      // work-group slots busy, and its K/V codes (from 4 MB up) fill the XCD's
      // L2: interleaving heads would multiply the K/V working set.
      bh = xcd * heads_per_xcd + idx / a.nmblk;
      mrank = idx % a.nmblk;
    }
  } else if (!a.varlen && !causal && ((nbh * a.nmblk) & 7) == 0) {
    // heads not a multiple of 8: XCD x takes the x-th eighth of the (head,
    // block) order, so that a head's work-groups share one or two L2s instead
    // of all eight
    const int flat = (wg & 7) * ((nbh * a.nmblk) >> 3) + (wg >> 3);
    bh = flat / a.nmblk;
    mrank = flat % a.nmblk;
  } else if (causal) {
    bh = wg % nbh;
    mrank = wg / nbh;
  } else {
    bh = wg / a.nmblk;
    mrank = wg % a.nmblk;
  }
}

}  // namespace sage
