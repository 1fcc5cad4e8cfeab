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

#include <type_traits>

#include "sage_impl.h"

namespace sage {

constexpr float kLog2_448 = 8.807354922057604f;

#ifndef SAGE_ATTN_TN_FP8
#define SAGE_ATTN_TN_FP8 128
#endif
#ifndef SAGE_ATTN_WPS_FP8
#define SAGE_ATTN_WPS_FP8 2
#endif
#ifndef SAGE_ATTN_WAVES_FP8
#define SAGE_ATTN_WAVES_FP8 4
#endif
#ifndef SAGE_ATTN_NBUF_FP8
#define SAGE_ATTN_NBUF_FP8 2
#endif  // log2(448): folds the static P~ scale into exp2

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

// Sum of N floats as a balanced tree (independent adds instead of one serial
// dependency chain).
template <int N>
__device__ __forceinline__ float tree_sum(const float *x) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    return tree_sum<N / 2>(x) + tree_sum<N - N / 2>(x + N / 2);
  }
}

// Copy a K tile (TN x D int8) and, in pv fp8 mode, its FP8 V blocks
// (TN/64 x D x 64, contiguous in HBM) into LDS, swizzled.  Each wavefront
// issues its share of the 1 KiB wave-copies as buffer loads: scalar resource
// and tile offset, per-lane offsets koff / voff computed once (tile_offsets).
template <int D, int TN, int WAVES>
struct TileCopy {
  static constexpr int KCH = D / 16;
  static constexpr int NCOPY = TN * D / 1024;                 // 1 KiB wave-copies per K (or V) tile
  static constexpr int LOADS = (NCOPY + WAVES - 1) / WAVES;  // per wavefront (the last round may be partial)
  uint32_t koff[LOADS], voff[LOADS];
  __device__ __forceinline__ TileCopy(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int w = wave + WAVES * i;
      const int krow = w * (1024 / D) + lane / KCH;
      koff[i] = (uint32_t)(krow * D + 16 * swz<KCH>(lane % KCH, krow));
      const int vrow = w * 16 + (lane >> 2);
      voff[i] = (uint32_t)(vrow * 64 + 16 * swz<4>(lane & 3, vrow));
    }
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
        dma16_buf(krs, koff[i], tile_off, kbuf + (wave + WAVES * i) * 1024);
    if (WITH_V) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        if (NCOPY % WAVES == 0 || wave + WAVES * i < NCOPY)
          dma16_buf(vrs, voff[i], tile_off, vbuf + (wave + WAVES * i) * 1024);
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
  uint32_t koff[LOADS], voff[VLOADS];
  __device__ __forceinline__ TileCopy4(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int krow = (wave + WAVES * i) * (1024 / ROWB) + lane / CPR;
      koff[i] = (uint32_t)(krow * ROWB + 16 * swz<CPR>(lane % CPR, krow));
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int vrow = (wave + WAVES * i) * 16 + (lane >> 2);
      voff[i] = (uint32_t)(vrow * 64 + 16 * swz<4>(lane & 3, vrow));
    }
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
        dma16_buf(krs, koff[i], j * TN * ROWB, kbuf + (wave + WAVES * i) * 1024);
    if (wave < NSC) dma4_buf(srs, (uint32_t)(4 * lane), j * SCB + 256 * wave, kbuf + TN * ROWB + 256 * wave);
    if (WITH_V) {
#pragma unroll
      for (int i = 0; i < VLOADS; ++i)
        if (VCOPY % WAVES == 0 || wave + WAVES * i < VCOPY)
          dma16_buf(vrs, voff[i], j * TN * D, vbuf + (wave + WAVES * i) * 1024);
    }
  }
};

// pv fp16: the tile's raw 16-bit V rows (TN keys x D channels, 2D bytes a
// row, as stored in the caller's layout) are copied into LDS as they are (bf16
// rows are then rounded to fp16 in place, each lane the chunks it copied);
// the PV MFMA's V^T operand is then read with the transposing LDS load
// ds_read_b64_tr_b16.  Within each 16-lane group, lane i receives element
// i % 4 of the 8-byte pieces addressed by lanes 4 j + i / 4 (j = 0..3): with
// lane p pointing at V[key0 + p / 4][c0 + 4 (p % 4) ..], lane i obtains
// channel c0 + i for keys key0 .. key0 + 3.
//
// 16-byte chunks of a V row are XOR-swizzled by the row so that the 32 lanes
// an LDS read serves together (4 rows x 16 chunks of 16 bytes for D = 128)
// hit 64 distinct banks.
template <int D>
__device__ __forceinline__ int swz16(int chunk, int row) {
  if (D == 128) return chunk ^ (4 * (row & 3));
  return chunk ^ (4 * ((row >> 1) & 1));
}

template <int D, int TN, int WAVES>
struct VCopy16 {
  static constexpr int ROWB = 2 * D;                // bytes of a V row
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int RPC = 1024 / ROWB;           // rows per 1 KiB wave-copy
  static constexpr int NCOPY = TN * ROWB / 1024;    // wave-copies per tile
  static constexpr int LOADS = NCOPY / WAVES;
  static_assert(NCOPY % WAVES == 0, "even split of the V copies");
  int lrow;       // row of this lane inside a wave-copy
  uint32_t lcol;  // byte offset of this lane's (swizzled) source chunk in its row
  __device__ __forceinline__ VCopy16(int lane) {
    lrow = lane / CPR;
    // the swizzle depends on row & 3 (D = 128) or (row >> 1) & 1 (D = 64) only,
    // and a copy's first row is a multiple of RPC (4 or 8): lrow decides it
    lcol = (uint32_t)(16 * swz16<D>(lane % CPR, lrow));
  }
  // rows key0 .. key0 + TN - 1 of the head; rows at or past S are outside the
  // buffer resource's range and read as zeros
  __device__ __forceinline__ void issue(const uint16_t *v, const HeadView &hv, int key0, int S, uint8_t *vb,
                                        int wave) const {
    const int nvalid = min(TN, S - key0);
    const long long ts2 = 2 * hv.tok_stride;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(v + hv.base + (long long)key0 * hv.tok_stride, (int)(nvalid * ts2));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int k = wave + WAVES * i;
      dma16_buf(rs, (uint32_t)((k * RPC + lrow) * ts2) + lcol, 0, vb + k * 1024);
    }
  }
  // bf16 input: once this lane's copies have landed, round the 16-byte chunks
  // it copied to fp16 in place (RNE), so that the tile is read as fp16 by every
  // wavefront; chunk positions (and the swizzle) are unchanged
  __device__ __forceinline__ void to_f16(uint8_t *vb, int wave, int lane) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      v4i *c = reinterpret_cast<v4i *>(vb + (wave + WAVES * i) * 1024 + 16 * lane);
      v4i u = *c;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = (uint32_t)u[w];
        const _Float16 lo = (_Float16)__uint_as_float(x << 16);
        const _Float16 hi = (_Float16)__uint_as_float(x & 0xffff0000u);
        u[w] = (int)((uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16));
      }
      *c = u;
    }
  }
};

// V^T fragment (channels 32 c .. 32 c + 31 down the lanes, keys 16 sb .. +15
// across them in the MFMA k order of the P registers) for v_mfma_f32_32x32x16_f16,
// from the fp16 tile in LDS.
template <int D>
__device__ __forceinline__ v8h vfrag16(const uint8_t *vb, int c, int sb, int lane) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s *lds_v4s;
  const int g = lane >> 4, p = lane & 15, hh = lane >> 5;
  const int cb = 64 * c + 32 * (g & 1) + 8 * (p & 3);  // byte of the lane's 4 channels in a row
  v4s h[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int key = 16 * sb + 8 * r + 4 * hh + (p >> 2);
    const int off = key * (2 * D) + 16 * swz16<D>(cb >> 4, key) + (cb & 15);
    h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)((__attribute__((address_space(3))) uint8_t *)vb + off));
  }
  v8h out;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = __builtin_bit_cast(_Float16, (uint16_t)h[i >> 2][i & 3]);
  return out;
}

// TN: keys per loop iteration (64 or 128, i.e. one or two INT8 K blocks);
// WPS: wavefronts per SIMD the register budget is sized for; WAVES: wavefronts
// per work-group (32 query rows each); NBUF: LDS tile buffers (prefetch
// distance NBUF - 1).  QK: the Q K^T operands.  0: INT8, one scale per
// 32-query block and per 64-key block.  1 (LANE): INT8 with thread-level scale
// granularity -- one Q scale per token (this lane's query) and one K scale per
// 16-key lane group (the keys this half-wave holds of each 32-key sub-tile), so
// every lane dequantises each sub-tile with one scale of its own.  2 (FP4):
// MXFP4 -- E2M1 codes with an E8M0 scale per 32 channels of a token, on the
// scaled FP4 MFMA, which applies the scales itself (fp32 scores).  3 (TOKEN):
// INT8 with one Q scale per token and one K scale per key; the tile's key
// scales are staged in LDS with the tile, and each score is dequantised by its
// key's scale in fp32 before the row max (the query's scale and sm_scale are
// one factor per lane, applied in the exponent).  QS:
// smoothed Q -- the scores gain the pre-processing term delta[query block][key]
// (a wavefront's 32 queries share one block), staged in LDS with each tile.
template <int D, int PV, int DT, bool CAUSAL, bool DUMP, int QK, bool QS, int TN, int WPS, int WAVES, int NBUF>
__global__ __attribute__((amdgpu_flat_work_group_size(WAVES * 64, WAVES * 64), amdgpu_waves_per_eu(WPS, WPS))) void
k_attn(const AttnArgs a) {
  constexpr bool LANE = QK == 1, FP4 = QK == 2, TOKEN = QK == 3;
  constexpr int kBlockM = WAVES * 32;
  constexpr int NC = D / 32;
  constexpr int KCH = D / 16;
  constexpr int NB = TN / 64;                                // INT8 K blocks per tile
  constexpr int NT = TN / 32;                                // 32-key sub-tiles per tile
  constexpr int KBYTES = TN * D;                             // K tile
  constexpr int VBYTES = PV == 0 ? TN * D : 2 * TN * D;     // fp8: NB 64-key blocks; fp16: TN raw 16-bit rows
  constexpr int NVBUF = PV == 0 ? NBUF : 1;                 // fp16 V: one buffer, refilled every tile
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[NBUF][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[NVBUF][VBYTES];
  __shared__ __attribute__((aligned(16))) float vsc[D];  // this head's V channel scales (pv fp8)
  __shared__ __attribute__((aligned(16))) float vmn[D];  // its channel means when V was smoothed
  // smoothed Q: each wavefront's row of the pre-processing term for the tile's keys
  __shared__ __attribute__((aligned(16))) float dsbuf[QS ? NBUF : 1][QS ? WAVES : 1][QS ? TN : 4];
  // per-token K scales: the tile's key scales (copied by the first TN / 64 wavefronts)
  __shared__ __attribute__((aligned(16))) float ksbuf[TOKEN ? NBUF : 1][TOKEN ? TN : 4];
  static_assert(!TOKEN || (TN / 64 <= WAVES && NBUF == 2), "key-scale copy split and whole-tile vm waits");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: branches on it stay scalar
  const int hh = lane >> 5, qn = lane & 31;

  // ---- work-group -> (head, query block), XCD-aware
  const int wg = blockIdx.x;
  const int nbh = a.B * a.H;
  int bh, mrank;
  if (a.varlen && (a.H & 7) == 0) {
    // packed batches: sequences differ in length, so every XCD takes the same
    // share of every sequence: XCD x owns heads [x H/8, (x+1) H/8) of each one
    // (consecutive heads, so a grouped-query K/V head stays in one L2)
    const int hx = a.H >> 3, xcd = wg & 7, idx = wg >> 3;
    const int pairs = a.B * hx;  // (sequence, head) pairs of this XCD
    int pair;
    if (CAUSAL) {  // longest blocks first
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
    if (CAUSAL) {  // longest blocks first; the XCD's heads interleaved
      bh = xcd * heads_per_xcd + idx % heads_per_xcd;
      mrank = idx / heads_per_xcd;
    } else {  // one head after the other inside this XCD
      bh = xcd * heads_per_xcd + idx / a.nmblk;
      mrank = idx % a.nmblk;
    }
  } else if (!a.varlen && !CAUSAL && ((nbh * a.nmblk) & 7) == 0) {
    // heads not a multiple of 8: XCD x takes the x-th eighth of the (head,
    // block) order, so that a head's work-groups share one or two L2s instead
    // of all eight
    const int flat = (wg & 7) * ((nbh * a.nmblk) >> 3) + (wg >> 3);
    bh = flat / a.nmblk;
    mrank = flat % a.nmblk;
  } else if (CAUSAL) {
    bh = wg % nbh;
    mrank = wg / nbh;
  } else {
    bh = wg / a.nmblk;
    mrank = wg % a.nmblk;
  }
  const int mblk = CAUSAL ? a.nmblk - 1 - mrank : mrank;
  const int b = bh / a.H, h = bh % a.H;
  // grouped-query attention: H / H_kv consecutive query heads read one K/V head
  const int hk = h / (a.H / a.H_kv), bhk = b * a.H_kv + hk;

  // ---- this head's queries and keys: a fixed-length batch entry, or one
  //      sequence of a packed batch (its own lengths and buffer rows)
  Seg qs, ks;  // rows of q_i8 / k_i8 and v_fp8; qs also places the output, ks the caller's V
  if (a.varlen) {
    qs = varlen_seg(a.sq, b, h, a.H, D, a.rows_q, kBlkQ);
    ks = varlen_seg(a.sk, b, hk, a.H_kv, D, a.rows_k, kKvPad);
  } else {
    qs = fixed_seg(a.layout, b, h, a.H, a.S, a.S_q, D);
    ks = fixed_seg(a.layout, b, hk, a.H_kv, a.S, a.S_k, D);
  }
  const int Sq = qs.S, Sk = ks.S;
  const int q0 = mblk * kBlockM;
  if (q0 >= Sq) return;           // past a short sequence of a packed batch (whole work-group)
  const int qw = q0 + 32 * wave;  // first query row of this wavefront
  const bool active = qw < Sq;
  const int qi = qw + qn;         // this lane's query row

  // ---- Q fragments: B operand of S^T = K.Q^T; lane (q, half) holds
  //      Q[q][32c + 16*half .. +16] for chunk c
  //      (FP4: Q[q][64c + 32*half .. +32] packed for chunk c < D / 64, and the
  //      query's E8M0 bytes shifted so that byte 2c is this half's block of chunk c)
  v4i qf[NC];
  float dq = 0.0f;
  uint32_t qsc = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = v4i{0, 0, 0, 0};
  if (active) {
    if constexpr (FP4) {
      const uint8_t *qrow = reinterpret_cast<const uint8_t *>(a.q_i8) + (qs.row0 + qi) * (D / 2);
#pragma unroll
      for (int c = 0; c < D / 64; ++c) qf[c] = *reinterpret_cast<const v4i *>(qrow + 32 * c + 16 * hh);
      const uint8_t *qsr = reinterpret_cast<const uint8_t *>(a.q_scale) + (qs.row0 + qi) * (D / 32);
      const uint32_t w = D == 128 ? *reinterpret_cast<const uint32_t *>(qsr) : *reinterpret_cast<const uint16_t *>(qsr);
      qsc = w >> (8 * hh);
    } else {
      const int8_t *qrow = a.q_i8 + (qs.row0 + qi) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const v4i *>(qrow + 32 * c + 16 * hh);
      dq = LANE || TOKEN ? a.q_scale[qs.row0 + qi] : a.q_scale[(qs.row0 + qw) >> 5];
    }
  }

  int ntiles = (Sk + TN - 1) / TN;
  if (CAUSAL) ntiles = min(ntiles, min(q0 + kBlockM - 1, Sk - 1) / TN + 1);

  float m = -INFINITY;  // running max (log2 domain, scaled scores)
  float l = 0.0f;       // running sum over this half-wave's keys
  v16f O[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[c][r] = 0.0f;

  const int8_t *kbase = a.k_i8 + ks.row0 * (FP4 ? D / 2 : D);
  const uint8_t *vbase = reinterpret_cast<const uint8_t *>(a.v) + ks.row0 * D;
  const float *kscale = a.k_scale + (TOKEN ? ks.row0 : LANE ? ks.row0 >> 4 : ks.row0 >> 6);  // INT8 modes
  const uint8_t *kscb = reinterpret_cast<const uint8_t *>(a.k_scale) + ks.row0 * (D / 32);  // FP4
  const HeadView hv{ks.base, ks.stride};  // pv fp16: the caller's V
  const TileCopy<D, TN, WAVES> copy(wave, lane);     // INT8 K
  const TileCopy4<D, TN, WAVES> copy4(wave, lane);   // FP4 K
  const VCopy16<D, TN, WAVES> vcopy(lane);
  const int vbytes = ntiles * TN * D;                // this head's V (and INT8 K) bytes that the tiles read
  const int kbytes = FP4 ? vbytes / 2 : vbytes;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, kbytes);
  const __amdgpu_buffer_rsrc_t srs = TOKEN ? make_rsrc(kscale, ntiles * TN * 4)  // per-key K scales
                                           : make_rsrc(kscb, ntiles * TN * (D / 32));  // FP4 K scales
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(PV == 0 ? (const void *)vbase : (const void *)kbase,
                                               PV == 0 ? vbytes : kbytes);  // (pv fp16 copies V itself)
  // smoothed Q: delta is stored [bh][128-key tile][query block][128]; this
  // wavefront's row of tile j (its query block) is 512 contiguous bytes at
  // dbase + j * dtile; only wavefronts with queries copy (a trailing wavefront's
  // block may not exist)
  const float *dbase = QS ? a.delta_s + ((long long)bh * (a.S_k / kKvPad) * a.nq + (qw >> 5)) * kKvPad : nullptr;
  const long long dtile = (long long)a.nq * kKvPad;  // floats from one tile to the next
  // copies of tile j into buffer buf; returns how many copy instructions this
  // wavefront issued without V (pv fp16 counts them to wait for its V alone)
  auto issue_tile = [&](int j, int buf, uint8_t *kb, uint8_t *vb) -> int {
    int n;
    if constexpr (FP4) {
      copy4.template issue<PV == 0>(krs, srs, vrs, j, kb, vb, wave, lane);
      n = copy4.k_loads(wave);
    } else {
      copy.template issue<PV == 0>(krs, vrs, j * TN * D, kb, vb, wave);
      n = copy.k_loads(wave);
    }
    if constexpr (TOKEN) {
      // every wavefront needs every key's scale: the first TN / 64 copy them,
      // whether or not they have queries of their own
      if (wave < TN / 64) {
        dma4_buf(srs, (uint32_t)(4 * lane), 4 * (j * TN + 64 * wave),
                 reinterpret_cast<uint8_t *>(&ksbuf[buf][0]) + 256 * wave);
        n += 1;
      }
    }
    if constexpr (QS) {
      if (active) {
#pragma unroll
        for (int i = 0; i < TN / 64; ++i) {
          const int key = j * TN + 64 * i;  // first key of this 64-key half: its 128-key delta tile and half
          const __amdgpu_buffer_rsrc_t drs = make_rsrc(dbase + (key / kKvPad) * dtile, kKvPad * 4);
          dma4_buf(drs, (uint32_t)(4 * lane), 256 * ((key / 64) & 1),
                   reinterpret_cast<uint8_t *>(&dsbuf[buf][wave][0]) + 256 * i);
        }
        n += TN / 64;
      }
    }
    return n;
  };

  // One TN-key tile: QK^T, online softmax, PV.  kb / vb: this tile's LDS.
  // pend (pv fp16): copy instructions this wavefront issued after the tile's V.
  auto tile = [&](int j, int buf, const uint8_t *kb, uint8_t *vb, int pend) {
    const float *dsr = &dsbuf[QS ? buf : 0][QS ? wave : 0][0];  // smoothed Q: this wavefront's delta row
    const float *ksr = &ksbuf[TOKEN ? buf : 0][0];               // per-token K: the tile's key scales
    const int key0 = j * TN;
    const bool work = active && !(CAUSAL && key0 > qw + 31);
    // the tile's K scales, read through a wave-uniform address (scalar loads)
    constexpr int NKS = LANE ? 2 * NT : NB;  // per lane group, or per 64-key block
    float ks[NKS];
    if constexpr (TOKEN) {
      // (per-key scales: read from ksr with the scores)
    } else if constexpr (LANE || NB > 2) {
      loadn_uniform<NKS>(kscale + NKS * j, ks);
    } else if constexpr (NB == 2) {
      const float2 ksv = load2_uniform(kscale + 2 * j);
      ks[0] = ksv.x;
      ks[NB - 1] = ksv.y;
    } else {
      ks[0] = load1_uniform(kscale + j);
    }
    float p[16 * NT];
    float alpha = 1.0f;
    if (work) {
      // ---- S^T = K . Q^T for the NT 32-key sub-tiles, one INT8 K block (two
      //      sub-tiles) after the other, so that the first block's row max and
      //      int -> float conversion can run while the second block's MFMAs do
      using acc_t = typename std::conditional<FP4, v16f, v16i>::type;
      acc_t s[NT];
      if constexpr (FP4 && QS) {
        // smoothed Q on the FP4 product: the scaled MFMA accumulates in fp32 on top of
        // its C operand, so the pre-processing term of each key is the accumulator's
        // starting value (keys 8 (r / 4) + 4 hh + r % 4 of the sub-tile)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 d4 = *reinterpret_cast<const float4 *>(dsr + 32 * t + 8 * g + 4 * hh);
            s[t][4 * g] = d4.x;
            s[t][4 * g + 1] = d4.y;
            s[t][4 * g + 2] = d4.z;
            s[t][4 * g + 3] = d4.w;
          }
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[t][r] = 0;
      }
      auto qk_block = [&](int blk) {
        if constexpr (FP4) {
          // per key: its E8M0 word, shifted so that byte 2c is this half's block of chunk c
#pragma unroll
          for (int t = 2 * blk; t < 2 * blk + 2; ++t) {
            const int row = 32 * t + qn;
            const uint8_t *ksr = kb + TN * (D / 2) + row * (D / 32);
            const uint32_t kw =
                D == 128 ? *reinterpret_cast<const uint32_t *>(ksr) : *reinterpret_cast<const uint16_t *>(ksr);
            const uint32_t ksc = kw >> (8 * hh);
#pragma unroll
            for (int c = 0; c < D / 64; ++c) {
              const v4i kf = *reinterpret_cast<const v4i *>(kb + row * (D / 2) + 16 * swz<D / 32>(2 * c + hh, row));
              const v8i ka = {kf[0], kf[1], kf[2], kf[3], 0, 0, 0, 0};
              const v8i qa = {qf[c][0], qf[c][1], qf[c][2], qf[c][3], 0, 0, 0, 0};
              s[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qa, s[t], 4, 4, 0, (int)(ksc >> (16 * c)), 0,
                                                                    (int)(qsc >> (16 * c)));
            }
          }
        } else {
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int t = 2 * blk; t < 2 * blk + 2; ++t) {
              const int row = 32 * t + qn;
              const v4i kf = *reinterpret_cast<const v4i *>(kb + row * D + 16 * swz<KCH>(2 * c + hh, row));
              s[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[c], s[t], 0, 0, 0);
            }
        }
      };
      auto dump_s = [&]() {
        if (DUMP && !FP4 && bh == a.dump_bh && qi < a.S) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
              if (key < a.S) a.dump[(long long)qi * a.S + key] = s[t][r];
            }
        }
      };
      // dequantisation factors: per 64-key block, or (LANE) per 32-key sub-tile
      // with this half-wave's group scale
      constexpr int NC2 = LANE ? NT : NB;
      float c2[NC2];
      float cdq[NC2];  // smoothed Q: the dequantisation factor alone (sm_scale applied later)
      if constexpr (QS) {
#pragma unroll
        for (int i = 0; i < NC2; ++i) {
          cdq[i] = TOKEN ? dq : LANE ? dq * (hh ? ks[2 * i + 1] : ks[2 * i]) : dq * ks[i];
          c2[i] = a.sm2;
        }
      } else if constexpr (LANE) {
#pragma unroll
        for (int t = 0; t < NT; ++t) c2[t] = (dq * (hh ? ks[2 * t + 1] : ks[2 * t])) * a.sm2;
      } else if constexpr (FP4) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) c2[blk] = a.sm2;  // the MFMA applied the micro-scales
      } else if constexpr (TOKEN) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) c2[blk] = dq * a.sm2;  // the key scales are in the scores
      } else {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) c2[blk] = (dq * ks[blk]) * a.sm2;
      }
      // ---- mask: only tiles that reach past S or cross the causal diagonal
      // key (key0 + 4hh + kofs(t, r)) is excluded iff kofs(t, r) > lim, where
      // kofs is a compile-time constant of the register slot
      const bool need_mask = (key0 + TN > Sk) || (CAUSAL && key0 + TN - 1 > qw);
      const int lim = (CAUSAL ? min(Sk - 1, qi) : Sk - 1) - key0 - 4 * hh;
      // ---- per INT8 block: row max of the int32 sums (c2 > 0 per block) and
      //      the sums converted to float
      int mxb[NC2];  // int32 max per scale (one c2 each)
      float mxf[NB];  // FP4: fp32 max per block
      float f[16 * NT];
      auto max_convert = [&](int blk, int mlim, auto mask_tag) {
        if constexpr (FP4 || QS || TOKEN) {  // fp32 scores: dequantised (+ delta), max in fp32
          float mx = -INFINITY;
#pragma unroll
          for (int t = 2 * blk; t < 2 * blk + 2; ++t) {
            float4 dv[4], kv[4];
            if constexpr (QS && !FP4)
#pragma unroll
              for (int g = 0; g < 4; ++g) dv[g] = *reinterpret_cast<const float4 *>(dsr + 32 * t + 8 * g + 4 * hh);
            if constexpr (TOKEN)
#pragma unroll
              for (int g = 0; g < 4; ++g) kv[g] = *reinterpret_cast<const float4 *>(ksr + 32 * t + 8 * g + 4 * hh);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const bool out = decltype(mask_tag)::value && 32 * t + 8 * (r >> 2) + (r & 3) > mlim;
              float val;
              if constexpr (FP4) {
                val = s[t][r];
              } else if constexpr (TOKEN) {
                const float4 k4 = kv[r >> 2];
                const float kr = (r & 3) == 0 ? k4.x : (r & 3) == 1 ? k4.y : (r & 3) == 2 ? k4.z : k4.w;
                if constexpr (QS) {
                  const float4 d4 = dv[r >> 2];
                  const float dr = (r & 3) == 0 ? d4.x : (r & 3) == 1 ? d4.y : (r & 3) == 2 ? d4.z : d4.w;
                  val = __builtin_fmaf((float)s[t][r] * kr, cdq[blk], dr);
                } else {
                  val = (float)s[t][r] * kr;  // x dq sm_scale in the exponent
                }
              } else {
                const float4 d4 = dv[r >> 2];
                const float dr = (r & 3) == 0 ? d4.x : (r & 3) == 1 ? d4.y : (r & 3) == 2 ? d4.z : d4.w;
                val = __builtin_fmaf((float)s[t][r], cdq[LANE ? t : blk], dr);
              }
              f[16 * t + r] = out ? -INFINITY : val;
              mx = fmaxf(mx, f[16 * t + r]);
            }
          }
          mxf[blk] = mx;
          return;
        }
        int mx = INT_MIN;
#pragma unroll
        for (int t = 2 * blk; t < 2 * blk + 2; ++t) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool out = decltype(mask_tag)::value && 32 * t + 8 * (r >> 2) + (r & 3) > mlim;
            mx = max(mx, out ? INT_MIN : s[t][r]);
            f[16 * t + r] = out ? -INFINITY : (float)s[t][r];
          }
          if constexpr (LANE) {
            mxb[t] = mx;
            mx = INT_MIN;
          }
        }
        if constexpr (!LANE) mxb[blk] = mx;
      };
      // The MFMAs are issued inside each arm so that the unmasked arm's max and
      // conversion sit in the same basic block as the MFMAs and can fill their
      // issue gaps (the asm markers keep the compiler from hoisting the common
      // MFMA code above the branch).
      if (!need_mask) {
        asm volatile("; unmasked tile" ::: "memory");
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) qk_block(blk);
        dump_s();
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) max_convert(blk, 0, std::false_type());
      } else {
        // the mask bound passes through the asm so that its 64 comparisons
        // stay in this arm rather than being hoisted into the common path
        int mlim = lim;
        asm volatile("; masked tile" : "+v"(mlim) :: "memory");
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) qk_block(blk);
        dump_s();
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) max_convert(blk, mlim, std::true_type());
      }
      float mt = -INFINITY;
      if constexpr (FP4 || QS) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) mt = fmaxf(mt, mxf[blk] * a.sm2);
      } else if constexpr (TOKEN) {
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
          if (mxf[blk] != -INFINITY) mt = fmaxf(mt, mxf[blk] * c2[blk]);  // (c2 may be 0)
      } else {
#pragma unroll
        for (int i = 0; i < NC2; ++i)
          if (mxb[i] != INT_MIN) mt = fmaxf(mt, (float)mxb[i] * c2[i]);
      }
      mt = halves_max(mt);
      const float mn = fmaxf(m, mt);
      alpha = __builtin_amdgcn_exp2f(m - mn);
      const float sub = PV == 0 ? mn - kLog2_448 : mn;
      m = mn;
      // ---- p = exp2(s * c2 - sub)  (= 448 p~ in fp8 mode); masked keys are then
      //      zeroed in a separate pass that only boundary tiles take; row sum
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[16 * t + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[16 * t + r], c2[LANE ? t : t >> 1], -sub));
      if (need_mask) {
        int mlim = lim;
        asm volatile("; zero masked p" : "+v"(mlim) :: "memory");
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * t + 8 * (r >> 2) + (r & 3) > mlim) p[16 * t + r] = 0.0f;
      }
      l = alpha * l + tree_sum<16 * NT>(p);
    }

    if constexpr (PV == 0) {
      if (work) {
        // ---- P~ -> E4M3: byte 16t' + r of operand blk = key of s[2 blk + t'][r]
        v8i pk[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int i0 = 32 * blk + 4 * w;
            // the word's upper half is written by the next conversion; its
            // initial content is p[i0]'s register, dead after this use
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[i0], p[i0 + 1], __float_as_int(p[i0]), false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(p[i0 + 2], p[i0 + 3], word, true);
            pk[blk][w] = word;
          }
        // ---- O^T = alpha * O^T + V^T . P^T.  Two-level accumulation: each MFMA
        //      sums its 64 FP8 products in the matrix core's own accumulator
        //      (level 1) and adds that partial sum to the fp32 O registers passed
        //      as its C operand (level 2).  O is rescaled in place first; the
        //      rescale is skipped when no row of the wavefront changed its max.
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[c][r] *= alpha;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) {
            const int row = blk * D + 32 * c + qn;
            const v4i lo = *reinterpret_cast<const v4i *>(vb + row * 64 + 16 * swz<4>(2 * hh, row));
            const v4i hi = *reinterpret_cast<const v4i *>(vb + row * 64 + 16 * swz<4>(2 * hh + 1, row));
            const v8i vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            O[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pk[blk], O[c], 0, 0, 0, 0, 0, 0);
          }
        }
      }
    } else {
      // ---- pv fp16: P~ -> fp16 and O rescaled while the V copy lands; then
      //      O^T += V^T . P^T with fp32 accumulation in the MFMA, V^T read from
      //      the raw rows with transposing LDS loads
      v8h ph[2 * NT];
      if (work) {
#pragma unroll
        for (int s8 = 0; s8 < 2 * NT; ++s8)
#pragma unroll
          for (int i = 0; i < 8; ++i) ph[s8][i] = (_Float16)p[8 * s8 + i];
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[c][r] *= alpha;
        }
      }
      wait_vm_n(pend);  // this wavefront's V copies have landed (the next K may still fly) ...
      if constexpr (DT == 1) vcopy.to_f16(vb, wave, lane);  // bf16 V: rounded to fp16 once per work-group
      __syncthreads();  // ... and every other wavefront's too
      if (work) {
#pragma unroll
        for (int sb = 0; sb < 2 * NT; ++sb)
#pragma unroll
          for (int c = 0; c < NC; ++c)
            O[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfrag16<D>(vb, c, sb, lane), ph[sb], O[c], 0, 0, 0);
      }
    }
  };

  if (PV == 0 && tid < D) {
    vsc[tid] = a.v_scale[(long long)bhk * D + tid];
    vmn[tid] = a.v_mean ? a.v_mean[(long long)bhk * D + tid] : 0.0f;
  }

  // ---- main loop: tile j is computed from buffer j % NBUF while tiles
  //      j + 1 .. j + NBUF - 1 are in flight; one barrier per tile publishes the next
  constexpr int LPT = (PV == 0 ? 2 : 1) * TN * D / 1024 / WAVES;  // DMA instructions per tile per wavefront
  static_assert(NBUF == 2 || (TN * D / 1024) % WAVES == 0, "partial vm waits need an even copy split");
  static_assert(NBUF == 2 || !FP4, "partial vm waits assume the INT8 copy counts");
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u)
    if (u < ntiles) issue_tile(u, u, kbuf[u], vbuf[PV == 0 ? u : 0]);
  wait_vm<0>();
  __syncthreads();
  for (int j0 = 0; j0 < ntiles; j0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int j = j0 + u;
      if (j >= ntiles) break;
      const int jn = j + NBUF - 1;  // prefetch target, into the buffer freed by tile j - 1
      const int un = (u + NBUF - 1) % NBUF;
      // pv fp16: this tile's V rows go into the single V buffer, which the
      // barrier that ended the previous tile has released; issued ahead of the
      // prefetch so that the tile can wait for its V alone
      if constexpr (PV == 1) vcopy.issue(reinterpret_cast<const uint16_t *>(a.v), hv, j * TN, Sk, vbuf[0], wave);
      int pend = 0;
      if (jn < ntiles) pend = issue_tile(jn, un, kbuf[un], vbuf[PV == 0 ? un : 0]);
      tile(j, u, kbuf[u], vbuf[PV == 0 ? u : 0], pend);
      if (jn < ntiles) wait_vm<LPT * (NBUF - 2)>();  // tile j + 1 complete; later ones may still fly
      else wait_vm<0>();
      __syncthreads();
    }
  }

  if (!active) return;
  // ---- epilogue: combine the two half-wave sums, normalise, store
  const float lt = halves_sum(l);
  if (qi >= Sq) return;
  const float rl = lt > 0.0f ? 1.0f / lt : 0.0f;  // a row without keys (empty sequence) is 0
  const long long off = qs.base + (long long)qi * qs.stride;
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
        if (a.v_mean) {  // smoothed V: add the channel means back
          const float4 vm = *reinterpret_cast<const float4 *>(vmn + d0);
          o[0] += vm.x;
          o[1] += vm.y;
          o[2] += vm.z;
          o[3] += vm.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = O[c][4 * g + i] * rl;
      }
      store4<DT>(a.out, off + d0, o[0], o[1], o[2], o[3]);
    }
}

// Tile shape per mode: 128-key tiles at 2 wavefronts per SIMD (measured on
// MI355X against 64-key tiles at 2 and 3 wavefronts per SIMD: fewer row-max
// exchanges and O rescales per key outweigh the lower occupancy).
template <int PV>
struct TileCfg {
  static constexpr int TN = PV == 0 ? SAGE_ATTN_TN_FP8 : 128;
  static constexpr int WPS = PV == 0 ? SAGE_ATTN_WPS_FP8 : 2;
  static constexpr int WAVES = PV == 0 ? SAGE_ATTN_WAVES_FP8 : 4;
  static constexpr int NBUF = PV == 0 ? SAGE_ATTN_NBUF_FP8 : 2;
};

template <int D, int PV, int DT, bool CAUSAL, int QK>
static hipError_t launch5(const AttnArgs &a, bool dump, hipStream_t st) {
  using C = TileCfg<PV>;
  AttnArgs b = a;
  b.nmblk = (a.S + 32 * C::WAVES - 1) / (32 * C::WAVES);
  const dim3 grid(a.B * a.H * b.nmblk), block(64 * C::WAVES);
  // (the API rejects the dump for MXFP4 and for smoothed Q)
  if (a.delta_s)
    hipLaunchKernelGGL((k_attn<D, PV, DT, CAUSAL, false, QK, true, C::TN, C::WPS, C::WAVES, C::NBUF>), grid, block,
                       0, st, b);
  else if (dump)
    hipLaunchKernelGGL((k_attn<D, PV, DT, CAUSAL, QK != 2, QK, false, C::TN, C::WPS, C::WAVES, C::NBUF>), grid, block,
                       0, st, b);
  else
    hipLaunchKernelGGL((k_attn<D, PV, DT, CAUSAL, false, QK, false, C::TN, C::WPS, C::WAVES, C::NBUF>), grid, block,
                       0, st, b);
  return hipGetLastError();
}

template <int D, int PV, int DT, bool CAUSAL>
static hipError_t launch4(const AttnArgs &a, bool dump, hipStream_t st) {
  if (a.qk == 2) return launch5<D, PV, DT, CAUSAL, 2>(a, dump, st);
  if (a.qk == 3) return launch5<D, PV, DT, CAUSAL, 3>(a, dump, st);
  return a.qk == 1 ? launch5<D, PV, DT, CAUSAL, 1>(a, dump, st) : launch5<D, PV, DT, CAUSAL, 0>(a, dump, st);
}

template <int D, int PV, int DT>
static hipError_t launch3(const AttnArgs &a, bool dump, hipStream_t st) {
  return a.causal ? launch4<D, PV, DT, true>(a, dump, st) : launch4<D, PV, DT, false>(a, dump, st);
}

template <int D, int PV>
static hipError_t launch2(const AttnArgs &a, bool dump, hipStream_t st) {
  return a.dtype == 0 ? launch3<D, PV, 0>(a, dump, st) : launch3<D, PV, 1>(a, dump, st);
}

template <int D>
static hipError_t launch1(const AttnArgs &a, bool dump, hipStream_t st) {
  return a.pv == 0 ? launch2<D, 0>(a, dump, st) : launch2<D, 1>(a, dump, st);
}

int attn_tile_keys(int pv_mode) { return pv_mode == 0 ? TileCfg<0>::TN : TileCfg<1>::TN; }

hipError_t launch_attn(const AttnArgs &a, bool dump, hipStream_t stream) {
  return a.D == 64 ? launch1<64>(a, dump, stream) : launch1<128>(a, dump, stream);
}

}  // namespace sage
