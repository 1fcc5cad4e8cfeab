// attn.hip -- fused quantized attention for gfx950.
//
// Method ("SageAttention2" summary, sections 相关工作 and SageAttention2方法;
// "Kairos" guide, sections 2.1 and 2.2): INT8 Q.K^T with int32 accumulation,
// dequantised by the product of the Q-block and K-block scales; an online
// fp32 softmax over key tiles (FlashAttention blocking); P~ quantised to FP8
// E4M3 with the static scale 448 and multiplied with per-channel FP8 V; the
// FP8 products of one tile are summed by the MFMA into a fresh accumulator and
// then folded into an fp32 output buffer (two-level accumulation).  A pv fp16
// mode keeps P~ and V in fp16 with fp32 accumulation; a pv fp4 mode quantises
// P~ and V to MXFP4 (E2M1 codes, an E8M0 scale per 32-key group of each query
// row and of each V channel) for the scaled FP4 MFMA ("Kairos" guide, 2.2).
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
//  * the softmax denominator sums the same E4M3 weights: one
//    v_mfma_f32_16x16x128_f8f6f4 per 64-key block multiplies them by a lane
//    selector of ones (rowsum_ones) and leaves each lane its own query's sum,
//    instead of 64 fp32 adds per lane and tile (pv fp16: v_dot2_f32_f16 on the
//    fp16 weights, two per instruction);
//  * work-groups are numbered so that each XCD (own L2) works through whole
//    heads; causal work is issued longest query blocks first.
#include "attn_common.h"

namespace sage {

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
#endif

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
template <int D, int PV, int DT, bool CAUSAL, bool DUMP, int QK, bool QS, int TN, int WPS, int WAVES, int NBUF,
          bool QR = false>
__global__ __attribute__((amdgpu_flat_work_group_size(WAVES * 64, WAVES * 64), amdgpu_waves_per_eu(WPS, WPS))) void
k_attn(const AttnArgs a) {
  constexpr bool LANE = QK == 1, FP4 = QK == 2, TOKEN = QK == 3;
  // smoothed Q with INT8 per-block scales: delta arrives in units of the block's
  // score scale and starts the INT8 MFMA accumulator (QSI); with the other
  // formats it is an fp32 term added to the scores (QSF)
  constexpr bool QSI = QS && QK == 0, QSF = QS && !QSI;
  // QR: Q arrives as the 16-bit input and each wavefront quantises its own
  // 32-row block (INT8 per block) before the key loop
  static_assert(!QR || (QK == 0 && !QS && !DUMP), "in-kernel Q quantisation: INT8 per block, plain Q");
  constexpr int kBlockM = WAVES * 32;
  constexpr int NC = D / 32;
  constexpr int KCH = D / 16;
  constexpr int NB = TN / 64;                                // INT8 K blocks per tile
  constexpr int NT = TN / 32;                                // 32-key sub-tiles per tile
  constexpr int KBYTES = TN * D;                             // K tile
  // V tile in LDS -- fp8: NB 64-key blocks of E4M3 codes; fp16: TN raw 16-bit
  // rows; fp4: NB 64-key blocks of packed E2M1 codes ([block][channel][32 bytes])
  // then their E8M0 bytes ([block][channel][key group]), padded to 1 KiB
  constexpr int V4CODES = TN * D / 2, V4SC = NB * D * 2;
  constexpr int VBYTES = PV == 0 ? TN * D : PV == 1 ? 2 * TN * D : (V4CODES + V4SC + 1023) / 1024 * 1024;
  constexpr int NVBUF = PV == 1 ? 1 : NBUF;                 // fp16 V: one buffer, refilled every tile
  // Every buffer of the multi-buffered tiles is a __shared__ variable of its
  // own.  The compiler gives distinct variables distinct alias scopes, so the
  // reads of the tile being computed do not wait for the copies in flight into
  // another buffer; within one array it would have to assume that they overlap
  // and wait for the next tile's copies before reading this one.
  static_assert(NBUF >= 2 && NBUF <= 3, "two or three tile buffers");
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf2[NBUF > 2 ? KBYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[NVBUF > 1 ? VBYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf2[NVBUF > 2 ? VBYTES : 16];
  __shared__ __attribute__((aligned(16))) float vsc[D];  // this head's V channel scales (pv fp8)
  __shared__ __attribute__((aligned(16))) float vmn[D];  // its channel means when V was smoothed
  // smoothed Q: each wavefront's row of the pre-processing term for the tile's keys
  __shared__ __attribute__((aligned(16))) float dsbuf0[QS ? WAVES : 1][QS ? TN : 4];
  __shared__ __attribute__((aligned(16))) float dsbuf1[QS ? WAVES : 1][QS ? TN : 4];
  __shared__ __attribute__((aligned(16))) float dsbuf2[QS && NBUF > 2 ? WAVES : 1][QS ? TN : 4];
  // per-token K scales: the tile's key scales (copied by the first TN / 64 wavefronts)
  __shared__ __attribute__((aligned(16))) float ksbuf0[TOKEN ? TN : 4];
  __shared__ __attribute__((aligned(16))) float ksbuf1[TOKEN ? TN : 4];
  static_assert(!TOKEN || (TN / 64 <= WAVES && NBUF == 2), "key-scale copy split and whole-tile vm waits");
  // buffer u (a compile-time constant wherever the unrolled loops below use these)
  auto kbuf = [&](int u) -> uint8_t * { return u == 0 ? kbuf0 : u == 1 ? kbuf1 : kbuf2; };
  auto vbuf = [&](int u) -> uint8_t * { return u == 0 ? vbuf0 : u == 1 ? vbuf1 : vbuf2; };
  auto dsbuf = [&](int u) -> float(*)[QS ? TN : 4] { return u == 0 ? dsbuf0 : u == 1 ? dsbuf1 : dsbuf2; };
  auto ksbuf = [&](int u) -> float * { return u == 0 ? ksbuf0 : ksbuf1; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: branches on it stay scalar
  const int hh = lane >> 5, qn = lane & 31;

  // ---- work-group -> (head, query block), XCD-aware
  int bh, mrank;
  map_work(a, CAUSAL, bh, mrank);
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
    } else if constexpr (QR) {
      // The INT8 rule of the Q pass ("SageAttention2" summary, per-block INT8
      // quantisation): the block's abs-max over its valid rows (rows past the
      // sequence are 0), code = clamp(rint(x * (127 / amax)), +-127), scale
      // amax / 127 -- the same fp32 operations, so the codes and the scale are
      // bit-identical to the pass's.  Lane (q, half) loads the 64 values it
      // holds as the MFMA operand: Q[q][32 c + 16 half .. +16].
      const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + qs.base + (long long)qi * qs.stride;
      float x[NC][16];
      float amax = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        v4i u[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
        if (qi < Sq) {
          u[0] = *reinterpret_cast<const v4i *>(qrow + 32 * c + 16 * hh);
          u[1] = *reinterpret_cast<const v4i *>(qrow + 32 * c + 16 * hh + 8);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t w = (uint32_t)u[i >> 3][(i >> 1) & 3];
          x[c][i] = in_to_f32<DT>((i & 1) ? w >> 16 : w & 0xffffu);
          amax = fmaxf(amax, fabsf(x[c][i]));
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
      dq = amax > 0.0f ? amax / 127.0f : 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float t = fminf(fmaxf(__builtin_rintf(x[c][4 * w + i] * inv), -127.0f), 127.0f);
            word |= (uint32_t)(uint8_t)(int8_t)(int)t << (8 * i);
          }
          qf[c][w] = (int)word;
        }
    } else {
      const int8_t *qrow = a.q_i8 + (qs.row0 + qi) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const v4i *>(qrow + 32 * c + 16 * hh);
      dq = LANE || TOKEN ? a.q_scale[qs.row0 + qi] : a.q_scale[(qs.row0 + qw) >> 5];
    }
  }
  if constexpr (QSI) {
    // the block's score scale, as the pre-processing pass forms it from the
    // block means; a block that takes the larger bound drops its INT8 codes
    // (every lane sums two or one of the D channels, then the wavefront)
    float sa = 0.0f;
    if (active) {
#pragma unroll
      for (int i = 0; i < D / 64; ++i) sa += fabsf(a.q_mean[(long long)((qs.row0 + qw) >> 5) * D + lane + 64 * i]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sa += __shfl_xor(sa, o, 64);
    const float dqe = smooth_q_unit(dq, sa);
    if (dqe > dq) {
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[c] = v4i{0, 0, 0, 0};
    }
    dq = dqe;
  }

  int ntiles = (Sk + TN - 1) / TN;
  if (CAUSAL) ntiles = min(ntiles, min(q0 + kBlockM - 1, Sk - 1) / TN + 1);

  float m = -INFINITY;  // running max (log2 domain, scaled scores)
  float l = 0.0f;       // pv fp16: running sum of the fp16 weights of this half-wave's keys
  // pv fp8 / fp4: running sum of the quantised weights over both half-waves, as
  // the fp32 accumulator of the row-sum product (element 0; the others are not read)
  v4f lacc = {0.0f, 0.0f, 0.0f, 0.0f};
  const v8i ones = PV == 2 ? rowsum_ones_fp4(lane) : rowsum_ones(lane);
  v16f O[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[c][r] = 0.0f;

  const int8_t *kbase = a.k_i8 + ks.row0 * (FP4 ? D / 2 : D);
  const uint8_t *vbase = reinterpret_cast<const uint8_t *>(a.v) + ks.row0 * (PV == 2 ? D / 2 : D);
  const uint8_t *v4sbase = reinterpret_cast<const uint8_t *>(a.v_scale) + ks.row0 * (D / 32);  // pv fp4 V scales
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
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(PV != 1 ? (const void *)vbase : (const void *)kbase,
                                               PV == 0 ? vbytes : PV == 2 ? ntiles * V4CODES : kbytes);
  const __amdgpu_buffer_rsrc_t v4srs = make_rsrc(v4sbase, PV == 2 ? ntiles * V4SC : 0);  // (pv fp16 copies V itself)
  // pv fp4 V codes: 1 KiB wave-copies of 32-byte channel rows, 16-byte chunks
  // swizzled by swz<2>, which depends on the row only through bit 3: copy w is
  // copy 0 shifted by 1 KiB w, and this is the lane's offset in copy 0
  const uint32_t v4off = (uint32_t)((lane >> 1) * 32 + 16 * swz<2>(lane & 1, lane >> 1));
  // smoothed Q: delta is stored [bh][128-key tile][query block][128]; this
  // wavefront's row of tile j (its query block) is 512 contiguous bytes at
  // dbase + j * dtile; only wavefronts with queries copy (a trailing wavefront's
  // block may not exist)
  // (packed batches: per query head, rows_k / 128 key tiles, the sequence's own
  // from its first K buffer row, and nq = the longest sequence's query blocks)
  const long long dtile0 = a.varlen ? (long long)h * (a.rows_k / kKvPad) + ((ks.row0 - (long long)hk * a.rows_k) >> 7)
                                    : (long long)bh * (a.S_k / kKvPad);
  const float *dbase = QS ? a.delta_s + (dtile0 * a.nq + (qw >> 5)) * kKvPad : nullptr;
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
    if constexpr (PV == 2) {  // FP4 V codes and scales
      constexpr int NCP = V4CODES / 1024;
#pragma unroll
      for (int i = 0; i < (NCP + WAVES - 1) / WAVES; ++i) {
        const int w = wave + WAVES * i;
        if (NCP % WAVES == 0 || w < NCP) dma16_buf(vrs, v4off, j * V4CODES + 1024 * w, vb + 1024 * w);
      }
      if (wave < V4SC / 256) dma4_buf(v4srs, (uint32_t)(4 * lane), j * V4SC + 256 * wave, vb + V4CODES + 256 * wave);
    }
    if constexpr (TOKEN) {
      // every wavefront needs every key's scale: the first TN / 64 copy them,
      // whether or not they have queries of their own
      if (wave < TN / 64) {
        dma4_buf(srs, (uint32_t)(4 * lane), 4 * (j * TN + 64 * wave),
                 reinterpret_cast<uint8_t *>(ksbuf(buf)) + 256 * wave);
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
                   reinterpret_cast<uint8_t *>(&dsbuf(buf)[wave][0]) + 256 * i);
        }
        n += TN / 64;
      }
    }
    return n;
  };

  // One TN-key tile: QK^T, online softmax, PV.  kb / vb: this tile's LDS.
  // pend (pv fp16): copy instructions this wavefront issued after the tile's V.
  // prefetch: issues the copies of a later tile, or nothing (called once on
  // every path, after the first K block's MFMAs where the wavefront has work,
  // so that its first LDS reads follow the barrier directly)
  auto tile = [&](int j, int buf, const uint8_t *kb, uint8_t *vb, int pend, auto &&prefetch) {
    const float *dsr = &dsbuf(QS ? buf : 0)[QS ? wave : 0][0];  // smoothed Q: this wavefront's delta row
    const float *ksr = ksbuf(TOKEN ? buf : 0);                   // per-token K: the tile's key scales
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
    float gq[NB];  // pv fp4: per block, this lane's largest exponent argument (its key group's largest weight)
    if (!work) prefetch();
    if (work) {
      // ---- S^T = K . Q^T for the NT 32-key sub-tiles, one INT8 K block (two
      //      sub-tiles) after the other, so that the first block's row max and
      //      int -> float conversion can run while the second block's MFMAs do
      using acc_t = typename std::conditional<FP4, v16f, v16i>::type;
      acc_t s[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] = 0;
      auto qk_block = [&](int blk) {
        if constexpr (QS && (FP4 || QSI)) {
          // smoothed Q on the FP4 product (fp32 accumulation) or with INT8
          // per-block scales (delta in score units, int32): the pre-processing
          // term of each key is the MFMA accumulator's starting value (keys
          // 8 (r / 4) + 4 hh + r % 4 of the sub-tile).  Read per block, after the
          // previous block's MFMAs were issued (the asm keeps the reads there), so
          // that only one block's starting values are live at a time.
          if (blk > 0) asm volatile("" ::: "memory");
#pragma unroll
          for (int t = 2 * blk; t < 2 * blk + 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const v4i d4 = *reinterpret_cast<const v4i *>(dsr + 32 * t + 8 * g + 4 * hh);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if constexpr (FP4) s[t][4 * g + e] = __int_as_float(d4[e]);
                else s[t][4 * g + e] = d4[e];
              }
            }
        }
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
      float cdq[NC2];  // smoothed Q (fp32 path): the dequantisation factor alone (sm_scale applied later)
      if constexpr (QSF) {
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
        if constexpr (FP4 || QSF || TOKEN) {  // fp32 scores: dequantised (+ delta), max in fp32
          float mx = -INFINITY;
#pragma unroll
          for (int t = 2 * blk; t < 2 * blk + 2; ++t) {
            float4 dv[4], kv[4];
            if constexpr (QSF && !FP4)
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
                if constexpr (QSF) {
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
      // the tile's row max from the block maxima (masked tiles: blocks whose keys
      // are all masked hold INT_MIN / -inf and are left out; unmasked tiles have none)
      auto tile_max = [&](auto mask_tag) -> float {
        constexpr bool MASKED = decltype(mask_tag)::value;
        float t = -INFINITY;
        if constexpr (FP4 || QSF) {
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) t = fmaxf(t, mxf[blk] * a.sm2);
        } else if constexpr (TOKEN) {
#pragma unroll
          for (int blk = 0; blk < NB; ++blk)
            if (!MASKED || mxf[blk] != -INFINITY) t = fmaxf(t, mxf[blk] * c2[blk]);  // (c2 may be 0)
        } else {
#pragma unroll
          for (int i = 0; i < NC2; ++i)
            if (!MASKED || mxb[i] != INT_MIN) t = fmaxf(t, (float)mxb[i] * c2[i]);
        }
        return t;
      };
      float mt;
      // The MFMAs are issued inside each arm so that the unmasked arm's max and
      // conversion sit in the same basic block as the MFMAs and can fill their
      // issue gaps (the asm markers keep the compiler from hoisting the common
      // MFMA code above the branch).
      if (!need_mask) {
        asm volatile("; unmasked tile" ::: "memory");
        qk_block(0);
        prefetch();
#pragma unroll
        for (int blk = 1; blk < NB; ++blk) qk_block(blk);
        dump_s();
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) max_convert(blk, 0, std::false_type());
        mt = tile_max(std::false_type());
      } else {
        // the mask bound passes through the asm so that its 64 comparisons
        // stay in this arm rather than being hoisted into the common path
        int mlim = lim;
        asm volatile("; masked tile" : "+v"(mlim) :: "memory");
        qk_block(0);
        prefetch();
#pragma unroll
        for (int blk = 1; blk < NB; ++blk) qk_block(blk);
        dump_s();
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) max_convert(blk, mlim, std::true_type());
        mt = tile_max(std::true_type());
        if constexpr (PV == 0) {
          // pv fp8 takes masked keys to weight 0 through exp2(-inf) alone: a
          // zero factor (an all-zero Q or K block, whose scores are all 0)
          // becomes the smallest normal float, so that -inf * c2 stays -inf
#pragma unroll
          for (int i = 0; i < NC2; ++i) c2[i] = fmaxf(c2[i], 0x1p-126f);
        }
      }
      mt = halves_max(mt);
      const float mn = fmaxf(m, mt);
      alpha = __builtin_amdgcn_exp2f(m - mn);
      const float sub = PV == 0 ? mn - kLog2_448 : mn;
      m = mn;
      if constexpr (PV == 2) {
        // log2 of each key group's largest weight, formed by the same FMA as the
        // weights below, plus a bound on that FMA's rounding against the row max
        // (the max is a rounded product, so the weight of the max key itself, 1 in
        // exact arithmetic, can come out a few ulps below 1; the MX exponent rule
        // would then drop a binade and saturate it to 6 * 2^-3 = 0.75).  With the
        // bound such a group takes the exponent of 1 and the key the code of 1.
        const float nudge = __builtin_fmaf(fabsf(sub), 0x1p-22f, 0x1p-24f);
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          // (the same arms as max_convert: fp32 maxima with smoothed Q, FP4 or
          // per-token scales; int32 maxima per lane group or per block otherwise)
          float g = -INFINITY;
          if constexpr (FP4 || QSF || TOKEN) {
            g = __builtin_fmaf(mxf[blk], c2[blk], -sub);
          } else if constexpr (LANE) {
#pragma unroll
            for (int t = 2 * blk; t < 2 * blk + 2; ++t)
              g = fmaxf(g, mxb[t] == INT_MIN ? -INFINITY : __builtin_fmaf((float)mxb[t], c2[t], -sub));
          } else {
            g = mxb[blk] == INT_MIN ? -INFINITY : __builtin_fmaf((float)mxb[blk], c2[blk], -sub);
          }
          gq[blk] = g + nudge;
        }
      }
      if constexpr (PV == 0) {
        // ---- pv fp8: O is rescaled first, so that the weights, their E4M3
        //      codes and the P V MFMAs of the tile form one basic block (the
        //      second block's exp2 and conversions can run under the first
        //      block's MFMAs).  p = exp2(s * c2 - sub) = 448 p~; masked keys
        //      (s = -inf) give 0.  Byte 16 t' + r of operand blk = key of
        //      s[2 blk + t'][r].  Two-level accumulation: each MFMA sums its 64
        //      FP8 products in the matrix core's own accumulator (level 1) and
        //      adds that partial sum to the fp32 O registers passed as its C
        //      operand (level 2).  The rescale is skipped when no row of the
        //      wavefront changed its max.
        // the first block's V fragments are read before the rescale, which
        // covers their LDS latency (the asm keeps the reads here)
        auto vfrag = [&](int blk, int c) -> v8i {
          const int row = blk * D + 32 * c + qn;
          const v4i lo = *reinterpret_cast<const v4i *>(vb + row * 64 + 16 * swz<4>(2 * hh, row));
          const v4i hi = *reinterpret_cast<const v4i *>(vb + row * 64 + 16 * swz<4>(2 * hh + 1, row));
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        v8i vf0[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) vf0[c] = vfrag(0, c);
        asm volatile("; v block 0 read" ::: "memory");
        lacc[0] *= alpha;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[c][r] *= alpha;
        }
        v8i pk[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int i0 = 32 * blk + 4 * w;
            float e[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int i = i0 + k;
              e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[i], c2[LANE ? i >> 4 : i >> 5], -sub));
            }
            // the word's upper half is written by the next conversion; its
            // initial content is e[0]'s register, dead after this use
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], __float_as_int(e[0]), false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], word, true);
            pk[blk][w] = word;
          }
          lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pk[blk], lacc, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const v8i vf = blk == 0 ? vf0[c] : vfrag(blk, c);
            O[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pk[blk], O[c], 0, 0, 0, 0, 0, 0);
          }
        }
      } else {
        // ---- pv fp16, fp4: p = exp2(s * c2 - sub) = p~; masked keys are then
        //      zeroed in a separate pass that only boundary tiles take
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            p[16 * t + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[16 * t + r], c2[LANE ? t : t >> 1], -sub));
        if (need_mask) {
          int mlim = lim;
          asm volatile("; zero masked p" : "+v"(mlim) :: "memory");
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * t + 8 * (r >> 2) + (r & 3) > mlim) p[16 * t + r] = 0.0f;
        }
      }
    }

    if constexpr (PV == 2) {
      if (work) {
        // ---- P~ -> MXFP4: this lane's 32 weights of each 64-key block are one
        //      key group; its E8M0 scale comes from the group's largest weight,
        //      formed by the same FMA and exp2 as that weight (so bit-identical),
        //      times 2^-2 (the MX rule); nibble 16 t' + r = weight of s[2 blk + t'][r]
        float sc[NB];
        int pe[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          // E8M0 byte = biased exponent of the group max, minus 2 (the MX rule);
          // the conversion takes the exponent of its scale operand, given here as
          // that power of two.  A group without weights (codes 0) takes the byte 1.
          const int ex = (int)((__float_as_uint(__builtin_amdgcn_exp2f(gq[blk])) >> 23) & 0xff);
          pe[blk] = max(ex - 2, 1);
          sc[blk] = __uint_as_float((uint32_t)pe[blk] << 23);
        }
        v8i pk[NB];
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int t = 2 * blk + (w >> 1), r0 = 8 * (w & 1);
            unsigned word = 0;
            static_for<0, 4>([&](auto SEL) {
              constexpr int sel = decltype(SEL)::value;
              const int i0 = 16 * t + r0 + 2 * sel;
              word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, p[i0], p[i0 + 1], sc[blk], sel);
            });
            pk[blk][w] = (int)word;
          }
#pragma unroll
          for (int w = 4; w < 8; ++w) pk[blk][w] = 0;
        }
        lacc[0] *= alpha;
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[c][r] *= alpha;
        }
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
          lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pk[blk], lacc, 4, 4, 0, 127, 0, pe[blk]);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) {
            const int row = blk * D + 32 * c + qn;
            const v4i vf = *reinterpret_cast<const v4i *>(vb + row * 32 + 16 * swz<2>(hh, row));
            const int vsb = vb[V4CODES + 2 * row + hh];
            const v8i va = {vf[0], vf[1], vf[2], vf[3], 0, 0, 0, 0};
            O[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pk[blk], O[c], 4, 4, 0, vsb, 0, pe[blk]);
          }
        }
      }
    } else if constexpr (PV == 0) {
      // (pv fp8: done above, with the weights)
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
        // row sum of the fp16 weights, two per v_dot2_f32_f16, in four chains
        const v2h one2 = {(_Float16)1.0f, (_Float16)1.0f};
        float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s8 = 0; s8 < 2 * NT; ++s8)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ls[i] = __builtin_amdgcn_fdot2(v2h{ph[s8][2 * i], ph[s8][2 * i + 1]}, one2, ls[i], false);
        l = alpha * l + ((ls[0] + ls[1]) + (ls[2] + ls[3]));
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

  if (PV != 1 && tid < D) {
    vsc[tid] = PV == 0 ? a.v_scale[(long long)bhk * D + tid] : 1.0f;
    vmn[tid] = a.v_mean ? a.v_mean[(long long)bhk * D + tid] : 0.0f;
  }

  // ---- main loop: tile j is computed from buffer j % NBUF while tiles
  //      j + 1 .. j + NBUF - 1 are in flight; one barrier per tile publishes the next
  constexpr int LPT = (PV == 0 ? 2 : 1) * TN * D / 1024 / WAVES;  // DMA instructions per tile per wavefront
  static_assert(PV != 2 || NBUF == 2, "pv fp4 copies count as whole-tile waits");
  static_assert(NBUF == 2 || (TN * D / 1024) % WAVES == 0, "partial vm waits need an even copy split");
  static_assert(NBUF == 2 || !FP4, "partial vm waits assume the INT8 copy counts");
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u)
    if (u < ntiles) issue_tile(u, u, kbuf(u), vbuf(PV != 1 ? u : 0));
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
      if constexpr (PV == 1) vcopy.issue(reinterpret_cast<const uint16_t *>(a.v), hv, j * TN, Sk, vbuf(0), wave);
      // non-causal pv fp8 issues the copies inside the tile, after the first
      // K block's MFMAs (elsewhere that costs registers: the copies go first)
      constexpr bool DEFER = PV == 0 && !CAUSAL;
      int pend = 0;
      if constexpr (!DEFER)
        if (jn < ntiles) pend = issue_tile(jn, un, kbuf(un), vbuf(PV != 1 ? un : 0));
      auto prefetch = [&]() {
        if constexpr (DEFER)
          if (jn < ntiles) issue_tile(jn, un, kbuf(un), vbuf(un));
      };
      tile(j, u, kbuf(u), vbuf(PV != 1 ? u : 0), pend, prefetch);
      if (jn < ntiles) wait_vm<LPT * (NBUF - 2)>();  // tile j + 1 complete; later ones may still fly
      else wait_vm<0>();
      __syncthreads();
    }
  }

  if (!active) return;
  // ---- epilogue: the row sum (pv fp16: combine the two half-wave sums), normalise, store
  const float lt = PV == 1 ? halves_sum(l) : lacc[0];
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
      } else {  // pv fp4: the V scales were applied inside the MFMA; pv fp16: unscaled V
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = O[c][4 * g + i] * rl;
      }
      if (PV != 1 && a.v_mean) {  // smoothed V: add the channel means back
        const float4 vm = *reinterpret_cast<const float4 *>(vmn + d0);
        o[0] += vm.x;
        o[1] += vm.y;
        o[2] += vm.z;
        o[3] += vm.w;
      }
      store4<DT>(a.out, off + d0, o[0], o[1], o[2], o[3]);
    }
}

// Tile shape per mode: 128-key tiles at 2 wavefronts per SIMD (measured on
// MI355X against 64-key tiles at 2 and 3 wavefronts per SIMD: fewer row-max
// exchanges and O rescales per key outweigh the lower occupancy).
template <int PV>
struct TileCfg {  // pv fp4 (PV == 2) shares the pv fp8 shape
  static constexpr int TN = PV != 1 ? SAGE_ATTN_TN_FP8 : 128;
  static constexpr int WPS = PV != 1 ? SAGE_ATTN_WPS_FP8 : 2;
  static constexpr int WAVES = PV != 1 ? SAGE_ATTN_WAVES_FP8 : 4;
  static constexpr int NBUF = PV != 1 ? SAGE_ATTN_NBUF_FP8 : 2;
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
  else if (a.q) {  // in-kernel Q quantisation (INT8 per block; the API admits no other format)
    if constexpr (QK == 0)
      hipLaunchKernelGGL((k_attn<D, PV, DT, CAUSAL, false, QK, false, C::TN, C::WPS, C::WAVES, C::NBUF, true>), grid,
                         block, 0, st, b);
    else
      return hipErrorInvalidValue;
  } else
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
  if (a.pv == 2) return launch2<D, 2>(a, dump, st);
  return a.pv == 0 ? launch2<D, 0>(a, dump, st) : launch2<D, 1>(a, dump, st);
}

int attn_tile_keys(int pv_mode) { return pv_mode == 1 ? TileCfg<1>::TN : TileCfg<0>::TN; }

hipError_t launch_attn(const AttnArgs &a, bool dump, hipStream_t stream) {
  return a.D == 64 ? launch1<64>(a, dump, stream) : launch1<128>(a, dump, stream);
}

}  // namespace sage
