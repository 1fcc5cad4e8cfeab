/*
 * sage.h -- C ABI of libsage: SageAttention-style quantized attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (web pages describing SageAttention, cited by title and section):
 *   [SA2]   "SageAttention2" paper summary, sections 相关工作 and SageAttention2方法:
 *           FlashAttention token-dim blocking; Q, K quantised to INT8 with K
 *           pre-processed (smoothed); P~ and V quantised to FP8 E4M3, P~ with a
 *           static scale and V per channel; a two-level accumulation into an
 *           FP32 buffer for the FP8 PV product.
 *   [KAI]   "Kairos的注意力加速利器：SageAttention INT8/FP8量化内核与FLA线性注意力解析指南",
 *           section 2.1 (INT8 QK^T with FP16 PV and fp32 accumulation, or FP8 PV
 *           with two-level accumulation) and 2.2 (per-block INT8, smoothing).
 *   [GUIDE] "SageAttention量化加速框架完整指南：从安装配置到性能调优的实战之路",
 *           section 五分钟跑通第一个加速样例 (sageattn(q, k, v, tensor_layout, is_causal),
 *           HND = (batch, head, seq, dim), NHD = (batch, seq, head, dim)),
 *           section 性能调优实战 (PV precision choice; layout and causality must match
 *           the tensors), section 替换时的三个注意事项 (no attention_mask argument) and
 *           section 最容易踩的四个安装坑 (unsupported GPUs raise an error).
 *   [REPO]  "SageAttention: Thư viện Attention lượng tử hóa" repository summary page,
 *           feature list (variable-length sequences through sageattn_varlen,
 *           native grouped-query attention).
 *   [OCP-MX] the Open Compute Project Microscaling (MX) Formats specification v1.0
 *           (public): the E2M1 element and E8M0 scale encodings of MXFP4, 32-element
 *           blocks.
 *
 * Pipeline: sage_smooth_quant_qk -> sage_quant_v (pv fp8) or sage_quant_v_fp4 (pv fp4)
 *           -> sage_attn_fwd; or, with INT8 per-block Q/K and unsmoothed Q, the Q/K pass
 *           without Q -> the V pass -> sage_attn_fwd_q16 (Q quantised in the attention
 *           kernel, same results).
 *
 * Common rules for every entry point:
 *  - Tensor pointers are DEVICE pointers; every call only enqueues work on
 *    `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 *    returns.  Inputs must stay alive and unmodified, and outputs untouched,
 *    until the stream has passed the call.  The caller owns all memory; the
 *    library allocates no device memory and keeps no per-call state.
 *  - Tensor pointers (q, k, v, out, q_codes, k_codes, v_fp8, dump buffers) must be
 *    16-byte aligned; scale / mean arrays 4-byte aligned.  Outputs must not
 *    overlap inputs.
 *  - Shapes: B, H >= 1; 1 <= S <= SAGE_MAX_S; D in {64, 128};
 *    B * H <= SAGE_MAX_BH.  K and V may have fewer heads than Q (grouped-query
 *    attention, [REPO] feature list): H_kv >= 1 divides H, and query head h
 *    uses K/V head h / (H / H_kv); H_kv = H is ordinary multi-head attention.
 *  - Errors are reported only through the return code.  All argument checks
 *    happen before anything is enqueued; on an error nothing is enqueued.
 *    SAGE_ERR_UNSUPPORTED means the current device is not gfx950.
 *  - Thread safety: calls may be made from several host threads; the only
 *    shared state is a per-device cache of the architecture check.
 *
 * Internal buffer layouts (all row-major, "[a][b]" = a outer):
 *   S_q = roundup(S, SAGE_BLK_Q), S_k = roundup(S, SAGE_KV_PAD),
 *   nq = S_q / SAGE_BLK_Q, nk = S_k / SAGE_BLK_K.
 *   q_codes int8  [B][H][S_q][D]   INT8 codes of Q; rows >= S are 0.
 *   q_scale float [B][H][nq]       one scale per block of SAGE_BLK_Q tokens
 *                                  (SAGE_QK_INT8_LANE, SAGE_QK_INT8_TOKEN: [B][H][S_q],
 *                                  one per token).
 *   k_codes int8  [B][H_kv][S_k][D] INT8 codes of K - k_mean; rows >= S are 0.
 *   k_scale float [B][H_kv][nk]    one scale per block of SAGE_BLK_K tokens (0 for blocks
 *                                  made only of padding keys; SAGE_QK_INT8_LANE:
 *                                  [B][H_kv][S_k / 16], one per lane group;
 *                                  SAGE_QK_INT8_TOKEN: [B][H_kv][S_k], one per token;
 *                                  SAGE_QK_INT8_HEAD: the per-block layouts of q_scale and
 *                                  k_scale, each slot holding its head's one scale).
 *   k_mean  float [B][H_kv][D]     per-channel mean of K over the S tokens.
 *   v_fp8   uint8 [B][H_kv][nk][D][64] E4M3 codes of V, one 64-key tile after the
 *           other, each tile stored channel-major; inside a tile, byte p of
 *           channel d holds key  SAGE_VPOS_KEY(p)  of that tile (keys >= S are 0).
 *   v_scale float [B][H_kv][D]     one scale per channel.
 *   v_mean  float [B][H_kv][D]     V smoothing only: the channel means subtracted from V
 *                                  before quantisation (same size as v_scale).
 *   q_mean  float [B][H][nq][D]    Q smoothing only: each Q block's channel means.
 *   delta_s float [B][H][S_k/128][nq][128]  Q smoothing only: the pre-processing term
 *           of query block blk and key n at [b][h][n / 128][blk][n % 128] (128-key
 *           tiles one after the other, so that each tile's rows are contiguous).
 *   pv fp4 (sage_quant_v_fp4) replaces v_fp8 and v_scale by
 *   v_codes uint8 [B][H_kv][nk][D][32]  E2M1 codes of V (or V - v_mean), per 64-key block
 *           and channel 32 bytes: nibble p (byte p / 2, the low nibble for even p) holds key
 *           SAGE_VPOS_KEY(p) of the block (keys >= S are 0);
 *   v_e8m0  uint8 [B][H_kv][nk][D][2]   the E8M0 byte of each block, channel and key group
 *           (group g: the block's keys n with (n / 4) mod 2 = g, i.e. nibbles 32 g .. 32 g + 31).
 *   SAGE_QK_MXFP4 replaces the Q/K codes and scales by (D / 2 and D / 32 bytes a row):
 *   q_codes uint8 [B][H][S_q][D/2]  E2M1 codes of Q, two per byte (channel 2j in the low
 *                                   nibble of byte j); q_scale uint8 [B][H][S_q][D/32], the
 *                                   E8M0 byte (e + 127) of each 32-channel block;
 *   k_codes uint8 [B][H_kv][S_k][D/2], k_scale uint8 [B][H_kv][S_k][D/32] likewise for
 *                                   K - k_mean.  Padding rows hold zero codes and byte 0.
 *   out: same dtype and layout (HND or NHD) as q.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define SAGE_OK 0
#define SAGE_ERR_INVALID_ARG 1 /* a null pointer, a bad shape / enum / alignment / sm_scale */
#define SAGE_ERR_UNSUPPORTED 2 /* the current device is not gfx950 */
#define SAGE_ERR_NO_DEVICE 3   /* no HIP device could be queried */
#define SAGE_ERR_LAUNCH 4      /* the HIP runtime rejected a kernel launch */

/* ---- enums ---- */
#define SAGE_LAYOUT_HND 0 /* [B][H][S][D] */
#define SAGE_LAYOUT_NHD 1 /* [B][S][H][D] */
#define SAGE_DTYPE_F16 0
#define SAGE_DTYPE_BF16 1
#define SAGE_PV_FP8 0  /* P~ and V in E4M3, two-level fp32 accumulation ([SA2]) */
#define SAGE_PV_FP16 1 /* P~ and V in fp16, fp32 accumulation ([KAI] 2.1, sm80 row) */
#define SAGE_PV_FP4 2  /* P~ and V in MXFP4 ([KAI] 2.2, the FP4 micro-scaling kernels of the next
                          generation; [OCP-MX]): E2M1 codes, an E8M0 scale per 32-key group of
                          each query row (P~) and of each V channel (sage_quant_v_fp4), fp32
                          accumulation across tiles */
/* Quantisation of Q and K for the Q K^T product (qk_quant):
 * INT8 with a scale granularity ([KAI] 2.2 per_block / per_warp choice; [SA2]
 * SageAttention2方法, thread-level quantisation), or micro-scaled FP4 ([KAI] 2.2,
 * the FP4 micro-scaling kernels of the next generation). */
#define SAGE_QK_INT8_BLOCK 0 /* INT8, one scale per SAGE_BLK_Q query tokens / SAGE_BLK_K keys */
#define SAGE_QK_INT8_LANE 1  /* INT8, one scale per query token and per 16-key lane group:
                                the keys one half-wave holds of each 32-key sub-tile of the
                                32 x 32 INT8 MFMA result, group of key n = 2 (n / 32) +
                                ((n / 4) mod 2); every lane dequantises with one scale */
#define SAGE_QK_MXFP4 2      /* MXFP4 ([OCP-MX]): E2M1 codes, each 32-channel block of a
                                token sharing an E8M0 scale 2^e, e = floor(log2 amax) - 2,
                                clamped to [-127, 127] (-127 for an all-zero block); codes
                                E2M1(x / 2^e), round to nearest even, saturating at 6 */
#define SAGE_QK_INT8_TOKEN 3 /* INT8, one scale per query token and per key token ([REPO]
                                feature list: granularity per token, per head or per thread) */
#define SAGE_QK_INT8_HEAD 4  /* INT8, one scale for all of a head's Q tokens and one for all of
                                its K - k_mean tokens ([REPO] feature list); the per-block
                                buffer layout, every block slot holding the head's scale.
                                Not with smoothed Q (q_mean / delta_s give SAGE_ERR_INVALID_ARG) */

/* ---- limits and granularity ---- */
#define SAGE_BLK_Q 32 /* Q tokens per INT8 scale: one wavefront's 32-row MFMA tile */
#define SAGE_BLK_K 64 /* K tokens per INT8 scale: one 64-key block of the attention loop */
#define SAGE_KV_PAD 128 /* K / V buffers are padded to whole 128-key tiles */
/* Keys per online-softmax tile of sage_attn_fwd (FlashAttention blocking); the
 * FP8 rounding of P~ and the fold of the two-level accumulation happen per tile. */
#define SAGE_TILE_K_FP8 128
#define SAGE_TILE_K_FP16 128
#define SAGE_MAX_S (1 << 20)
#define SAGE_MAX_BH (1 << 16)
/* key held by byte p (0..63) of a v_fp8 tile row */
#define SAGE_VPOS_KEY(p) (32 * (((p) & 31) >> 4) + 8 * (((p) & 15) >> 2) + 4 * ((p) >> 5) + ((p) & 3))

/* Quantisation granularity (tokens per scale) and the attention key tile per
 * pv mode used by every entry point (the constants above). */
int sage_get_config(int *blk_q, int *blk_k, int *tile_k_fp8, int *tile_k_fp16);

/* Bytes of each intermediate buffer for a problem shape (see the layouts
 * above).  Any output pointer may be NULL. */
int sage_buffer_sizes(int B, int H, int H_kv, int S, int D, int qk_quant, size_t *q_codes, size_t *q_scale,
                      size_t *k_codes, size_t *k_scale, size_t *k_mean, size_t *v_fp8, size_t *v_scale,
                      size_t *q_mean, size_t *delta_s);

/*
 * K smoothing + per-block INT8 quantisation of Q and K ([SA2] 相关工作,
 * SageAttention2方法; [KAI] 2.2).
 *   k_mean[d] = fp32( (sum_s K[s][d], summed in binary64) / S )
 *   blocks of SAGE_BLK_Q tokens of Q, and of SAGE_BLK_K tokens of K - k_mean
 *   (one fp32 subtraction per element), each over all D channels:
 *     amax = max |x|;  scale = amax / 127;  code = rint(x * (127 / amax)) in [-127, 127];
 *     an all-zero block has scale 0 and codes 0.   (IEEE fp32, round half to even)
 *   qk_quant = SAGE_QK_INT8_LANE: the same rule with each Q token, and each 16-key lane
 *   group of K - k_mean, as its own block; SAGE_QK_INT8_TOKEN: with each Q token and
 *   each token of K - k_mean as its own block; SAGE_QK_INT8_HEAD: with all of a head's
 *   tokens of Q, and of K - k_mean, as one block; SAGE_QK_MXFP4: the MXFP4 rule above on each
 *   32-channel block of every Q token and of every token of K - k_mean.
 * q: dtype (SAGE_DTYPE_*) tensor in `layout` (SAGE_LAYOUT_*) with H heads; k: the
 * same with H_kv heads.
 * q_mean non-NULL selects smoothed Q ([SA2] SageAttention2方法; any qk_quant): each
 * SAGE_BLK_Q-token block's channel means (binary64 sums over its valid tokens divided
 * by their number, rounded once) are written to q_mean, fp32 [B][H][nq][D], and
 * subtracted (one fp32 subtraction) before the INT8 or MXFP4 rule; sage_qk_delta then forms the
 * term the attention adds back.
 * Writes q_codes, q_scale, k_codes, k_scale, k_mean (layouts above; their element
 * types follow qk_quant).  q, q_codes and q_scale may all be NULL with
 * SAGE_QK_INT8_BLOCK and q_mean = NULL: K alone is smoothed and quantised, for
 * sage_attn_fwd_q16, which quantises Q itself.  The call is several kernel launches; while it runs,
 * k_codes also holds intermediate
 * per-chunk channel sums, so its content is defined only after the stream has
 * passed the call.
 */
int sage_smooth_quant_qk(const void *q, const void *k, int dtype, int B, int H, int H_kv, int S, int D,
                         int layout, int qk_quant, void *q_codes, void *q_scale, void *k_codes, void *k_scale,
                         float *k_mean, float *q_mean, void *stream);

/*
 * The pre-processing stage of smoothed Q ([SA2] SageAttention2方法: Q minus its block
 * means, with K smoothing, splits Q K^T into a pre-processing and an attention stage):
 *   delta_s[b][h][blk][n] = sum_d q_mean[b][h][blk][d] * (K[b][h / (H / H_kv)][n][d] - k_mean[d])
 * for n < S, 0 for the padding keys n < S_k, evaluated as q_mean . K - q_mean . k_mean
 * with fp32 accumulation of exact products (q_mean enters as 16-bit pieces: 2^-22
 * relative residual for fp16 inputs, exact for bf16).  q_mean and k_mean: from
 * sage_smooth_quant_qk called with q_mean (16-byte aligned); k: the same K tensor.
 * delta_s: the tiled layout above (16-byte aligned): fp32, or with qk_quant =
 * SAGE_QK_INT8_BLOCK the int32 rint(delta / (u * k_scale[key block])) in the score units
 * of its Q block, u = max(q_scale[blk], 127 * sum_d |q_mean[blk][d]| * 2^-30) (fp32,
 * the sum in channel order), which the attention uses as the starting value of the INT8
 * accumulator (q_scale, k_scale: from the same sage_smooth_quant_qk call; ignored
 * otherwise).  The attention then adds delta * sm_scale to every score.  qk_quant as
 * given to sage_smooth_quant_qk (not SAGE_QK_INT8_HEAD).  is_causal (0 or 1): 1 forms
 * only what a causal attention reads -- for each 128-key tile n0 .. n0 + 127 the rows
 * of the query blocks whose last query 32 blk + 31 is >= n0 (a causal query sees no
 * later key), in chunks of 32 blocks from a multiple of 32 -- and leaves the other
 * rows unwritten; the term is then only valid for sage_attn_fwd with is_causal = 1.
 */
int sage_qk_delta(const void *k, int dtype, int B, int H, int H_kv, int S, int D, int layout, int qk_quant,
                  int is_causal, const float *q_mean, const float *k_mean, const void *q_scale, const void *k_scale,
                  float *delta_s, void *stream);

/*
 * Per-channel FP8 E4M3 quantisation of V ([SA2] SageAttention2方法):
 *   amax_d = max_s |V[s][d]|;  v_scale[d] = amax_d / 448;
 *   code = E4M3(V[s][d] * (448 / amax_d)), round to nearest even, |x| clamped to 448;
 *   an all-zero channel has scale 0 and codes 0.
 * H is the number of V heads (H_kv of the other entry points).
 * v_mean non-NULL selects V smoothing ([SA2] SageAttention2方法, optional smooth V):
 *   v_mean[d] = fp32( (sum_s V[s][d], binary64) / S ), the rule above is applied to
 *   V[s][d] - v_mean[d] (one fp32 subtraction), and sage_attn_fwd adds v_mean back.
 * Writes v_fp8 in the tiled layout above, v_scale (and v_mean).  While the call's
 * launches run, v_fp8 and v_scale hold intermediate per-channel statistics, so
 * they are defined only after the stream has passed the call.
 */
int sage_quant_v(const void *v, int dtype, int B, int H, int S, int D, int layout, uint8_t *v_fp8,
                 float *v_scale, float *v_mean, void *stream);

/*
 * MXFP4 quantisation of V for the FP4 P~ V product (SAGE_PV_FP4; [KAI] 2.2; [OCP-MX]):
 * for each 64-key block, channel d and key group g (the block's keys n with
 * (n / 4) mod 2 = g; 32 keys, padding keys >= S counting as 0):
 *   amax = max |x|;  e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 if amax = 0);
 *   v_e8m0 = e + 127;  code = E2M1(x / 2^e), round to nearest even, saturating at 6,
 * with x = V[s][d], or V[s][d] - v_mean[d] (one fp32 subtraction) when v_mean is
 * non-NULL (V smoothing, the means as in sage_quant_v; sage_attn_fwd adds them back).
 * H is the number of V heads.  Buffer sizes: sage_v_fp4_buffer_sizes.  v_codes 16-byte,
 * v_e8m0 4-byte aligned.  With v_mean, both buffers hold intermediate statistics while
 * the call's launches run (defined once the stream has passed the call).
 */
int sage_quant_v_fp4(const void *v, int dtype, int B, int H, int S, int D, int layout, uint8_t *v_codes,
                     uint8_t *v_e8m0, float *v_mean, void *stream);

/* Bytes of v_codes and v_e8m0 of sage_quant_v_fp4 (either pointer may be NULL). */
int sage_v_fp4_buffer_sizes(int B, int H_kv, int S, int D, size_t *v_codes, size_t *v_e8m0);

/*
 * sage_smooth_quant_qk followed by sage_quant_v (on V's H_kv heads), in one call:
 * the same arguments, checks and results (every output buffer bit for bit), with
 * the passes that do not depend on each other sharing kernel launches (four
 * launches instead of eight).  For pv fp8; v: the V tensor (dtype, layout,
 * H_kv heads).  q_mean and v_mean select Q and V smoothing as in the two calls, and
 * q, q_codes, q_scale may all be NULL as in sage_smooth_quant_qk (K and V only).
 */
int sage_quantize_qkv(const void *q, const void *k, const void *v, int dtype, int B, int H, int H_kv, int S, int D,
                      int layout, int qk_quant, void *q_codes, void *q_scale, void *k_codes, void *k_scale,
                      float *k_mean, float *q_mean, uint8_t *v_fp8, float *v_scale, float *v_mean, void *stream);

/*
 * Fused quantized attention ([SA2]; [KAI] 2.1; [GUIDE] 五分钟跑通, 性能调优实战).
 * For each query row i, key tiles (SAGE_TILE_K_FP8 / SAGE_TILE_K_FP16 keys) in order,
 * fp32 online softmax:
 *   s_n = float(q_codes[i] . k_codes[n]) * (q_scale * k_scale) * sm_scale   (INT8 MFMA,
 *         int32 sums; the scales of query i's block and key n's block, lane group or
 *         token);
 *         SAGE_QK_MXFP4: s_n = (sum_d Q~[i][d] K~[n][d]) * sm_scale over the dequantised
 *         E2M1 * 2^e values (scaled FP4 MFMA, fp32 sums).  qk_quant must be the mode
 *         the codes were made with.
 *   keys n >= S, and n > i when is_causal (square, top-left aligned), are excluded
 *   m' = max(m, max_n s_n);  alpha = exp(m - m');  p_n = exp(s_n - m');  l = alpha*l + sum p_n
 *   pv fp8 : P = E4M3(448 * p_n) (static scale), inner = P . V_fp8 (FP8 MFMA, fresh per tile),
 *            O = alpha*O + inner (fp32 buffer);  out = O * v_scale[d] / (448 * l)
 *            (+ v_mean[d] when v_mean is non-NULL: V was smoothed by sage_quant_v)
 *   smoothed Q (delta_s non-NULL): s_n += delta_s[query block][n] * sm_scale (MXFP4: the
 *         term is the starting value of the fp32 accumulator the FP4 MFMA adds to; INT8
 *         per-block scales: delta_s holds the term in score units, the starting value of
 *         the INT8 accumulator, and the block's scale is u of sage_qk_delta -- a block with
 *         u > q_scale drops its INT8 codes, its residual being below fp32 resolution of
 *         q_mean)
 *   pv fp16: P = fp16(p_n), O = alpha*O + P . fp16(V) (fp32);  out = O / l
 *   pv fp4 : for each 32-key group G of a row (keys of one 64-key block with equal
 *            (n / 4) mod 2): e = floor(log2 max_G p_n) - 2 (clamped to [-126, 127]),
 *            P_n = dec(E2M1(p_n / 2^e)) 2^e; inner = P . dec(V) (scaled FP4 MFMA, V from
 *            sage_quant_v_fp4), O = alpha*O + inner;  l sums the P_n;
 *            out = O / l (+ v_mean[d] when V was smoothed)
 * q_codes .. k_scale: from sage_smooth_quant_qk.  pv fp8: v = v_fp8 and v_scale from
 * sage_quant_v, v_mean = NULL or the means sage_quant_v wrote.  pv fp16: v = the
 * original V tensor (dtype, layout, H_kv heads), v_scale = v_mean = NULL (bf16 V is
 * rounded to fp16).  delta_s: NULL, or the buffer sage_qk_delta filled for these
 * codes; q_mean: with delta_s and SAGE_QK_INT8_BLOCK the block means sage_smooth_quant_qk
 * wrote (they fix the score units), else not read (may be NULL).  pv fp4: v = v_codes and v_scale = v_e8m0 (the byte buffer passed as a
 * float pointer, 4-byte aligned) from sage_quant_v_fp4, v_mean as for pv fp8.
 * out: dtype tensor in `layout`, shape of q.  Query head h reads K/V head
 * h / (H / H_kv).
 * is_causal in {0, 1}; sm_scale finite and > 0 (the usual choice is 1/sqrt(D)).
 * pv fp16 with NHD layout additionally needs H_kv * D * 2 * SAGE_KV_PAD < 2^31
 * (128-token slices of V are addressed through a 32-bit byte range).
 */
int sage_attn_fwd(const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale,
                  const void *v, const float *v_scale, const float *v_mean, const float *q_mean, const float *delta_s,
                  void *out, int dtype, int B, int H, int H_kv, int S, int D, int layout, int is_causal,
                  float sm_scale, int pv_mode, int qk_quant, void *stream);

/*
 * sage_attn_fwd with the Q quantisation folded in (SAGE_QK_INT8_BLOCK, unsmoothed Q):
 * q is the dtype tensor of sage_smooth_quant_qk (16-byte aligned), and each
 * SAGE_BLK_Q-token block of it is quantised inside the attention kernel by the rule
 * of the Q pass -- block abs-max over its valid tokens, code = clamp(rint(x * (127 /
 * amax)), -127, 127), scale amax / 127, in the same fp32 operations -- so the codes,
 * and the output, are bit-identical to sage_smooth_quant_qk followed by sage_attn_fwd
 * with SAGE_QK_INT8_BLOCK.  This saves the Q pass's read of q and write of the codes
 * and the attention's read of the codes.  k_codes, k_scale: from sage_smooth_quant_qk
 * or sage_quantize_qkv with SAGE_QK_INT8_BLOCK (either may omit Q); the other
 * arguments as in sage_attn_fwd.
 */
int sage_attn_fwd_q16(const void *q, const void *k_codes, const void *k_scale, const void *v, const float *v_scale,
                      const float *v_mean, void *out, int dtype, int B, int H, int H_kv, int S, int D, int layout,
                      int is_causal, float sm_scale, int pv_mode, void *stream);

/*
 * Debug variant of sage_attn_fwd (INT8 modes, no smoothed-Q term): the same
 * kernel code, which additionally writes the int32 accumulators of Q K^T for
 * query head (b, h) to qk, an int32 [S][S] array:
 *   qk[i][n] = sum_d q_codes[i][d] * k_codes[n][d].
 * With is_causal, entries with n > i may be left unwritten (key tiles the mask
 * excludes for a whole work-group are skipped); every entry with n <= i is
 * written.  `out` is written as by sage_attn_fwd.
 */
int sage_attn_fwd_dump_qk(const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale,
                          const void *v, const float *v_scale, const float *v_mean, void *out, int dtype, int B,
                          int H, int H_kv, int S, int D, int layout, int is_causal, float sm_scale, int pv_mode,
                          int qk_quant, int b, int h, int32_t *qk, void *stream);

/* ------------------------------------------------------------------------
 * Packed variable-length batches ([REPO] feature list: variable-length
 * sequences through sageattn_varlen).
 *
 * q: [total_q][H][D], k and v: [total_k][H_kv][D], token-major (NHD without
 * the batch axis), dtype as above.  Sequence b owns rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1 of k and v.  cu_seqlens_q, cu_seqlens_k: device int32
 * arrays of B + 1 entries that start at 0, do not decrease and end at total_q /
 * total_k.  max_seqlen_q, max_seqlen_k: host-side bounds of every sequence
 * length, 1 .. SAGE_MAX_S (launch sizes follow them, so tight bounds are
 * faster).  The tables live on the device and are not checked: entries that
 * break these rules cannot make any access leave the buffers (each length is
 * clamped to [0, total] and to max_seqlen) but give unspecified results.
 *
 * Each sequence is attended on its own, exactly as a fixed-length batch of one:
 * its own K mean, INT8 blocks, V scales and causal mask (key n is kept for
 * query i when n <= i, both counted from the sequence's first token; query and
 * key lengths may differ).  A query row that sees no key (a sequence with no
 * keys) is 0.
 *
 * Intermediate buffers (sizes from sage_varlen_buffer_sizes).  Per head, the
 * rows of sequence b start at
 *   rq(b) = 32 * (cu_seqlens_q[b] / 32 + b),  rk(b) = 128 * (cu_seqlens_k[b] / 128 + b)
 * of RQ = 32 * (total_q / 32 + B + 1) and RK = 128 * (total_k / 128 + B + 1) rows:
 *   q_codes int8  [H][RQ][D]          q_scale float [H][RQ / 32]    (lane, token: [H][RQ])
 *   k_codes int8  [H_kv][RK][D]       k_scale float [H_kv][RK / 64] (lane: [H_kv][RK / 16];
 *                                                                    token: [H_kv][RK])
 *   (MXFP4: codes D / 2 and scales D / 32 bytes a row, as in the fixed layout)
 *   k_mean  float [B][H_kv][D]        v_scale float [B][H_kv][D]
 *   v_fp8   uint8 [H_kv][RK / 64][D][64]  (64-key tiles as in the fixed layout)
 * Smoothed Q (sizes from sage_varlen_smooth_q_sizes; any qk_quant but
 * SAGE_QK_INT8_HEAD):
 *   q_mean  float [H][RQ / 32][D]    each Q block's channel means (block rows as q_codes)
 *   delta_s float [H][RK / 128][MQ][128]  the pre-processing term, MQ = ceil(max_seqlen_q
 *           / 32): per query head and 128-row tile of the K buffer, the MQ query-block
 *           rows of 128 keys; sequence b's tiles hold its own query blocks 0 ..
 *           ceil(len_q(b) / 32) - 1 (the rest is neither written nor read).
 * A sequence's rows past its length, up to the next multiple of 32 (Q) or 128
 * (K, V), hold zero codes; rows between sequences are neither written nor read.
 * Other rules (alignment, errors, stream order, staging) as above.
 * ------------------------------------------------------------------------ */
int sage_varlen_buffer_sizes(int B, int H, int H_kv, int total_q, int total_k, int D, int qk_quant,
                             size_t *q_codes, size_t *q_scale, size_t *k_codes, size_t *k_scale, size_t *k_mean,
                             size_t *v_fp8, size_t *v_scale);

/* Bytes of q_mean and delta_s for smoothed Q on a packed batch (layouts above;
 * either pointer may be NULL).  Errors as sage_varlen_buffer_sizes. */
int sage_varlen_smooth_q_sizes(int B, int H, int total_q, int total_k, int max_seqlen_q, int D, size_t *q_mean,
                               size_t *delta_s);

/* sage_smooth_quant_qk for a packed batch; q_mean: NULL, or the [H][RQ / 32][D]
 * buffer of block means (smoothed Q, as in the fixed-length call: each block's
 * means are of the sequence's own tokens in it).  q, q_codes and q_scale may all be
 * NULL as in the fixed-length call (for sage_attn_fwd_varlen_q16). */
int sage_smooth_quant_qk_varlen(const void *q, const void *k, int dtype, const int32_t *cu_seqlens_q,
                                const int32_t *cu_seqlens_k, int B, int H, int H_kv, int total_q, int total_k,
                                int max_seqlen_q, int max_seqlen_k, int D, int qk_quant, void *q_codes,
                                void *q_scale, void *k_codes, void *k_scale, float *k_mean, float *q_mean,
                                void *stream);

/* sage_qk_delta for a packed batch: each sequence's query blocks against its own
 * keys and K mean (k: [total_k][H_kv][D]); q_mean, k_mean, q_scale, k_scale from
 * sage_smooth_quant_qk_varlen called with q_mean; delta_s: the layout above,
 * 16-byte aligned, in fp32 or (SAGE_QK_INT8_BLOCK) in score units, and is_causal
 * (tiles counted from the sequence's first key), as in the fixed-length call. */
int sage_qk_delta_varlen(const void *k, int dtype, const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int B,
                         int H, int H_kv, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D,
                         int qk_quant, int is_causal, const float *q_mean, const float *k_mean, const void *q_scale,
                         const void *k_scale, float *delta_s, void *stream);

/* sage_quant_v for a packed batch (v: [total_k][H_kv][D]); v_mean as there. */
int sage_quant_v_varlen(const void *v, int dtype, const int32_t *cu_seqlens_k, int B, int H_kv, int total_k,
                        int max_seqlen_k, int D, uint8_t *v_fp8, float *v_scale, float *v_mean, void *stream);

/* Bytes of v_codes and v_e8m0 of sage_quant_v_fp4_varlen: [H_kv][RK / 64][D][32] and
 * [H_kv][RK / 64][D][2] (the fixed layout's 64-key blocks, rows as for v_fp8). */
int sage_varlen_v_fp4_buffer_sizes(int B, int H_kv, int total_k, int D, size_t *v_codes, size_t *v_e8m0);

/* sage_quant_v_fp4 for a packed batch (v: [total_k][H_kv][D]); v_mean as there. */
int sage_quant_v_fp4_varlen(const void *v, int dtype, const int32_t *cu_seqlens_k, int B, int H_kv, int total_k,
                            int max_seqlen_k, int D, uint8_t *v_codes, uint8_t *v_e8m0, float *v_mean,
                            void *stream);

/* sage_attn_fwd for a packed batch.  pv fp16: v = the original [total_k][H_kv][D]
 * V, v_scale = v_mean = NULL.  q_mean, delta_s: NULL, or smoothed Q's buffers
 * (sage_smooth_quant_qk_varlen, sage_qk_delta_varlen), as in the fixed-length
 * call.  out: [total_q][H][D] in dtype. */
int sage_attn_fwd_varlen(const void *q_codes, const void *q_scale, const void *k_codes, const void *k_scale,
                         const void *v, const float *v_scale, const float *v_mean, const float *q_mean,
                         const float *delta_s, void *out, int dtype,
                         const int32_t *cu_seqlens_q,
                         const int32_t *cu_seqlens_k, int B, int H, int H_kv, int total_q, int total_k,
                         int max_seqlen_q, int max_seqlen_k, int D, int is_causal, float sm_scale, int pv_mode,
                         int qk_quant, void *stream);

/* sage_attn_fwd_varlen with the Q quantisation folded in, as sage_attn_fwd_q16: q is
 * the packed [total_q][H][D] dtype tensor; each sequence's 32-token blocks (from its
 * first token) are quantised in the kernel. */
int sage_attn_fwd_varlen_q16(const void *q, const void *k_codes, const void *k_scale, const void *v,
                             const float *v_scale, const float *v_mean, void *out, int dtype,
                             const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int B, int H, int H_kv,
                             int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int D, int is_causal,
                             float sm_scale, int pv_mode, void *stream);

/* Human-readable name of a status code (static string). */
const char *sage_status_str(int status);

/* Pure check of an architecture name as reported by hipDeviceProp_t::gcnArchName
 * (e.g. "gfx950:sramecc+:xnack-"): SAGE_OK for gfx950, else SAGE_ERR_UNSUPPORTED
 * (SAGE_ERR_INVALID_ARG for NULL).  Touches no device. */
int sage_check_arch(const char *gcn_arch_name);

#ifdef __cplusplus
}
#endif
#endif
