"""SageAttention-style quantized attention for AMD Instinct MI355X (gfx950).

Thin Python binding over ``libsage.so`` (C ABI in ``include/sage.h``).  The
functions named ``sage_*`` mirror the C entry points one to one and only
marshal arguments: every step of the method runs in the HIP kernels.  PyTorch
is used for device memory and streams only.

``sageattn(q, k, v, tensor_layout="HND", is_causal=False, ...)`` chains the
three entry points the way the pages' high-level API is used ("完整指南" page,
section 五分钟跑通第一个加速样例): it allocates the intermediate buffers with
torch and returns a tensor shaped like ``q``.

There is no CPU fallback: if ``libsage.so`` is missing or the device is not a
gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsage.so")

SAGE_OK, SAGE_ERR_INVALID_ARG, SAGE_ERR_UNSUPPORTED, SAGE_ERR_NO_DEVICE, SAGE_ERR_LAUNCH = 0, 1, 2, 3, 4
LAYOUT = {"HND": 0, "NHD": 1}
DTYPE = {"fp16": 0, "bf16": 1}
PV = {"fp8": 0, "fp16": 1, "fp4": 2}
QK = {"int8": 0, "int8_lane": 1, "mxfp4": 2, "int8_token": 3, "int8_head": 4}  # Q/K quantisation (include/sage.h SAGE_QK_*)
BLK_Q, BLK_K, KV_PAD = 32, 64, 128
TILE_K = {"fp8": 128, "fp16": 128, "fp4": 128}  # keys per online-softmax tile of the attention kernel

EXPORTED = ["sage_get_config", "sage_buffer_sizes", "sage_smooth_quant_qk", "sage_quant_v", "sage_quantize_qkv", "sage_attn_fwd",
            "sage_attn_fwd_dump_qk", "sage_qk_delta", "sage_varlen_buffer_sizes", "sage_smooth_quant_qk_varlen", "sage_quant_v_varlen",
            "sage_attn_fwd_varlen", "sage_status_str", "sage_check_arch", "sage_quant_v_fp4", "sage_v_fp4_buffer_sizes",
            "sage_quant_v_fp4_varlen", "sage_varlen_v_fp4_buffer_sizes", "sage_varlen_smooth_q_sizes",
            "sage_qk_delta_varlen", "sage_attn_fwd_q16", "sage_attn_fwd_varlen_q16"]

_lib = None


class SageError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libsage.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m quantized_attention_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_float, c_void_p, c_size_p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
        L.sage_get_config.argtypes = [ctypes.POINTER(c_int)] * 4
        L.sage_buffer_sizes.argtypes = [c_int] * 6 + [c_size_p] * 9
        L.sage_smooth_quant_qk.argtypes = [c_void_p, c_void_p] + [c_int] * 8 + [c_void_p] * 6 + [c_void_p]
        L.sage_qk_delta.argtypes = [c_void_p] + [c_int] * 9 + [c_void_p] * 6
        L.sage_quant_v.argtypes = [c_void_p] + [c_int] * 6 + [c_void_p] * 4
        L.sage_quantize_qkv.argtypes = [c_void_p] * 3 + [c_int] * 8 + [c_void_p] * 10
        tail = [c_int] * 8 + [c_float, c_int, c_int]
        L.sage_attn_fwd.argtypes = [c_void_p] * 10 + tail + [c_void_p]
        L.sage_attn_fwd_dump_qk.argtypes = [c_void_p] * 8 + tail + [c_int, c_int, c_void_p, c_void_p]
        L.sage_varlen_buffer_sizes.argtypes = [c_int] * 7 + [c_size_p] * 7
        L.sage_smooth_quant_qk_varlen.argtypes = [c_void_p, c_void_p, c_int, c_void_p, c_void_p] + [c_int] * 9 + \
            [c_void_p] * 6 + [c_void_p]
        L.sage_varlen_smooth_q_sizes.argtypes = [c_int] * 6 + [c_size_p] * 2
        L.sage_qk_delta_varlen.argtypes = [c_void_p, c_int, c_void_p, c_void_p] + [c_int] * 10 + [c_void_p] * 6
        L.sage_quant_v_varlen.argtypes = [c_void_p, c_int, c_void_p] + [c_int] * 5 + [c_void_p] * 4
        L.sage_attn_fwd_varlen.argtypes = [c_void_p] * 10 + [c_int, c_void_p, c_void_p] + [c_int] * 8 + \
            [c_int, c_float, c_int, c_int, c_void_p]
        L.sage_attn_fwd_q16.argtypes = [c_void_p] * 7 + [c_int] * 8 + [c_float, c_int, c_void_p]
        L.sage_attn_fwd_varlen_q16.argtypes = [c_void_p] * 7 + [c_int, c_void_p, c_void_p] + [c_int] * 9 + \
            [c_float, c_int, c_void_p]
        L.sage_quant_v_fp4.argtypes = [c_void_p] + [c_int] * 6 + [c_void_p] * 4
        L.sage_v_fp4_buffer_sizes.argtypes = [c_int] * 4 + [c_size_p] * 2
        L.sage_quant_v_fp4_varlen.argtypes = [c_void_p, c_int, c_void_p] + [c_int] * 5 + [c_void_p] * 4
        L.sage_varlen_v_fp4_buffer_sizes.argtypes = [c_int] * 4 + [c_size_p] * 2
        L.sage_status_str.argtypes = [c_int]
        L.sage_status_str.restype = ctypes.c_char_p
        L.sage_check_arch.argtypes = [ctypes.c_char_p]
        for n in EXPORTED:
            if n != "sage_status_str":
                getattr(L, n).restype = c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().sage_status_str(status).decode()


def _check(status: int, what: str):
    if status == SAGE_ERR_UNSUPPORTED:
        raise ValueError(f"{what}: {status_str(status)}")
    if status != SAGE_OK:
        raise SageError(status, what)


# ----------------------------------------------------------------- raw entry points
def sage_get_config():
    """(blk_q, blk_k, tile_k_fp8, tile_k_fp16)"""
    v = [ctypes.c_int() for _ in range(4)]
    _check(lib().sage_get_config(*[ctypes.byref(x) for x in v]), "sage_get_config")
    return tuple(x.value for x in v)


def sage_buffer_sizes(B, H, H_kv, S, D, qk_quant=0):
    vals = [ctypes.c_size_t() for _ in range(9)]
    _check(lib().sage_buffer_sizes(B, H, H_kv, S, D, qk_quant, *[ctypes.byref(v) for v in vals]), "sage_buffer_sizes")
    names = ["q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_fp8", "v_scale", "q_mean", "delta_s"]
    return {n: v.value for n, v in zip(names, vals)}


def sage_smooth_quant_qk(q, k, dtype, B, H, H_kv, S, D, layout, qk_quant, q_i8, q_scale, k_i8, k_scale, k_mean,
                         q_mean, stream):
    """All tensor arguments are device pointers (ints); returns the status code."""
    return lib().sage_smooth_quant_qk(q, k, dtype, B, H, H_kv, S, D, layout, qk_quant, q_i8, q_scale, k_i8, k_scale,
                                      k_mean, q_mean, stream)


def sage_quantize_qkv(q, k, v, dtype, B, H, H_kv, S, D, layout, qk_quant, q_i8, q_scale, k_i8, k_scale, k_mean,
                      q_mean, v_fp8, v_scale, v_mean, stream):
    return lib().sage_quantize_qkv(q, k, v, dtype, B, H, H_kv, S, D, layout, qk_quant, q_i8, q_scale, k_i8, k_scale,
                                   k_mean, q_mean, v_fp8, v_scale, v_mean, stream)


def sage_qk_delta(k, dtype, B, H, H_kv, S, D, layout, qk_quant, is_causal, q_mean, k_mean, q_scale, k_scale, delta_s,
                  stream):
    return lib().sage_qk_delta(k, dtype, B, H, H_kv, S, D, layout, qk_quant, is_causal, q_mean, k_mean, q_scale,
                               k_scale, delta_s, stream)


def sage_quant_v(v, dtype, B, H, S, D, layout, v_fp8, v_scale, v_mean, stream):
    return lib().sage_quant_v(v, dtype, B, H, S, D, layout, v_fp8, v_scale, v_mean, stream)


def sage_quant_v_fp4(v, dtype, B, H, S, D, layout, v_codes, v_e8m0, v_mean, stream):
    return lib().sage_quant_v_fp4(v, dtype, B, H, S, D, layout, v_codes, v_e8m0, v_mean, stream)


def _sizes2(fn, *args):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(fn(*args, ctypes.byref(a), ctypes.byref(b)), fn.__name__)
    return {"v_codes": a.value, "v_e8m0": b.value}


def sage_v_fp4_buffer_sizes(B, H_kv, S, D):
    return _sizes2(lib().sage_v_fp4_buffer_sizes, B, H_kv, S, D)


def sage_varlen_v_fp4_buffer_sizes(B, H_kv, total_k, D):
    return _sizes2(lib().sage_varlen_v_fp4_buffer_sizes, B, H_kv, total_k, D)


def sage_quant_v_fp4_varlen(v, dtype, cu_seqlens_k, B, H_kv, total_k, max_seqlen_k, D, v_codes, v_e8m0, v_mean,
                            stream):
    return lib().sage_quant_v_fp4_varlen(v, dtype, cu_seqlens_k, B, H_kv, total_k, max_seqlen_k, D, v_codes, v_e8m0,
                                         v_mean, stream)


def sage_attn_fwd(q_i8, q_scale, k_i8, k_scale, v, v_scale, v_mean, q_mean, delta_s, out, dtype, B, H, H_kv, S, D,
                  layout, is_causal, sm_scale, pv_mode, qk_quant, stream):
    return lib().sage_attn_fwd(q_i8, q_scale, k_i8, k_scale, v, v_scale, v_mean, q_mean, delta_s, out, dtype, B, H,
                               H_kv, S, D, layout, is_causal, sm_scale, pv_mode, qk_quant, stream)


def sage_attn_fwd_q16(q, k_i8, k_scale, v, v_scale, v_mean, out, dtype, B, H, H_kv, S, D, layout, is_causal, sm_scale,
                      pv_mode, stream):
    return lib().sage_attn_fwd_q16(q, k_i8, k_scale, v, v_scale, v_mean, out, dtype, B, H, H_kv, S, D, layout,
                                   is_causal, sm_scale, pv_mode, stream)


def sage_attn_fwd_varlen_q16(q, k_i8, k_scale, v, v_scale, v_mean, out, dtype, cu_seqlens_q, cu_seqlens_k, B, H, H_kv,
                             total_q, total_k, max_seqlen_q, max_seqlen_k, D, is_causal, sm_scale, pv_mode, stream):
    return lib().sage_attn_fwd_varlen_q16(q, k_i8, k_scale, v, v_scale, v_mean, out, dtype, cu_seqlens_q, cu_seqlens_k,
                                          B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D, is_causal,
                                          sm_scale, pv_mode, stream)


def sage_attn_fwd_dump_qk(q_i8, q_scale, k_i8, k_scale, v, v_scale, v_mean, out, dtype, B, H, H_kv, S, D, layout,
                          is_causal, sm_scale, pv_mode, qk_quant, b, h, qk, stream):
    return lib().sage_attn_fwd_dump_qk(q_i8, q_scale, k_i8, k_scale, v, v_scale, v_mean, out, dtype, B, H, H_kv, S,
                                       D, layout, is_causal, sm_scale, pv_mode, qk_quant, b, h, qk, stream)


def sage_varlen_buffer_sizes(B, H, H_kv, total_q, total_k, D, qk_quant=0):
    vals = [ctypes.c_size_t() for _ in range(7)]
    _check(lib().sage_varlen_buffer_sizes(B, H, H_kv, total_q, total_k, D, qk_quant,
                                          *[ctypes.byref(v) for v in vals]), "sage_varlen_buffer_sizes")
    names = ["q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_fp8", "v_scale"]
    return {n: v.value for n, v in zip(names, vals)}


def sage_varlen_smooth_q_sizes(B, H, total_q, total_k, max_seqlen_q, D):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().sage_varlen_smooth_q_sizes(B, H, total_q, total_k, max_seqlen_q, D, ctypes.byref(a),
                                            ctypes.byref(b)), "sage_varlen_smooth_q_sizes")
    return {"q_mean": a.value, "delta_s": b.value}


def sage_smooth_quant_qk_varlen(q, k, dtype, cu_seqlens_q, cu_seqlens_k, B, H, H_kv, total_q, total_k, max_seqlen_q,
                                max_seqlen_k, D, qk_quant, q_i8, q_scale, k_i8, k_scale, k_mean, q_mean, stream):
    return lib().sage_smooth_quant_qk_varlen(q, k, dtype, cu_seqlens_q, cu_seqlens_k, B, H, H_kv, total_q, total_k,
                                             max_seqlen_q, max_seqlen_k, D, qk_quant, q_i8, q_scale, k_i8, k_scale,
                                             k_mean, q_mean, stream)


def sage_qk_delta_varlen(k, dtype, cu_seqlens_q, cu_seqlens_k, B, H, H_kv, total_q, total_k, max_seqlen_q,
                         max_seqlen_k, D, qk_quant, is_causal, q_mean, k_mean, q_scale, k_scale, delta_s, stream):
    return lib().sage_qk_delta_varlen(k, dtype, cu_seqlens_q, cu_seqlens_k, B, H, H_kv, total_q, total_k, max_seqlen_q,
                                      max_seqlen_k, D, qk_quant, is_causal, q_mean, k_mean, q_scale, k_scale, delta_s,
                                      stream)


def sage_quant_v_varlen(v, dtype, cu_seqlens_k, B, H_kv, total_k, max_seqlen_k, D, v_fp8, v_scale, v_mean, stream):
    return lib().sage_quant_v_varlen(v, dtype, cu_seqlens_k, B, H_kv, total_k, max_seqlen_k, D, v_fp8, v_scale,
                                     v_mean, stream)


def sage_attn_fwd_varlen(q_i8, q_scale, k_i8, k_scale, v, v_scale, v_mean, q_mean, delta_s, out, dtype, cu_seqlens_q,
                         cu_seqlens_k, B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D, is_causal, sm_scale,
                         pv_mode, qk_quant, stream):
    return lib().sage_attn_fwd_varlen(q_i8, q_scale, k_i8, k_scale, v, v_scale, v_mean, q_mean, delta_s, out, dtype,
                                      cu_seqlens_q,
                                      cu_seqlens_k, B, H, H_kv, total_q, total_k, max_seqlen_q, max_seqlen_k, D,
                                      is_causal, sm_scale, pv_mode, qk_quant, stream)


def sage_status_str(status):
    return status_str(status)


def sage_check_arch(name: str) -> int:
    return lib().sage_check_arch(None if name is None else name.encode())


# ----------------------------------------------------------------- torch helpers
def default_sm_scale(D: int) -> float:
    """1/sqrt(D), rounded once to fp32."""
    import numpy as np

    return float(np.float32(1.0 / math.sqrt(D)))


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape(t, layout):
    if t.dim() != 4:
        raise ValueError("expected a 4-d tensor")
    if layout == "HND":
        B, H, S, D = t.shape
    elif layout == "NHD":
        B, S, H, D = t.shape
    else:
        raise ValueError(f"tensor_layout must be HND or NHD, got {layout!r}")
    return B, H, S, D


def _dtype_code(t):
    import torch

    if t.dtype == torch.float16:
        return DTYPE["fp16"]
    if t.dtype == torch.bfloat16:
        return DTYPE["bf16"]
    raise ValueError(f"q/k/v must be float16 or bfloat16, got {t.dtype}")


class Quantized:
    """Device buffers produced by the two quantisation entry points (K and V
    buffers have H_kv heads; H_kv = H unless K/V are grouped).  q_i8 / k_i8 hold
    the Q / K codes: INT8, or (qk_quant "mxfp4") packed E2M1 pairs, with
    q_scale / k_scale then the E8M0 bytes of each 32-channel block."""

    def __init__(self, B, H, S, D, device, H_kv=None, qk_quant="int8"):
        import torch

        H_kv = H if H_kv is None else H_kv
        self.B, self.H, self.H_kv, self.S, self.D, self.qk = B, H, H_kv, S, D, QK[qk_quant]
        sq, sk = (S + BLK_Q - 1) // BLK_Q * BLK_Q, (S + KV_PAD - 1) // KV_PAD * KV_PAD
        lane, token = self.qk == QK["int8_lane"], self.qk == QK["int8_token"]
        if self.qk == QK["mxfp4"]:  # packed E2M1 pairs and E8M0 bytes per 32 channels of a row
            self.q_i8 = torch.empty((B, H, sq, D // 2), dtype=torch.uint8, device=device)
            self.q_scale = torch.empty((B, H, sq, D // 32), dtype=torch.uint8, device=device)
            self.k_i8 = torch.empty((B, H_kv, sk, D // 2), dtype=torch.uint8, device=device)
            self.k_scale = torch.empty((B, H_kv, sk, D // 32), dtype=torch.uint8, device=device)
        else:
            self.q_i8 = torch.empty((B, H, sq, D), dtype=torch.int8, device=device)
            self.q_scale = torch.empty((B, H, sq if lane or token else sq // BLK_Q), dtype=torch.float32,
                                       device=device)
            self.k_i8 = torch.empty((B, H_kv, sk, D), dtype=torch.int8, device=device)
            self.k_scale = torch.empty((B, H_kv, sk if token else sk // 16 if lane else sk // BLK_K),
                                       dtype=torch.float32, device=device)
        self.k_mean = torch.empty((B, H_kv, D), dtype=torch.float32, device=device)
        self.v_fp8 = torch.empty((B, H_kv, sk // BLK_K, D, BLK_K), dtype=torch.uint8, device=device)
        self.v_scale = torch.empty((B, H_kv, D), dtype=torch.float32, device=device)
        self.v_mean = torch.empty((B, H_kv, D), dtype=torch.float32, device=device)
        # pv fp4 V: packed E2M1 codes [B][H_kv][S_k / 64][D][32] and E8M0 bytes
        # [B][H_kv][S_k / 64][D][2] (allocated on first use)
        self.v_fp4 = self.v_e8m0 = None
        self._v4_shape = (B, H_kv, sk // BLK_K, D)
        self.smooth_v = False  # set by quantize: whether the V codes hold V minus v_mean
        self.smooth_q = False  # set by quantize: whether q_i8 holds Q minus its block means
        self.delta_causal = False  # set by quantize: delta_s holds only what a causal attention reads
        self.q_in_attn = False  # set by quantize: Q left unquantised, for the attention to quantise
        self.v_mode = None  # set by quantize: the pv mode whose V codes hold this V ("fp8", "fp4"; None)
        self.q_mean = self.delta_s = None  # smoothed Q: allocated on first use
        self._device = device

    def alloc_v_fp4(self):
        import torch

        if self.v_fp4 is None:
            self.v_fp4 = torch.empty(self._v4_shape + (32,), dtype=torch.uint8, device=self._device)
            self.v_e8m0 = torch.empty(self._v4_shape + (2,), dtype=torch.uint8, device=self._device)


def _kv_heads(q, k, v, tensor_layout):
    """Number of K/V heads; checks that k, v match q apart from the head count."""
    B, H, S, D = _shape(q, tensor_layout)
    kb, H_kv, ks, kd = _shape(k, tensor_layout)
    if (kb, ks, kd) != (B, S, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must match q in batch, sequence length, head dim and dtype, and each other")
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"the number of query heads ({H}) must be a multiple of the K/V heads ({H_kv})")
    return H_kv


def quantize(q, k, v, tensor_layout="HND", pv_mode="fp8", bufs: Quantized | None = None,
             qk_quant="int8", smooth_v=False, smooth_q=False, fused=True, is_causal=False,
             q_in_attn=False) -> Quantized:
    """Run sage_quantize_qkv in pv fp8 mode (fused=False: sage_smooth_quant_qk and
    sage_quant_v, same results), sage_smooth_quant_qk and sage_quant_v_fp4 in pv
    fp4 mode, or sage_smooth_quant_qk alone in pv fp16 mode, on torch tensors.
    k and v may have fewer heads than q (grouped-query attention); qk_quant "int8"
    (per block), "int8_lane" (one scale per Q token and per 16-key lane group of
    K), "int8_token" (one per Q token and per K token), "int8_head" (one per
    head of Q and of K; not with smooth_q) or "mxfp4"; smooth_v
    (pv fp8, fp4): quantise V minus its channel mean; smooth_q: quantise Q minus its
    32-token block means and form the pre-processing term (is_causal: only the part
    a causal attention reads; the buffers then serve causal attention only);
    q_in_attn (INT8 per block, unsmoothed Q): leave Q to the attention kernel
    (sage_attn_fwd_q16: attn_fwd then needs q), same results."""
    if pv_mode not in PV:
        raise ValueError(f"pv_mode must be one of {sorted(PV)}, got {pv_mode!r}")
    if smooth_v and pv_mode == "fp16":
        raise ValueError("smooth_v applies to the quantised V of pv_mode 'fp8' and 'fp4'")
    if q_in_attn and (qk_quant != "int8" or smooth_q):
        raise ValueError("q_in_attn: the attention kernel quantises Q with INT8 per-block scales, unsmoothed")
    layout = LAYOUT[tensor_layout]
    B, H, S, D = _shape(q, tensor_layout)
    H_kv = _kv_heads(q, k, v, tensor_layout)
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    dt = _dtype_code(q)
    bufs = bufs or Quantized(B, H, S, D, q.device, H_kv, qk_quant)
    if (bufs.B, bufs.H, bufs.H_kv, bufs.S, bufs.D, bufs.qk) != (B, H, H_kv, S, D, QK[qk_quant]):
        raise ValueError("bufs were allocated for another shape or granularity")
    st = _stream()
    if smooth_q and bufs.q_mean is None:
        import torch

        nq, sk = bufs.q_i8.shape[2] // BLK_Q, bufs.k_i8.shape[2]
        bufs.q_mean = torch.empty((B, H, nq, D), dtype=torch.float32, device=q.device)
        bufs.delta_s = torch.empty((B, H, sk // KV_PAD, nq, KV_PAD), dtype=torch.float32, device=q.device)
    bufs.smooth_q = bool(smooth_q)
    bufs.delta_causal = bool(smooth_q and is_causal)
    bufs.q_in_attn = bool(q_in_attn)
    bufs.smooth_v = bool(smooth_v)
    bufs.v_mode = pv_mode if pv_mode != "fp16" else None
    qm = bufs.q_mean.data_ptr() if smooth_q else None
    vm = bufs.v_mean.data_ptr() if smooth_v else None
    # Q omitted (all three NULL) when the attention kernel quantises it
    qp, q8, qs = (None, None, None) if q_in_attn else (q.data_ptr(), bufs.q_i8.data_ptr(), bufs.q_scale.data_ptr())
    if pv_mode == "fp8" and fused:
        _check(sage_quantize_qkv(qp, k.data_ptr(), v.data_ptr(), dt, B, H, H_kv, S, D, layout, bufs.qk, q8, qs,
                                 bufs.k_i8.data_ptr(), bufs.k_scale.data_ptr(), bufs.k_mean.data_ptr(), qm,
                                 bufs.v_fp8.data_ptr(), bufs.v_scale.data_ptr(), vm, st), "sage_quantize_qkv")
    else:
        _check(sage_smooth_quant_qk(qp, k.data_ptr(), dt, B, H, H_kv, S, D, layout, bufs.qk, q8, qs,
                                    bufs.k_i8.data_ptr(), bufs.k_scale.data_ptr(), bufs.k_mean.data_ptr(), qm, st),
               "sage_smooth_quant_qk")
        if pv_mode == "fp8":
            _check(sage_quant_v(v.data_ptr(), dt, B, H_kv, S, D, layout, bufs.v_fp8.data_ptr(),
                                bufs.v_scale.data_ptr(), vm, st), "sage_quant_v")
        elif pv_mode == "fp4":
            bufs.alloc_v_fp4()
            _check(sage_quant_v_fp4(v.data_ptr(), dt, B, H_kv, S, D, layout, bufs.v_fp4.data_ptr(),
                                    bufs.v_e8m0.data_ptr(), vm, st), "sage_quant_v_fp4")
    if smooth_q:
        _check(sage_qk_delta(k.data_ptr(), dt, B, H, H_kv, S, D, layout, bufs.qk, int(bufs.delta_causal),
                             bufs.q_mean.data_ptr(), bufs.k_mean.data_ptr(), bufs.q_scale.data_ptr(),
                             bufs.k_scale.data_ptr(), bufs.delta_s.data_ptr(), st), "sage_qk_delta")
    return bufs


def attn_fwd(bufs: Quantized, v, out, tensor_layout="HND", is_causal=False, sm_scale=None, pv_mode="fp8",
             dump_head=None, dump=None, q=None):
    """Run sage_attn_fwd (or the dump variant when dump_head=(b, h)) into `out`;
    with buffers quantised with q_in_attn, sage_attn_fwd_q16 on q (the input Q)."""
    layout = LAYOUT[tensor_layout]
    B, H, S, D = _shape(out, tensor_layout)
    if (bufs.B, bufs.H, bufs.S, bufs.D) != (B, H, S, D):
        raise ValueError("out does not match the quantised buffers' shape")
    H_kv = bufs.H_kv
    if pv_mode == "fp16" and (_shape(v, tensor_layout) != (B, H_kv, S, D) or not v.is_contiguous()):
        raise ValueError("pv fp16 reads the original V: it must be contiguous with H_kv heads")
    dt = _dtype_code(out)
    sm = default_sm_scale(D) if sm_scale is None else float(sm_scale)
    if bufs.delta_causal and not is_causal:
        raise ValueError("these buffers hold the pre-processing term of a causal attention only")
    vptr, vs, vm = _v_operands(bufs, v, pv_mode)
    pv = PV[pv_mode]
    ds = bufs.delta_s.data_ptr() if bufs.smooth_q else None
    qm = bufs.q_mean.data_ptr() if bufs.smooth_q else None
    head = (bufs.q_i8.data_ptr(), bufs.q_scale.data_ptr(), bufs.k_i8.data_ptr(), bufs.k_scale.data_ptr(), vptr, vs, vm)
    tail = (out.data_ptr(), dt, B, H, H_kv, S, D, layout, int(bool(is_causal)), sm, pv, bufs.qk)
    if bufs.q_in_attn:
        if q is None or tuple(q.shape) != tuple(out.shape) or q.dtype != out.dtype or not q.is_contiguous():
            raise ValueError("these buffers hold no Q codes: pass q, the input Q (same shape, dtype and layout as out)")
        if dump_head is not None:
            raise ValueError("the Q K^T dump reads Q codes: quantise without q_in_attn")
        _check(sage_attn_fwd_q16(q.data_ptr(), bufs.k_i8.data_ptr(), bufs.k_scale.data_ptr(), vptr, vs, vm,
                                 out.data_ptr(), dt, B, H, H_kv, S, D, layout, int(bool(is_causal)), sm, pv,
                                 _stream()), "sage_attn_fwd_q16")
        return out
    if dump_head is None:
        _check(sage_attn_fwd(*head, qm, ds, *tail, _stream()), "sage_attn_fwd")
    else:
        if bufs.smooth_q:
            raise ValueError("the Q K^T dump is not available with smooth_q")
        _check(sage_attn_fwd_dump_qk(*head, *tail, dump_head[0], dump_head[1], dump.data_ptr(), _stream()),
               "sage_attn_fwd_dump_qk")
    return out


def _v_operands(bufs, v, pv_mode):
    """(v, v_scale, v_mean) pointers of the attention call for pv_mode: the
    quantised V codes and scales (pv fp8, fp4) or the caller's V (pv fp16)."""
    if pv_mode not in PV:
        raise ValueError(f"pv_mode must be one of {sorted(PV)}, got {pv_mode!r}")
    if pv_mode == "fp16":
        return v.data_ptr(), None, None
    if bufs.v_mode != pv_mode:
        raise ValueError(f"pv {pv_mode} reads the {pv_mode.upper()} V codes: quantize these buffers with "
                         f"pv_mode={pv_mode!r} first")
    vm = bufs.v_mean.data_ptr() if bufs.smooth_v else None
    if pv_mode == "fp8":
        return bufs.v_fp8.data_ptr(), bufs.v_scale.data_ptr(), vm
    return bufs.v_fp4.data_ptr(), bufs.v_e8m0.data_ptr(), vm


# pv_accum_dtype names of the P V accumulation -> pv mode.  "fp32+fp32" is the
# FP8 P V product whose two accumulation levels (the MFMA's internal sum of a
# tile's products, then the fp32 output registers) are both fp32-class; "fp32"
# is the fp16 P V product with fp32 accumulation.  "fp32+fp16" (an fp16 inner
# accumulator) is not built and is rejected rather than silently replaced.
PV_ACCUM = {"fp32+fp32": "fp8", "fp32": "fp16"}


def sageattn(q, k, v, tensor_layout="HND", is_causal=False, sm_scale=None, pv_mode="fp8", qk_quant="int8",
             smooth_v=False, smooth_q=False, pv_accum_dtype=None):
    """Quantized attention: same shape, dtype and layout out as q.  pv_accum_dtype,
    when given, selects pv_mode by its accumulation name (PV_ACCUM)."""
    import torch

    if pv_accum_dtype is not None:
        if pv_accum_dtype not in PV_ACCUM:
            raise ValueError(f"pv_accum_dtype must be one of {sorted(PV_ACCUM)} (an fp16 inner accumulator, "
                             f"'fp32+fp16', is not built), got {pv_accum_dtype!r}")
        pv_mode = PV_ACCUM[pv_accum_dtype]
    # INT8 per-block scales without Q smoothing: Q is quantised in the attention kernel
    q_in_attn = qk_quant == "int8" and not smooth_q
    bufs = quantize(q, k, v, tensor_layout, pv_mode, qk_quant=qk_quant, smooth_v=smooth_v, smooth_q=smooth_q,
                    is_causal=is_causal, q_in_attn=q_in_attn)
    out = torch.empty_like(q)
    return attn_fwd(bufs, v, out, tensor_layout, is_causal, sm_scale, pv_mode, q=q)


# ----------------------------------------------------------------- packed variable-length batches
def varlen_rows(total: int, B: int, pad: int) -> int:
    """Rows per head of a packed batch's quantised buffer (include/sage.h)."""
    return pad * (total // pad + B + 1)


def varlen_row0(start: int, b: int, pad: int) -> int:
    """First buffer row of sequence b, whose first token is `start`."""
    return pad * (start // pad + b)


class QuantizedVarlen:
    """Device buffers of the packed-batch quantisation entry points."""

    def __init__(self, B, H, H_kv, total_q, total_k, D, device, qk_quant="int8"):
        import torch

        self.B, self.H, self.H_kv, self.total_q, self.total_k, self.D = B, H, H_kv, total_q, total_k, D
        self.qk = QK[qk_quant]
        lane, token = self.qk == QK["int8_lane"], self.qk == QK["int8_token"]
        rq, rk = varlen_rows(total_q, B, BLK_Q), varlen_rows(total_k, B, KV_PAD)
        self.rows_q, self.rows_k = rq, rk
        if self.qk == QK["mxfp4"]:
            self.q_i8 = torch.empty((H, rq, D // 2), dtype=torch.uint8, device=device)
            self.q_scale = torch.empty((H, rq, D // 32), dtype=torch.uint8, device=device)
            self.k_i8 = torch.empty((H_kv, rk, D // 2), dtype=torch.uint8, device=device)
            self.k_scale = torch.empty((H_kv, rk, D // 32), dtype=torch.uint8, device=device)
        else:
            self.q_i8 = torch.empty((H, rq, D), dtype=torch.int8, device=device)
            self.q_scale = torch.empty((H, rq if lane or token else rq // BLK_Q), dtype=torch.float32,
                                       device=device)
            self.k_i8 = torch.empty((H_kv, rk, D), dtype=torch.int8, device=device)
            self.k_scale = torch.empty((H_kv, rk if token else rk // 16 if lane else rk // BLK_K),
                                       dtype=torch.float32, device=device)
        self.k_mean = torch.empty((B, H_kv, D), dtype=torch.float32, device=device)
        self.v_fp8 = torch.empty((H_kv, rk // BLK_K, D, BLK_K), dtype=torch.uint8, device=device)
        self.v_scale = torch.empty((B, H_kv, D), dtype=torch.float32, device=device)
        self.v_mean = torch.empty((B, H_kv, D), dtype=torch.float32, device=device)
        self.v_fp4 = self.v_e8m0 = None  # pv fp4: [H_kv][RK / 64][D][32] and [..][2], on first use
        self._v4_shape = (H_kv, rk // BLK_K, D)
        self._device = device
        self.smooth_v = False
        self.smooth_q = False  # set by quantize_varlen: whether q_i8 holds Q minus its block means
        self.delta_causal = False  # set by quantize_varlen: delta_s holds only what a causal attention reads
        self.q_in_attn = False  # set by quantize_varlen: Q left to the attention kernel
        # smoothed Q: q_mean [H][RQ / 32][D] and delta_s [H][RK / 128][MQ][128],
        # MQ = ceil(max_seqlen_q / 32) (allocated by quantize_varlen on first use)
        self.q_mean = self.delta_s = None
        self.v_mode = None

    alloc_v_fp4 = Quantized.alloc_v_fp4

    def alloc_smooth_q(self, max_seqlen_q):
        import torch

        mq = (max_seqlen_q + BLK_Q - 1) // BLK_Q
        if self.q_mean is None:
            self.q_mean = torch.empty((self.H, self.rows_q // BLK_Q, self.D), dtype=torch.float32,
                                      device=self._device)
        if self.delta_s is None or self.delta_s.shape[2] != mq:
            self.delta_s = torch.empty((self.H, self.rows_k // KV_PAD, mq, KV_PAD), dtype=torch.float32,
                                       device=self._device)


def _cu(t, name):
    import torch

    if not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 device tensor")
    return t


def quantize_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, pv_mode="fp8",
                    bufs: QuantizedVarlen | None = None, qk_quant="int8", smooth_v=False,
                    smooth_q=False, is_causal=False, q_in_attn=False) -> QuantizedVarlen:
    """sage_smooth_quant_qk_varlen (and sage_quant_v_varlen in pv fp8 mode,
    sage_quant_v_fp4_varlen in pv fp4 mode, sage_qk_delta_varlen with smooth_q)
    on a packed batch: q [total_q, H, D], k / v [total_k, H_kv, D], cu_seqlens
    int32 [B + 1]; smooth_v, smooth_q, is_causal, q_in_attn as in quantize."""
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total_q, H, D] and k, v [total_k, H_kv, D]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must have the same dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    cq, ck = _cu(cu_seqlens_q, "cu_seqlens_q"), _cu(cu_seqlens_k, "cu_seqlens_k")
    if cq.numel() != ck.numel() or cq.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 >= 2 entries")
    B = cq.numel() - 1
    (total_q, H, D), (total_k, H_kv, _) = q.shape, k.shape
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"the number of query heads ({H}) must be a multiple of the K/V heads ({H_kv})")
    if pv_mode not in PV:
        raise ValueError(f"pv_mode must be one of {sorted(PV)}, got {pv_mode!r}")
    if smooth_v and pv_mode == "fp16":
        raise ValueError("smooth_v applies to the quantised V of pv_mode 'fp8' and 'fp4'")
    if q_in_attn and (qk_quant != "int8" or smooth_q):
        raise ValueError("q_in_attn: the attention kernel quantises Q with INT8 per-block scales, unsmoothed")
    dt = _dtype_code(q)
    bufs = bufs or QuantizedVarlen(B, H, H_kv, total_q, total_k, D, q.device, qk_quant)
    if (bufs.B, bufs.H, bufs.H_kv, bufs.total_q, bufs.total_k, bufs.D, bufs.qk) != \
            (B, H, H_kv, total_q, total_k, D, QK[qk_quant]):
        raise ValueError("bufs were allocated for another shape or granularity")
    bufs.max_seqlen_q, bufs.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    if smooth_q:
        bufs.alloc_smooth_q(bufs.max_seqlen_q)
    bufs.smooth_q = bool(smooth_q)
    bufs.delta_causal = bool(smooth_q and is_causal)
    bufs.q_in_attn = bool(q_in_attn)
    qm = bufs.q_mean.data_ptr() if smooth_q else None
    qp, q8, qs = (None, None, None) if q_in_attn else (q.data_ptr(), bufs.q_i8.data_ptr(), bufs.q_scale.data_ptr())
    st = _stream()
    _check(sage_smooth_quant_qk_varlen(qp, k.data_ptr(), dt, cq.data_ptr(), ck.data_ptr(), B, H, H_kv, total_q,
                                       total_k, bufs.max_seqlen_q, bufs.max_seqlen_k, D, bufs.qk, q8, qs,
                                       bufs.k_i8.data_ptr(), bufs.k_scale.data_ptr(), bufs.k_mean.data_ptr(), qm, st),
           "sage_smooth_quant_qk_varlen")
    bufs.smooth_v = bool(smooth_v)
    bufs.v_mode = pv_mode if pv_mode != "fp16" else None
    vm = bufs.v_mean.data_ptr() if smooth_v else None
    if pv_mode == "fp8":
        _check(sage_quant_v_varlen(v.data_ptr(), dt, ck.data_ptr(), B, H_kv, total_k, bufs.max_seqlen_k, D,
                                   bufs.v_fp8.data_ptr(), bufs.v_scale.data_ptr(), vm, st), "sage_quant_v_varlen")
    elif pv_mode == "fp4":
        bufs.alloc_v_fp4()
        _check(sage_quant_v_fp4_varlen(v.data_ptr(), dt, ck.data_ptr(), B, H_kv, total_k, bufs.max_seqlen_k, D,
                                       bufs.v_fp4.data_ptr(), bufs.v_e8m0.data_ptr(), vm, st),
               "sage_quant_v_fp4_varlen")
    if smooth_q:
        _check(sage_qk_delta_varlen(k.data_ptr(), dt, cq.data_ptr(), ck.data_ptr(), B, H, H_kv, total_q, total_k,
                                    bufs.max_seqlen_q, bufs.max_seqlen_k, D, bufs.qk, int(bufs.delta_causal),
                                    bufs.q_mean.data_ptr(), bufs.k_mean.data_ptr(), bufs.q_scale.data_ptr(),
                                    bufs.k_scale.data_ptr(), bufs.delta_s.data_ptr(), st), "sage_qk_delta_varlen")
    return bufs


def attn_fwd_varlen(bufs: QuantizedVarlen, v, out, cu_seqlens_q, cu_seqlens_k, is_causal=False, sm_scale=None,
                    pv_mode="fp8", q=None):
    """sage_attn_fwd_varlen into out [total_q, H, D] (sage_attn_fwd_varlen_q16 on q
    with buffers quantised with q_in_attn)."""
    B, H, H_kv, D = bufs.B, bufs.H, bufs.H_kv, bufs.D
    if tuple(out.shape) != (bufs.total_q, H, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [total_q, H, D] tensor")
    if pv_mode == "fp16" and (tuple(v.shape) != (bufs.total_k, H_kv, D) or not v.is_contiguous()):
        raise ValueError("pv fp16 reads the original V: it must be a contiguous [total_k, H_kv, D] tensor")
    cq, ck = _cu(cu_seqlens_q, "cu_seqlens_q"), _cu(cu_seqlens_k, "cu_seqlens_k")
    if bufs.delta_causal and not is_causal:
        raise ValueError("these buffers hold the pre-processing term of a causal attention only")
    vptr, vs, vm = _v_operands(bufs, v, pv_mode)
    pv = PV[pv_mode]
    sm = default_sm_scale(D) if sm_scale is None else float(sm_scale)
    if bufs.q_in_attn:
        if q is None or tuple(q.shape) != tuple(out.shape) or q.dtype != out.dtype or not q.is_contiguous():
            raise ValueError("these buffers hold no Q codes: pass q, the input Q (same shape and dtype as out)")
        _check(sage_attn_fwd_varlen_q16(q.data_ptr(), bufs.k_i8.data_ptr(), bufs.k_scale.data_ptr(), vptr, vs, vm,
                                        out.data_ptr(), _dtype_code(out), cq.data_ptr(), ck.data_ptr(), B, H, H_kv,
                                        bufs.total_q, bufs.total_k, bufs.max_seqlen_q, bufs.max_seqlen_k, D,
                                        int(bool(is_causal)), sm, pv, _stream()), "sage_attn_fwd_varlen_q16")
        return out
    qm = bufs.q_mean.data_ptr() if bufs.smooth_q else None
    ds = bufs.delta_s.data_ptr() if bufs.smooth_q else None
    _check(sage_attn_fwd_varlen(bufs.q_i8.data_ptr(), bufs.q_scale.data_ptr(), bufs.k_i8.data_ptr(),
                                bufs.k_scale.data_ptr(), vptr, vs, vm, qm, ds, out.data_ptr(), _dtype_code(out),
                                cq.data_ptr(), ck.data_ptr(), B, H, H_kv, bufs.total_q, bufs.total_k,
                                bufs.max_seqlen_q, bufs.max_seqlen_k, D, int(bool(is_causal)), sm, pv, bufs.qk,
                                _stream()),
           "sage_attn_fwd_varlen")
    return out


def sageattn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, is_causal=False, sm_scale=None,
                    pv_mode="fp8", qk_quant="int8", smooth_v=False, smooth_q=False):
    """Quantized attention over a packed batch of sequences ("SageAttention: Thư viện
    Attention lượng tử hóa" page, feature list: sageattn_varlen):
    q [total_q, H, D], k / v [total_k, H_kv, D]; returns [total_q, H, D]."""
    import torch

    q_in_attn = qk_quant == "int8" and not smooth_q  # as in sageattn
    bufs = quantize_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, pv_mode, qk_quant=qk_quant,
                           smooth_v=smooth_v, smooth_q=smooth_q, is_causal=is_causal, q_in_attn=q_in_attn)
    out = torch.empty_like(q)
    return attn_fwd_varlen(bufs, v, out, cu_seqlens_q, cu_seqlens_k, is_causal, sm_scale, pv_mode, q=q)
