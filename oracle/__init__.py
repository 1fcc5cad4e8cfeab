"""CPU oracle for SageAttention-style quantized attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.

This module is bookkeeping only: it builds/loads ``liboracle.so`` (the plain C
reference in ``sage_oracle.c``), cuts heads out of HND/NHD tensors and passes
them to the C functions, which do all of the method's arithmetic.

Layouts: ``HND`` = [B, H, S, D], ``NHD`` = [B, S, H, D] ("完整指南" page,
section 五分钟跑通第一个加速样例: tensor_layout).  Inputs are the raw 16-bit
codes (``numpy.uint16``) of fp16 or bf16 tensors, exactly the bytes uploaded to
the GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
PV_FP8, PV_FP16, PV_FP4 = 0, 1, 2
# Method parameters used by default: INT8 scale blocks of 32 Q tokens and 64 K
# tokens, online-softmax tiles of 128 keys.
BLK_Q, BLK_K, TILE_K = 32, 64, 128
DTYPES = {"fp16": F16, "bf16": BF16}
CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]

_lib = None


def build() -> str:
    """Compile liboracle.so from sage_oracle.c (always recompiles)."""
    tmp = _SO + ".tmp"
    cmd = ["gcc"] + CFLAGS + [_SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, _SO)
    return _SO


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def lib():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is None:
        hdr = os.path.join(_HERE, "sage_oracle.h")
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < max(os.path.getmtime(_SRC), os.path.getmtime(hdr)):
            build()
        L = ctypes.CDLL(_SO)
        L.orc_e4m3_decode.restype = ctypes.c_float
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e2m1_decode.restype = ctypes.c_float
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e2m1_encode.argtypes = [ctypes.c_float]
        for name in ("orc_decode16", "orc_encode16", "orc_e4m3_encode_n", "orc_int8_quant_block",
                     "orc_channel_mean", "orc_quant_q_head", "orc_quant_k_head", "orc_quant_k_head_lane",
                     "orc_quant_v_head", "orc_quant_v_head_smooth", "orc_qk_int32_head", "orc_attn_head_rows",
                     "orc_attn_exact_head", "orc_mxfp4_quant_rows", "orc_quant_k_head_mxfp4", "orc_qk_mxfp4_rows",
                     "orc_quant_q_head_smooth", "orc_qk_delta_head", "orc_quant_q_head_mxfp4_smooth",
                     "orc_quant_v_head_mxfp4"):
            getattr(L, name).restype = None
        L.orc_lane_group.restype = ctypes.c_int
        L.orc_lane_group.argtypes = [ctypes.c_int]
        L.orc_pv_group.restype = ctypes.c_int
        L.orc_pv_group.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


class use_library:
    """Context manager: route every call in this module to another build of the
    oracle source (the test suite uses it to run the pins against copies of the
    oracle with a deliberately planted mistake)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = None
        saved_so = globals()["_SO"]
        globals()["_SO"] = self.path
        try:
            lib()
        finally:
            globals()["_SO"] = saved_so
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def build_variant(src: str, out_so: str) -> str:
    """Compile another copy of the oracle source with the same flags."""
    subprocess.run(["gcc"] + CFLAGS + ["-I", _HERE, src, "-o", out_so, "-lm"], check=True)
    return out_so


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- formats
def decode16(codes: np.ndarray, dtype: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint16)
    out = np.empty(c.shape, np.float32)
    lib().orc_decode16(_p(c, ctypes.c_uint16), ctypes.c_size_t(c.size), dtype, _p(out, ctypes.c_float))
    return out


def encode16(x: np.ndarray, dtype: int) -> np.ndarray:
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib().orc_encode16(_p(x, ctypes.c_float), ctypes.c_size_t(x.size), dtype, _p(out, ctypes.c_uint16))
    return out


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib().orc_e4m3_decode(int(v)) for v in c.ravel()], np.float32).reshape(c.shape)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    x = _f32(x)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode_n(_p(x, ctypes.c_float), ctypes.c_size_t(x.size), _p(out, ctypes.c_uint8))
    return out


def int8_quant_block(x: np.ndarray):
    x = _f32(x)
    codes = np.empty(x.shape, np.int8)
    scale = ctypes.c_float()
    lib().orc_int8_quant_block(_p(x, ctypes.c_float), ctypes.c_size_t(x.size), _p(codes, ctypes.c_int8),
                               ctypes.byref(scale))
    return codes, np.float32(scale.value)


def channel_mean(x: np.ndarray) -> np.ndarray:
    x = _f32(x)
    S, D = x.shape
    out = np.empty(D, np.float32)
    lib().orc_channel_mean(_p(x, ctypes.c_float), S, D, _p(out, ctypes.c_float))
    return out


# ---------------------------------------------------------------- per head
def head(x: np.ndarray, layout: str, b: int, h: int) -> np.ndarray:
    """Return head (b, h) of a physical HND/NHD tensor as a contiguous [S, D] array."""
    if layout == "HND":
        return np.ascontiguousarray(x[b, h])
    if layout == "NHD":
        return np.ascontiguousarray(x[b, :, h, :])
    raise ValueError(layout)


def quant_q_head(qf: np.ndarray, blk: int):
    qf = _f32(qf)
    S, D = qf.shape
    codes = np.empty((S, D), np.int8)
    scales = np.empty((S + blk - 1) // blk, np.float32)
    lib().orc_quant_q_head(_p(qf, ctypes.c_float), S, D, blk, _p(codes, ctypes.c_int8), _p(scales, ctypes.c_float))
    return codes, scales


def quant_k_head(kf: np.ndarray, blk: int, smooth: bool = True):
    kf = _f32(kf)
    S, D = kf.shape
    codes = np.empty((S, D), np.int8)
    scales = np.empty((S + blk - 1) // blk, np.float32)
    mean = np.empty(D, np.float32)
    lib().orc_quant_k_head(_p(kf, ctypes.c_float), S, D, blk, int(smooth), _p(codes, ctypes.c_int8),
                           _p(scales, ctypes.c_float), _p(mean, ctypes.c_float))
    return codes, scales, mean


def quant_q_head_smooth(qf: np.ndarray, blk: int, blk_scale: int | None = None):
    """Smoothed Q: (codes, scales, block means [nb, D]) of Q minus each blk-token
    block's channel means; INT8 scale blocks of blk_scale tokens (default blk)."""
    qf = _f32(qf)
    S, D = qf.shape
    bs = blk if blk_scale is None else blk_scale
    codes = np.empty((S, D), np.int8)
    scales = np.empty((S + bs - 1) // bs, np.float32)
    qmean = np.empty(((S + blk - 1) // blk, D), np.float32)
    lib().orc_quant_q_head_smooth(_p(qf, ctypes.c_float), S, D, blk, bs, _p(codes, ctypes.c_int8),
                                  _p(scales, ctypes.c_float), _p(qmean, ctypes.c_float))
    return codes, scales, qmean


def qk_delta_head(qmean: np.ndarray, kf: np.ndarray, kmean: np.ndarray) -> np.ndarray:
    """delta[b][n] = qmean[b] . (K[n] - k_mean) (the subtraction in fp32, the dot
    product in binary64, rounded to fp32)."""
    qmean, kf, kmean = _f32(qmean), _f32(kf), _f32(kmean)
    nb, D = qmean.shape
    S = kf.shape[0]
    out = np.empty((nb, S), np.float32)
    lib().orc_qk_delta_head(_p(qmean, ctypes.c_float), nb, _p(kf, ctypes.c_float), _p(kmean, ctypes.c_float), S, D,
                            _p(out, ctypes.c_float))
    return out


def lane_group(n: int) -> int:
    """K scale group of key n under thread-level granularity (see sage_oracle.c)."""
    return int(lib().orc_lane_group(int(n)))


def quant_k_head_lane(kf: np.ndarray, smooth: bool = True):
    """K codes, one scale per 16-key lane group (2 * ceil(S / 32) scales), K mean."""
    kf = _f32(kf)
    S, D = kf.shape
    codes = np.empty((S, D), np.int8)
    scales = np.empty(2 * ((S + 31) // 32), np.float32)
    mean = np.empty(D, np.float32)
    lib().orc_quant_k_head_lane(_p(kf, ctypes.c_float), S, D, int(smooth), _p(codes, ctypes.c_int8),
                                _p(scales, ctypes.c_float), _p(mean, ctypes.c_float))
    return codes, scales, mean


def e2m1_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    return np.array([lib().orc_e2m1_decode(int(c)) for c in codes.ravel()], np.float32).reshape(codes.shape)


def e2m1_encode(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    return np.array([lib().orc_e2m1_encode(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def quant_mxfp4_rows(xf: np.ndarray):
    """MXFP4 of each row: (E2M1 codes [S, D] one per byte, E8M0 scales [S, D / 32])."""
    xf = _f32(xf)
    S, D = xf.shape
    codes = np.empty((S, D), np.uint8)
    e8m0 = np.empty((S, D // 32), np.uint8)
    lib().orc_mxfp4_quant_rows(_p(xf, ctypes.c_float), S, D, _p(codes, ctypes.c_uint8), _p(e8m0, ctypes.c_uint8))
    return codes, e8m0


def quant_q_head_mxfp4_smooth(qf: np.ndarray, blk: int = BLK_Q):
    """Smoothed Q for the FP4 product: (codes, e8m0, block means [nb, D]) of Q minus
    each blk-token block's channel means."""
    qf = _f32(qf)
    S, D = qf.shape
    codes = np.empty((S, D), np.uint8)
    e8m0 = np.empty((S, D // 32), np.uint8)
    qmean = np.empty(((S + blk - 1) // blk, D), np.float32)
    lib().orc_quant_q_head_mxfp4_smooth(_p(qf, ctypes.c_float), S, D, blk, _p(codes, ctypes.c_uint8),
                                        _p(e8m0, ctypes.c_uint8), _p(qmean, ctypes.c_float))
    return codes, e8m0, qmean


def pv_group(n: int) -> int:
    """Key group of key n in the micro-scaled FP4 P~ V product (see sage_oracle.c)."""
    return int(lib().orc_pv_group(int(n)))


def quant_v_head_mxfp4(vf: np.ndarray, smooth: bool = False):
    """V for the FP4 P~ V product: (E2M1 codes [S, D], E8M0 scales [2 ceil(S/64), D],
    channel means [D] -- zeros unless smooth)."""
    vf = _f32(vf)
    S, D = vf.shape
    codes = np.empty((S, D), np.uint8)
    e8m0 = np.empty((2 * ((S + 63) // 64), D), np.uint8)
    mean = np.empty(D, np.float32)
    lib().orc_quant_v_head_mxfp4(_p(vf, ctypes.c_float), S, D, int(smooth), _p(codes, ctypes.c_uint8),
                                 _p(e8m0, ctypes.c_uint8), _p(mean, ctypes.c_float))
    return codes, e8m0, mean


def quant_k_head_mxfp4(kf: np.ndarray, smooth: bool = True):
    """K for the FP4 product: (codes, e8m0, mean) of K minus its channel mean."""
    kf = _f32(kf)
    S, D = kf.shape
    codes = np.empty((S, D), np.uint8)
    e8m0 = np.empty((S, D // 32), np.uint8)
    mean = np.empty(D, np.float32)
    lib().orc_quant_k_head_mxfp4(_p(kf, ctypes.c_float), S, D, int(smooth), _p(codes, ctypes.c_uint8),
                                 _p(e8m0, ctypes.c_uint8), _p(mean, ctypes.c_float))
    return codes, e8m0, mean


def qk_mxfp4_rows(q4, qe, k4, ke, rows=None) -> np.ndarray:
    """fp32 Q K^T of MXFP4 rows (exact dot products, rounded once): [len(rows), S_k]."""
    q4, qe, k4, ke = (np.ascontiguousarray(a, np.uint8) for a in (q4, qe, k4, ke))
    Sq, D = q4.shape
    S = k4.shape[0]
    rows = np.arange(Sq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    out = np.empty((rows.size, S), np.float32)
    lib().orc_qk_mxfp4_rows(_p(q4, ctypes.c_uint8), _p(qe, ctypes.c_uint8), _p(k4, ctypes.c_uint8),
                            _p(ke, ctypes.c_uint8), S, D, _p(rows, ctypes.c_int), rows.size, _p(out, ctypes.c_float))
    return out


def quant_v_head(vf: np.ndarray, smooth: bool = False):
    """E4M3 codes + per-channel scales of V; with smooth, of V minus its channel
    mean, which is returned as a third value."""
    vf = _f32(vf)
    S, D = vf.shape
    codes = np.empty((S, D), np.uint8)
    scales = np.empty(D, np.float32)
    if smooth:
        mean = np.empty(D, np.float32)
        lib().orc_quant_v_head_smooth(_p(vf, ctypes.c_float), S, D, _p(codes, ctypes.c_uint8),
                                      _p(scales, ctypes.c_float), _p(mean, ctypes.c_float))
        return codes, scales, mean
    lib().orc_quant_v_head(_p(vf, ctypes.c_float), S, D, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_float))
    return codes, scales


def qk_int32_head(q8: np.ndarray, k8: np.ndarray) -> np.ndarray:
    q8 = np.ascontiguousarray(q8, np.int8)
    k8 = np.ascontiguousarray(k8, np.int8)
    S, D = q8.shape
    out = np.empty((S, S), np.int32)
    lib().orc_qk_int32_head(_p(q8, ctypes.c_int8), _p(k8, ctypes.c_int8), S, D, _p(out, ctypes.c_int32))
    return out


def attn_head_rows(q8, q_scale, k8, k_scale, v8, v_scale, vf, *, in_dtype, is_causal, sm_scale,
                   pv_mode, rows=None, blk_q=32, blk_k=64, tile_k=TILE_K, k_lane=False, v_mean=None,
                   qk=None, delta=None, blk_d=BLK_Q, v_e8m0=None) -> np.ndarray:
    """Quantized attention for the given query rows of one head (fp32 [len(rows), D]).

    blk_q / blk_k: tokens per INT8 scale of Q / K (k_lane: K scales per lane group
    instead of blocks, as quant_k_head_lane makes them); tile_k: keys per online-softmax
    tile (the two-level accumulation folds once per tile).  The query rows (q8)
    and the keys (k8, v8, vf) may differ in number.  qk: fp32 Q K^T of the FP4
    product for these rows (qk_mxfp4_rows); then q8 .. k_scale are not used.
    pv fp4: v8 holds V's E2M1 codes and v_e8m0 its scales (quant_v_head_mxfp4)."""
    Sq, D = q8.shape
    S = k8.shape[0]  # keys
    rows = np.arange(Sq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    if rows.size and (rows.min() < 0 or rows.max() >= Sq):
        raise ValueError("query row out of range")
    out = np.empty((rows.size, D), np.float32)
    q8 = np.ascontiguousarray(q8, np.int8)
    k8 = np.ascontiguousarray(k8, np.int8)
    q_scale = _f32(q_scale)
    k_scale = _f32(k_scale)
    v8 = np.ascontiguousarray(v8 if v8 is not None else np.zeros((S, D), np.uint8), np.uint8)
    v_scale = _f32(v_scale if v_scale is not None else np.zeros(D, np.float32))
    vf = _f32(vf if vf is not None else np.zeros((S, D), np.float32))
    vm = None if v_mean is None else _f32(v_mean)
    if vm is not None and pv_mode == PV_FP16:
        raise ValueError("V smoothing applies to the FP8 and FP4 PV products only")
    if pv_mode == PV_FP4 and tile_k % 64:
        raise ValueError("pv fp4 needs tiles of a multiple of 64 keys")
    ve = np.ascontiguousarray(v_e8m0 if v_e8m0 is not None else np.zeros((2 * ((S + 63) // 64), D), np.uint8),
                              np.uint8)
    dl = None
    if delta is not None:  # smoothed Q: [ceil(Sq / blk_q), S] fp32, the pre-processing stage
        dl = _f32(delta)
        if dl.shape != ((Sq + blk_d - 1) // blk_d, S):
            raise ValueError("delta must be [query blocks, S_k]")
    qkr = None
    if qk is not None:
        qkr = np.ascontiguousarray(qk, np.float32)
        if qkr.shape != (rows.size, S):
            raise ValueError("qk must be [len(rows), S_k]")
    lib().orc_attn_head_rows(_p(q8, ctypes.c_int8), _p(q_scale, ctypes.c_float), blk_q,
                             _p(k8, ctypes.c_int8), _p(k_scale, ctypes.c_float), blk_k, int(bool(k_lane)), tile_k,
                             _p(v8, ctypes.c_uint8), _p(v_scale, ctypes.c_float), _p(ve, ctypes.c_uint8),
                             None if vm is None else _p(vm, ctypes.c_float), _p(vf, ctypes.c_float),
                             in_dtype, S, D, int(bool(is_causal)), ctypes.c_float(sm_scale), pv_mode,
                             _p(rows, ctypes.c_int), rows.size, None if qkr is None else _p(qkr, ctypes.c_float),
                             None if dl is None else _p(dl, ctypes.c_float), blk_d, _p(out, ctypes.c_float))
    return out


def attn_exact_head(qf, kf, vf, *, is_causal, sm_scale, rows=None) -> np.ndarray:
    qf, kf, vf = _f32(qf), _f32(kf), _f32(vf)
    Sq, D = qf.shape
    S = kf.shape[0]  # keys
    rows = np.arange(Sq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    out = np.empty((rows.size, D), np.float64)
    lib().orc_attn_exact_head(_p(qf, ctypes.c_float), _p(kf, ctypes.c_float), _p(vf, ctypes.c_float), S, D,
                              int(bool(is_causal)), ctypes.c_double(sm_scale), _p(rows, ctypes.c_int), rows.size,
                              _p(out, ctypes.c_double))
    return out


# ---------------------------------------------------------------- whole tensors
def smooth_quant_qk(q, k, dtype: int, layout: str, blk_q: int = 32, blk_k: int = 64, smooth: bool = True):
    """Quantise physical Q, K (uint16 codes) -> logical [B,H,S,D] Q codes + scales and
    [B,H_kv,S,D] K codes + scales + K means (K may have fewer heads than Q)."""
    B, H, S, D = logical_shape(q.shape, layout)
    Hkv = logical_shape(k.shape, layout)[1]
    nq, nk = (S + blk_q - 1) // blk_q, (S + blk_k - 1) // blk_k
    q8 = np.empty((B, H, S, D), np.int8)
    k8 = np.empty((B, Hkv, S, D), np.int8)
    qs = np.empty((B, H, nq), np.float32)
    ks = np.empty((B, Hkv, nk), np.float32)
    km = np.empty((B, Hkv, D), np.float32)
    for b in range(B):
        for h in range(H):
            q8[b, h], qs[b, h] = quant_q_head(decode16(head(q, layout, b, h), dtype), blk_q)
        for h in range(Hkv):
            k8[b, h], ks[b, h], km[b, h] = quant_k_head(decode16(head(k, layout, b, h), dtype), blk_k, smooth)
    return q8, qs, k8, ks, km


def quant_v(v, dtype: int, layout: str):
    """Quantise physical V (uint16 codes) -> logical [B,H,S,D] E4M3 codes + [B,H,D] scales."""
    B, H, S, D = logical_shape(v.shape, layout)
    v8 = np.empty((B, H, S, D), np.uint8)
    vs = np.empty((B, H, D), np.float32)
    for b in range(B):
        for h in range(H):
            v8[b, h], vs[b, h] = quant_v_head(decode16(head(v, layout, b, h), dtype))
    return v8, vs


def default_sm_scale(D: int) -> float:
    """1/sqrt(D) rounded once to fp32 (the usual softmax temperature)."""
    return float(np.float32(1.0 / np.sqrt(np.float64(D))))


def logical_shape(shape, layout):
    if layout == "HND":
        return tuple(shape)
    B, S, H, D = shape
    return B, H, S, D


def kv_head(h: int, H: int, Hkv: int) -> int:
    """K/V head used by query head h when K and V have Hkv <= H heads (grouped-query
    attention, "Thư viện SageAttention" page, feature list: native group-query
    attention).  Reading: the usual grouping, H / Hkv consecutive query heads share
    one K/V head."""
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"query heads {H} must be a multiple of K/V heads {Hkv}")
    return h // (H // Hkv)


def attn(q, k, v, dtype: int, layout: str, *, is_causal=False, sm_scale=None, pv_mode=PV_FP8,
         heads=None, rows=None, blk_q=BLK_Q, blk_k=BLK_K, tile_k=TILE_K, smooth=True, gran="block",
         smooth_v=False, qk_format="int8", smooth_q=False):
    """Full pipeline (smooth + quantise + attention) for the given heads/rows.

    smooth_q: Q minus its 32-token block means is quantised (INT8 or MXFP4), and
    the attention adds the pre-processing term (block mean . (K - k_mean)) * sm_scale.

    qk_format "fp4": Q and K - mean in MXFP4 (E2M1 with an E8M0 scale per 32
    channels of a token) instead of INT8 blocks; gran is then not used.

    smooth_v (pv fp8 and fp4): V minus its channel mean is quantised, and the
    mean is added back to the output.

    pv_mode PV_FP4: P~ and V in MXFP4 (scales per 32-key group of pv_group).

    gran: "block" (blk_q / blk_k tokens per scale), "lane" (thread-level: one
    scale per Q token, one per 16-key lane group of K), "token" (one scale per
    Q token and per K token: the block rule with blocks of one token) or "head"
    (one scale for all of a head's Q tokens and one for all of its K tokens:
    the block rule with one block spanning the head).
    Returns {(b, h): fp32 [len(rows), D]}; rows default to all S rows.
    """
    if gran not in ("block", "lane", "token", "head"):
        raise ValueError(gran)
    lane = gran == "lane"
    if lane:
        blk_q = 1
    if gran == "token":
        blk_q = blk_k = 1
    B, H, S, D = logical_shape(q.shape, layout)
    Hkv = logical_shape(k.shape, layout)[1]
    if sm_scale is None:
        sm_scale = default_sm_scale(D)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    res = {}
    for (b, h) in heads:
        hk = kv_head(h, H, Hkv)
        qf = decode16(head(q, layout, b, h), dtype)
        kf = decode16(head(k, layout, b, hk), dtype)
        vf = decode16(head(v, layout, b, hk), dtype)
        bq, bk = (max(qf.shape[0], 1), max(kf.shape[0], 1)) if gran == "head" else (blk_q, blk_k)
        qk = None
        if qk_format == "fp4":
            if smooth_q:  # Q minus its 32-token block means, then the MXFP4 rule
                q4, qe, qm = quant_q_head_mxfp4_smooth(qf, BLK_Q)
            else:
                q4, qe = quant_mxfp4_rows(qf)
            k4, ke, km = quant_k_head_mxfp4(kf, smooth)
            qk = qk_mxfp4_rows(q4, qe, k4, ke, rows)
            q8, qs = np.zeros(qf.shape, np.int8), np.zeros(1, np.float32)
            k8, ks = np.zeros(kf.shape, np.int8), np.zeros(1, np.float32)
        elif qk_format == "int8":
            if smooth_q:
                q8, qs, qm = quant_q_head_smooth(qf, BLK_Q, bq)
            else:
                q8, qs = quant_q_head(qf, bq)
            k8, ks, km = quant_k_head_lane(kf, smooth) if lane else quant_k_head(kf, bk, smooth)
        else:
            raise ValueError(qk_format)
        vm, ve = None, None
        if pv_mode == PV_FP8 and smooth_v:
            v8, vs, vm = quant_v_head(vf, True)
        elif pv_mode == PV_FP8:
            v8, vs = quant_v_head(vf)
        elif pv_mode == PV_FP4:
            v8, ve, vm = quant_v_head_mxfp4(vf, smooth_v)
            vs = None
            if not smooth_v:
                vm = None
        else:
            v8, vs = None, None
        res[(b, h)] = attn_head_rows(q8, qs, k8, ks, v8, vs, vf, in_dtype=dtype, is_causal=is_causal,
                                     sm_scale=sm_scale, pv_mode=pv_mode, rows=rows, blk_q=bq, blk_k=bk,
                                     tile_k=tile_k, k_lane=lane, v_mean=vm, qk=qk, v_e8m0=ve,
                                     delta=qk_delta_head(qm, kf, km) if smooth_q else None)
    return res


def attn_exact(q, k, v, dtype: int, layout: str, *, is_causal=False, sm_scale=None, heads=None, rows=None):
    B, H, S, D = logical_shape(q.shape, layout)
    Hkv = logical_shape(k.shape, layout)[1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    res = {}
    for (b, h) in heads:
        hk = kv_head(h, H, Hkv)
        res[(b, h)] = attn_exact_head(decode16(head(q, layout, b, h), dtype), decode16(head(k, layout, b, hk), dtype),
                                      decode16(head(v, layout, b, hk), dtype), is_causal=is_causal,
                                      sm_scale=sm_scale, rows=rows)
    return res


# ---------------------------------------------------------------- packed variable-length batches
def seq_slices(cu_seqlens) -> list:
    """[(start, end)] of each sequence from the prefix sums cu_seqlens[0..B]."""
    cu = [int(x) for x in cu_seqlens]
    if not cu or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    return list(zip(cu[:-1], cu[1:]))


def attn_varlen(q, k, v, cu_q, cu_k, dtype: int, *, is_causal=False, sm_scale=None, pv_mode=PV_FP8,
                heads=None, rows=None, blk_q=BLK_Q, blk_k=BLK_K, tile_k=TILE_K, smooth=True, gran="block",
                smooth_v=False, qk_format="int8", smooth_q=False):
    """Quantized attention over a packed batch of sequences of different lengths
    ("Thư viện SageAttention" page, feature list: variable-length sequences through
    sageattn_varlen).

    q: [Tq, H, D] and k, v: [Tk, Hkv, D] uint16 codes, the tokens of sequence b
    at rows cu_q[b] .. cu_q[b+1] of q and cu_k[b] .. cu_k[b+1] of k and v.
    Reading: each sequence is attended on its own, exactly as a batch of one
    (the K mean, the INT8 blocks, the V scales and the causal mask all start
    at the sequence's first token); query and key counts may differ, causal
    keeps key n for query i when n <= i, and a sequence without keys gives 0.
    smooth_q: each sequence's Q blocks (32 tokens from its first token) are
    smoothed as in attn.

    heads: [(b, h)] (default: all); rows: query rows within each sequence.
    Returns {(b, h): fp32 [rows, D]}.
    """
    sq, sk = seq_slices(cu_q), seq_slices(cu_k)
    if len(sq) != len(sk) or sq[-1][1] != q.shape[0] or sk[-1][1] != k.shape[0] or v.shape != k.shape:
        raise ValueError("cu_seqlens do not describe q / k / v")
    H, Hkv = q.shape[1], k.shape[1]
    heads = [(b, h) for b in range(len(sq)) for h in range(H)] if heads is None else heads
    res = {}
    for (b, h) in heads:
        (q0, q1), (k0, k1) = sq[b], sk[b]
        one = attn(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], dtype, "NHD", is_causal=is_causal,
                   sm_scale=sm_scale, pv_mode=pv_mode, heads=[(0, h)], rows=rows, blk_q=blk_q, blk_k=blk_k,
                   tile_k=tile_k, smooth=smooth, gran=gran, smooth_v=smooth_v, qk_format=qk_format,
                   smooth_q=smooth_q)
        res[(b, h)] = one[(0, h)]
    return res
