"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point that include/sage.h declares, and rejects bad arguments
before touching a device."""
import os
import re

import pytest

import quantized_attention_02_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|char|void)\s*\*?\s*(sage_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(qa.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = qa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    nm = os.popen(f"nm -D --defined-only {qa.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", nm), name


def test_config_and_sizes():
    assert qa.sage_get_config() == (32, 64, qa.TILE_K["fp8"], qa.TILE_K["fp16"])
    s = qa.sage_buffer_sizes(2, 3, 3, 100, 64)
    sq = {"q_mean": 6 * 4 * 64 * 4, "delta_s": 6 * 4 * 128 * 4}  # smoothed Q: [B][H][nq][D], [B][H][nq][S_k]
    assert s == {"q_i8": 6 * 128 * 64, "q_scale": 6 * 4 * 4, "k_i8": 6 * 128 * 64, "k_scale": 6 * 2 * 4,
                 "k_mean": 6 * 64 * 4, "v_fp8": 6 * 128 * 64, "v_scale": 6 * 64 * 4, **sq}
    # lane granularity: one Q scale per (padded) token row, one K scale per 16-key group
    # MXFP4: D / 2 code bytes and D / 32 E8M0 bytes a row
    s4 = qa.sage_buffer_sizes(2, 3, 3, 100, 64, qa.QK["mxfp4"])
    assert s4 == {"q_i8": 6 * 128 * 32, "q_scale": 6 * 128 * 2, "k_i8": 6 * 128 * 32, "k_scale": 6 * 128 * 2,
                  "k_mean": 6 * 64 * 4, "v_fp8": 6 * 128 * 64, "v_scale": 6 * 64 * 4, **sq}
    s = qa.sage_buffer_sizes(2, 3, 3, 100, 64, qa.QK["int8_lane"])
    assert s == {"q_i8": 6 * 128 * 64, "q_scale": 6 * 128 * 4, "k_i8": 6 * 128 * 64, "k_scale": 6 * 8 * 4,
                 "k_mean": 6 * 64 * 4, "v_fp8": 6 * 128 * 64, "v_scale": 6 * 64 * 4, **sq}
    # per-head granularity: the per-block layout
    assert qa.sage_buffer_sizes(2, 3, 3, 100, 64, qa.QK["int8_head"]) == qa.sage_buffer_sizes(2, 3, 3, 100, 64)
    # per-token granularity: one scale per (padded) Q row and per (padded) K row
    s = qa.sage_buffer_sizes(2, 3, 3, 100, 64, qa.QK["int8_token"])
    assert s == {"q_i8": 6 * 128 * 64, "q_scale": 6 * 128 * 4, "k_i8": 6 * 128 * 64, "k_scale": 6 * 128 * 4,
                 "k_mean": 6 * 64 * 4, "v_fp8": 6 * 128 * 64, "v_scale": 6 * 64 * 4, **sq}
    # grouped K/V: the K and V buffers hold B * H_kv heads
    s = qa.sage_buffer_sizes(2, 6, 2, 100, 64)
    assert s == {"q_i8": 12 * 128 * 64, "q_scale": 12 * 4 * 4, "k_i8": 4 * 128 * 64, "k_scale": 4 * 2 * 4,
                 "k_mean": 4 * 64 * 4, "v_fp8": 4 * 128 * 64, "v_scale": 4 * 64 * 4,
                 "q_mean": 12 * 4 * 64 * 4, "delta_s": 12 * 4 * 128 * 4}
    L = qa.lib()
    assert L.sage_get_config(None, None, None, None) == qa.SAGE_ERR_INVALID_ARG
    for bad in [(0, 1, 1, 1, 64, 0), (1, 0, 1, 1, 64, 0), (1, 1, 1, 0, 64, 0), (1, 1, 1, 1, 96, 0),
                (1, 1, 1, (1 << 20) + 1, 64, 0), (1, 4, 0, 1, 64, 0), (1, 4, 3, 1, 64, 0), (1, 4, 8, 1, 64, 0),
                (1, 4, -4, 1, 64, 0), (1, 1, 1, 1, 64, 5), (1, 1, 1, 1, 64, -1)]:
        assert L.sage_buffer_sizes(*bad, *([None] * 9)) == qa.SAGE_ERR_INVALID_ARG


def test_arch_check():
    assert qa.sage_check_arch("gfx950") == qa.SAGE_OK
    assert qa.sage_check_arch("gfx950:sramecc+:xnack-") == qa.SAGE_OK
    for other in ("gfx942", "gfx942:sramecc+:xnack-", "gfx90a", "gfx9500", "sm_90", ""):
        assert qa.sage_check_arch(other) == qa.SAGE_ERR_UNSUPPORTED, other
    assert qa.sage_check_arch(None) == qa.SAGE_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert qa.status_str(s) and qa.status_str(s) != "unknown status"
    assert qa.status_str(99) == "unknown status"


def test_vpos_key_is_a_permutation():
    f = lambda p: 32 * ((p & 31) >> 4) + 8 * ((p & 15) >> 2) + 4 * (p >> 5) + (p & 3)
    assert sorted(f(p) for p in range(64)) == list(range(64))


# a valid-looking set of (fake, aligned, non-null) device pointers
P = 1 << 12
GOOD_QK = dict(q=P, k=P, dtype=0, B=1, H=2, H_kv=2, S=100, D=64, layout=0, qk_quant=0, q_i8=P, q_scale=P, k_i8=P,
               k_scale=P, k_mean=P, q_mean=None, stream=None)
GOOD_DELTA = dict(k=P, dtype=0, B=1, H=4, H_kv=2, S=100, D=64, layout=1, qk_quant=0, is_causal=0, q_mean=P, k_mean=P,
                  q_scale=P, k_scale=P, delta_s=P, stream=None)
GOOD_V = dict(v=P, dtype=0, B=1, H=2, S=100, D=64, layout=0, v_fp8=P, v_scale=P, v_mean=None, stream=None)
GOOD_ATTN = dict(q_i8=P, q_scale=P, k_i8=P, k_scale=P, v=P, v_scale=P, v_mean=None, q_mean=None, delta_s=None, out=P, dtype=0, B=1,
                 H=2, H_kv=2, S=100,
                 D=64, layout=0, is_causal=0, sm_scale=0.125, pv_mode=0, qk_quant=0, stream=None)

BAD_QK = [dict(q=None), dict(k_mean=None), dict(q_i8=P + 8), dict(k=P + 2), dict(q_scale=P + 2), dict(dtype=2),
          dict(layout=-1), dict(B=0), dict(H=-1), dict(S=0), dict(D=32), dict(D=256), dict(S=(1 << 20) + 1),
          dict(B=1 << 9, H=1 << 8, H_kv=1 << 8), dict(H_kv=0), dict(H_kv=3), dict(H=3, H_kv=2), dict(H_kv=-2),
          dict(qk_quant=5), dict(qk_quant=-1), dict(q_mean=P + 2),
          dict(qk_quant=4, q_mean=P)]  # per-head scales: no smoothed Q
BAD_DELTA = [dict(k=None), dict(q_mean=None), dict(k_mean=None), dict(delta_s=None), dict(q_mean=P + 4),
             dict(delta_s=P + 2), dict(delta_s=P + 4), dict(k=P + 8), dict(H_kv=3), dict(D=96), dict(layout=2),
             # INT8 per-block scales: the term in score units needs both scale buffers
             dict(q_scale=None), dict(k_scale=None), dict(q_scale=P + 2), dict(qk_quant=4), dict(qk_quant=5),
             dict(dtype=4), dict(S=0), dict(is_causal=2), dict(is_causal=-1)]
BAD_V = [dict(v=None), dict(v_fp8=P + 4), dict(v_scale=None), dict(dtype=7), dict(layout=3), dict(D=80),
         dict(v_mean=P + 2)]
BAD_ATTN = [dict(q_i8=None), dict(out=None), dict(v=P + 1), dict(out=P + 8), dict(v_scale=None),
            dict(sm_scale=0.0), dict(sm_scale=-1.0), dict(sm_scale=float("inf")), dict(sm_scale=float("nan")),
            dict(is_causal=2), dict(pv_mode=3), dict(pv_mode=-1), dict(pv_mode=2, v_scale=None), dict(pv_mode=2, v_scale=P + 2), dict(dtype=5), dict(D=100), dict(S=0),
            dict(H_kv=0), dict(H_kv=4), dict(H=6, H_kv=4), dict(H_kv=-1), dict(qk_quant=5), dict(qk_quant=4, delta_s=P, q_mean=P),
            dict(v_mean=P + 1), dict(pv_mode=1, v_scale=None, v_mean=P),  # smoothing is for the FP8 V codes
            dict(delta_s=P + 2),
            # INT8 per-block scales: the term in score units comes with the block means
            dict(delta_s=P), dict(delta_s=P, q_mean=P + 2),
            # pv fp16 reads 128-token slices of an NHD V through a 32-bit byte range: H_kv * D * 2 * 128 < 2^31
            dict(pv_mode=1, v_scale=None, layout=1, B=1, H=1 << 16, H_kv=1 << 16, D=128)]


GOOD_QKV = dict(q=P, k=P, v=P, dtype=0, B=1, H=4, H_kv=2, S=100, D=64, layout=0, qk_quant=0, q_i8=P, q_scale=P,
                k_i8=P, k_scale=P, k_mean=P, q_mean=None, v_fp8=P, v_scale=P, v_mean=None, stream=None)
# every check of the Q/K call and of the V call (on the H_kv V heads)
BAD_QKV = [b for b in BAD_QK if "H" not in b and "B" not in b] + [dict(v=None), dict(v=P + 2), dict(v_fp8=P + 4),
                                                                   dict(v_scale=None), dict(v_scale=P + 1),
                                                                   dict(v_mean=P + 2), dict(H_kv=3), dict(H=3)]


def _call_qkv(**kw):
    a = {**GOOD_QKV, **kw}
    return qa.sage_quantize_qkv(*a.values())


@pytest.mark.parametrize("bad", BAD_QKV, ids=[str(b) for b in BAD_QKV])
def test_quantize_qkv_rejects(bad):
    assert _call_qkv(**bad) == qa.SAGE_ERR_INVALID_ARG


def _call_qk(**kw):
    a = {**GOOD_QK, **kw}
    return qa.sage_smooth_quant_qk(*a.values())


def _call_v(**kw):
    a = {**GOOD_V, **kw}
    return qa.sage_quant_v(*a.values())


def _call_attn(**kw):
    a = {**GOOD_ATTN, **kw}
    return qa.sage_attn_fwd(*a.values())


@pytest.mark.parametrize("bad", BAD_QK, ids=[str(b) for b in BAD_QK])
def test_smooth_quant_qk_rejects(bad):
    assert _call_qk(**bad) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_DELTA, ids=[str(b) for b in BAD_DELTA])
def test_qk_delta_rejects(bad):
    assert qa.sage_qk_delta(*{**GOOD_DELTA, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_V, ids=[str(b) for b in BAD_V])
def test_quant_v_rejects(bad):
    assert _call_v(**bad) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_ATTN, ids=[str(b) for b in BAD_ATTN])
def test_attn_fwd_rejects(bad):
    assert _call_attn(**bad) == qa.SAGE_ERR_INVALID_ARG


def test_attn_fp16_mode_accepts_null_v_scale_then_needs_device():
    rc = _call_attn(pv_mode=1, v_scale=None)
    assert rc in (qa.SAGE_ERR_NO_DEVICE, qa.SAGE_OK, qa.SAGE_ERR_UNSUPPORTED) or rc != qa.SAGE_ERR_INVALID_ARG
    # the largest NHD head count the fp16 mode takes passes the argument checks
    rc = _call_attn(pv_mode=1, v_scale=None, layout=1, B=1, H=(1 << 16) - 1, H_kv=(1 << 16) - 1, D=128)
    assert rc != qa.SAGE_ERR_INVALID_ARG
    # the limit is on the V tensor's heads: many query heads over few K/V heads pass
    rc = _call_attn(pv_mode=1, v_scale=None, layout=1, B=1, H=1 << 16, H_kv=1 << 10, D=128)
    assert rc != qa.SAGE_ERR_INVALID_ARG


def test_dump_rejects_bad_head_and_buffer():
    a = [v for k, v in GOOD_ATTN.items() if k not in ("q_mean", "delta_s", "stream")]  # no smoothed-Q term
    assert qa.sage_attn_fwd_dump_qk(*a, 0, 2, P, None) == qa.SAGE_ERR_INVALID_ARG  # h out of range
    a[-1] = 5
    assert qa.sage_attn_fwd_dump_qk(*a, 0, 0, P, None) == qa.SAGE_ERR_INVALID_ARG  # bad Q/K mode
    a[-1] = qa.QK["mxfp4"]
    assert qa.sage_attn_fwd_dump_qk(*a, 0, 0, P, None) == qa.SAGE_ERR_INVALID_ARG  # the dump is INT8 only
    a[-1] = 0
    assert qa.sage_attn_fwd_dump_qk(*a, -1, 0, P, None) == qa.SAGE_ERR_INVALID_ARG
    assert qa.sage_attn_fwd_dump_qk(*a, 0, 0, None, None) == qa.SAGE_ERR_INVALID_ARG


def _no_gpu():
    import torch

    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful on a host without a GPU")
def test_valid_arguments_without_a_device_report_no_device():
    assert _call_qk() == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(H=8, H_kv=2) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(qk_quant=1) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(qk_quant=1) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(qk_quant=2) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(qk_quant=2) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(qk_quant=3) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(qk_quant=3) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(qk_quant=4) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(qk_quant=4, delta_s=None) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qkv(qk_quant=4) == qa.SAGE_ERR_NO_DEVICE
    assert _call_v(v_mean=P) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(q_mean=P) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(delta_s=P, q_mean=P) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(delta_s=P, qk_quant=1) == qa.SAGE_ERR_NO_DEVICE  # fp32 terms: no means needed
    assert qa.sage_qk_delta(*GOOD_DELTA.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_qk_delta(*{**GOOD_DELTA, "is_causal": 1}.values()) == qa.SAGE_ERR_NO_DEVICE
    # the other Q/K formats write fp32 terms and do not read the scales
    assert qa.sage_qk_delta(*{**GOOD_DELTA, "qk_quant": 1, "q_scale": None, "k_scale": None}.values()) == \
        qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(v_mean=P) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(H=8, H_kv=1) == qa.SAGE_ERR_NO_DEVICE
    assert _call_v() == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn() == qa.SAGE_ERR_NO_DEVICE
    assert _call_qkv() == qa.SAGE_ERR_NO_DEVICE
    assert _call_qkv(q_mean=P, v_mean=P, qk_quant=1) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qkv(qk_quant=2, H=8, H_kv=1) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(q_mean=P, qk_quant=2) == qa.SAGE_ERR_NO_DEVICE  # smoothed Q with MXFP4
    assert _call_attn(delta_s=P, qk_quant=2) == qa.SAGE_ERR_NO_DEVICE


def test_python_wrapper_maps_unsupported_to_value_error(monkeypatch):
    with pytest.raises(ValueError):
        qa._check(qa.SAGE_ERR_UNSUPPORTED, "x")
    with pytest.raises(qa.SageError):
        qa._check(qa.SAGE_ERR_INVALID_ARG, "x")


# ---- packed variable-length batches
def test_varlen_buffer_sizes():
    s = qa.sage_varlen_buffer_sizes(3, 4, 2, 100, 200, 64)
    rq, rk = 32 * (100 // 32 + 3 + 1), 128 * (200 // 128 + 3 + 1)
    assert (rq, rk) == (qa.varlen_rows(100, 3, 32), qa.varlen_rows(200, 3, 128)) == (224, 640)
    assert s == {"q_i8": 4 * rq * 64, "q_scale": 4 * (rq // 32) * 4, "k_i8": 2 * rk * 64, "k_scale": 2 * (rk // 64) * 4,
                 "k_mean": 3 * 2 * 64 * 4, "v_fp8": 2 * rk * 64, "v_scale": 3 * 2 * 64 * 4}
    s = qa.sage_varlen_buffer_sizes(3, 4, 2, 100, 200, 64, qa.QK["int8_lane"])
    assert s["q_scale"] == 4 * rq * 4 and s["k_scale"] == 2 * (rk // 16) * 4
    s = qa.sage_varlen_buffer_sizes(3, 4, 2, 100, 200, 64, qa.QK["int8_token"])
    assert s["q_scale"] == 4 * rq * 4 and s["k_scale"] == 2 * rk * 4
    # every sequence's padded run fits in the buffer wherever the sequence starts
    for total, B, pad in ((100, 3, 32), (200, 3, 128), (0, 1, 32), (4095, 7, 128)):
        rows = qa.varlen_rows(total, B, pad)
        for b in range(B):
            for start in range(total + 1):
                for n in (0, 1, pad - 1, pad, total - start):
                    if 0 <= n <= total - start:
                        r0 = qa.varlen_row0(start, b, pad)
                        assert r0 % pad == 0 and r0 + -(-n // pad) * pad <= rows
    L = qa.lib()
    for bad in [(0, 1, 1, 1, 1, 64, 0), (1, 4, 3, 1, 1, 64, 0), (1, 1, 1, -1, 1, 64, 0), (1, 1, 1, 1, -5, 64, 0),
                (1, 1, 1, 1, 1, 96, 0), (1, 1, 1, (1 << 30) + 1, 1, 64, 0), (1, 1, 1, 1, 1, 64, 5)]:
        assert L.sage_varlen_buffer_sizes(*bad, *([None] * 7)) == qa.SAGE_ERR_INVALID_ARG, bad


GOOD_QK_VL = dict(q=P, k=P, dtype=0, cu_q=P, cu_k=P, B=3, H=4, H_kv=2, total_q=100, total_k=200, max_q=50,
                  max_k=90, D=64, qk_quant=1, q_i8=P, q_scale=P, k_i8=P, k_scale=P, k_mean=P, q_mean=None, stream=None)
GOOD_V_VL = dict(v=P, dtype=1, cu_k=P, B=3, H_kv=2, total_k=200, max_k=90, D=128, v_fp8=P, v_scale=P, v_mean=P,
                 stream=None)
GOOD_ATTN_VL = dict(q_i8=P, q_scale=P, k_i8=P, k_scale=P, v=P, v_scale=P, v_mean=P, q_mean=None, delta_s=None, out=P,
                    dtype=0, cu_q=P, cu_k=P, B=3, H=4, H_kv=2, total_q=100, total_k=200, max_q=50, max_k=90, D=64, is_causal=1, sm_scale=0.125,
                    pv_mode=0, qk_quant=0, stream=None)
BAD_QK_VL = [dict(cu_q=None), dict(cu_k=P + 2), dict(B=0), dict(H_kv=3), dict(total_q=-1), dict(max_q=0),
             dict(max_k=(1 << 20) + 1), dict(D=32), dict(dtype=3), dict(q=None), dict(k_i8=P + 1), dict(qk_quant=5),
             # smoothed Q: aligned means, and not with one scale per head
             dict(q_mean=P + 2), dict(q_mean=P, qk_quant=4)]
BAD_V_VL = [dict(cu_k=None), dict(v=P + 8), dict(max_k=0), dict(total_k=-3), dict(H_kv=0), dict(v_scale=None),
            dict(v_mean=P + 2)]
BAD_ATTN_VL = [dict(cu_q=None), dict(cu_k=None), dict(cu_q=P + 1), dict(is_causal=3), dict(pv_mode=5), dict(qk_quant=7),
               dict(v_mean=P + 3), dict(pv_mode=1, v_scale=None), dict(pv_mode=2, v_scale=None), dict(pv_mode=3),
               dict(sm_scale=0.0), dict(v_scale=None), dict(out=P + 4), dict(H_kv=3), dict(max_q=0), dict(B=-1),
               # pv fp16 reads 128-token slices of V through a 32-bit byte range: H_kv * D * 2 * 128 < 2^31
               dict(pv_mode=1, v_scale=None, B=1, H=1 << 16, H_kv=1 << 16, D=128),
               # smoothed Q: the term in score units needs the block means; aligned; not per head
               dict(delta_s=P), dict(delta_s=P + 2, q_mean=P), dict(delta_s=P, q_mean=P + 1),
               dict(delta_s=P, qk_quant=4)]
GOOD_DELTA_VL = dict(k=P, dtype=0, cu_q=P, cu_k=P, B=3, H=4, H_kv=2, total_q=100, total_k=200, max_q=50, max_k=90,
                     D=64, qk_quant=0, is_causal=1, q_mean=P, k_mean=P, q_scale=P, k_scale=P, delta_s=P, stream=None)
BAD_DELTA_VL = [dict(k=None), dict(cu_q=None), dict(cu_k=P + 1), dict(q_mean=None), dict(q_mean=P + 4),
                dict(k_mean=None), dict(delta_s=P + 8), dict(delta_s=None), dict(q_scale=None), dict(k_scale=P + 2),
                dict(qk_quant=4), dict(qk_quant=6), dict(dtype=2), dict(D=96), dict(H_kv=3), dict(max_q=0),
                dict(B=0), dict(total_k=-1), dict(is_causal=3)]


@pytest.mark.parametrize("bad", BAD_QK_VL, ids=[str(b) for b in BAD_QK_VL])
def test_smooth_quant_qk_varlen_rejects(bad):
    assert qa.sage_smooth_quant_qk_varlen(*{**GOOD_QK_VL, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_V_VL, ids=[str(b) for b in BAD_V_VL])
def test_quant_v_varlen_rejects(bad):
    assert qa.sage_quant_v_varlen(*{**GOOD_V_VL, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_ATTN_VL, ids=[str(b) for b in BAD_ATTN_VL])
def test_attn_fwd_varlen_rejects(bad):
    assert qa.sage_attn_fwd_varlen(*{**GOOD_ATTN_VL, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_DELTA_VL, ids=[str(b) for b in BAD_DELTA_VL])
def test_qk_delta_varlen_rejects(bad):
    assert qa.sage_qk_delta_varlen(*{**GOOD_DELTA_VL, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


def test_varlen_smooth_q_sizes():
    # q_mean [H][RQ / 32][D] fp32; delta_s [H][RK / 128][ceil(max_q / 32)][128] fp32
    rq, rk = qa.varlen_rows(100, 3, 32), qa.varlen_rows(200, 3, 128)
    assert qa.sage_varlen_smooth_q_sizes(3, 4, 100, 200, 50, 64) == \
        {"q_mean": 4 * (rq // 32) * 64 * 4, "delta_s": 4 * (rk // 128) * 2 * 128 * 4}
    assert qa.sage_varlen_smooth_q_sizes(1, 1, 1, 1, 1, 128)["delta_s"] == qa.varlen_rows(1, 1, 128) * 4
    L = qa.lib()
    for bad in [(0, 1, 1, 1, 1, 64), (1, 0, 1, 1, 1, 64), (1, 1, -1, 1, 1, 64), (1, 1, 1, 1, 0, 64),
                (1, 1, 1, 1, 1, 80), (1, 1, 1, 1, (1 << 20) + 1, 64)]:
        assert L.sage_varlen_smooth_q_sizes(*bad, None, None) == qa.SAGE_ERR_INVALID_ARG, bad


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful on a host without a GPU")
def test_valid_varlen_arguments_without_a_device_report_no_device():
    assert qa.sage_qk_delta_varlen(*GOOD_DELTA_VL.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_qk_delta_varlen(*{**GOOD_DELTA_VL, "qk_quant": 2, "q_scale": None, "k_scale": None}.values()) == \
        qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_smooth_quant_qk_varlen(*{**GOOD_QK_VL, "q_mean": P}.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_varlen(*{**GOOD_ATTN_VL, "q_mean": P, "delta_s": P}.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_varlen(*{**GOOD_ATTN_VL, "qk_quant": 1, "delta_s": P}.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_smooth_quant_qk_varlen(*GOOD_QK_VL.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_quant_v_varlen(*GOOD_V_VL.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_varlen(*GOOD_ATTN_VL.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_varlen(*{**GOOD_ATTN_VL, "pv_mode": 1, "v_scale": None, "v_mean": None}.values()) == \
        qa.SAGE_ERR_NO_DEVICE


def test_size_limits_in_the_header():
    """The maximum sizes the GPU limit tests run at are the header's."""
    import re

    hdr = open(HEADER).read()
    assert re.search(r"#define SAGE_MAX_S \(1 << 20\)", hdr)
    assert re.search(r"#define SAGE_MAX_BH \(1 << 16\)", hdr)
    assert qa.sage_buffer_sizes(1, 1, 1, 1 << 20, 128, 0)["q_i8"] == 1 << 27  # q codes of the longest head
    with pytest.raises(qa.SageError):
        qa.sage_buffer_sizes(1, 1, 1, (1 << 20) + 1, 128, 0)
    assert qa.sage_buffer_sizes(256, 256, 64, 33, 64, 0)["k_i8"] == 256 * 64 * 128 * 64  # the most heads
    with pytest.raises(qa.SageError):
        qa.sage_buffer_sizes(257, 256, 64, 33, 64, 0)


# MXFP4 V (pv fp4): codes 16-byte and E8M0 bytes 4-byte aligned
GOOD_V4 = dict(v=P, dtype=1, B=2, H=3, S=300, D=128, layout=1, v_codes=P, v_e8m0=P, v_mean=P, stream=None)
BAD_V4 = [dict(v=None), dict(v_codes=None), dict(v_e8m0=None), dict(v_codes=P + 8), dict(v_e8m0=P + 2),
          dict(v_mean=P + 1), dict(v=P + 4), dict(dtype=2), dict(layout=2), dict(D=96), dict(S=0), dict(B=0),
          dict(H=0), dict(S=(1 << 20) + 1)]
GOOD_V4_VL = dict(v=P, dtype=0, cu_k=P, B=3, H_kv=2, total_k=200, max_k=90, D=64, v_codes=P, v_e8m0=P, v_mean=None,
                  stream=None)
BAD_V4_VL = [dict(cu_k=None), dict(cu_k=P + 2), dict(v=None), dict(v_codes=P + 4), dict(v_e8m0=None),
             dict(v_e8m0=P + 1), dict(max_k=0), dict(total_k=-1), dict(H_kv=0), dict(D=32), dict(v_mean=P + 2)]


@pytest.mark.parametrize("bad", BAD_V4, ids=[str(b) for b in BAD_V4])
def test_quant_v_fp4_rejects(bad):
    assert qa.sage_quant_v_fp4(*{**GOOD_V4, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_V4_VL, ids=[str(b) for b in BAD_V4_VL])
def test_quant_v_fp4_varlen_rejects(bad):
    assert qa.sage_quant_v_fp4_varlen(*{**GOOD_V4_VL, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


def test_v_fp4_buffer_sizes():
    # [B][H_kv][S_k / 64][D][32] code bytes and [..][2] E8M0 bytes, S_k = roundup(S, 128)
    assert qa.sage_v_fp4_buffer_sizes(2, 3, 300, 128) == {"v_codes": 6 * 384 * 64, "v_e8m0": 6 * 6 * 128 * 2}
    assert qa.sage_v_fp4_buffer_sizes(1, 1, 1, 64) == {"v_codes": 128 * 32, "v_e8m0": 2 * 64 * 2}
    rk = qa.varlen_rows(200, 3, 128)
    assert qa.sage_varlen_v_fp4_buffer_sizes(3, 2, 200, 64) == {"v_codes": 2 * rk * 32, "v_e8m0": 2 * (rk // 64) * 128}
    L = qa.lib()
    for bad in [(0, 1, 1, 64), (1, 0, 1, 64), (1, 1, 0, 64), (1, 1, 1, 96), (1, 1, (1 << 20) + 1, 64)]:
        assert L.sage_v_fp4_buffer_sizes(*bad, None, None) == qa.SAGE_ERR_INVALID_ARG, bad
    for bad in [(0, 1, 1, 64), (1, 0, 1, 64), (1, 1, -1, 64), (1, 1, 1, 32)]:
        assert L.sage_varlen_v_fp4_buffer_sizes(*bad, None, None) == qa.SAGE_ERR_INVALID_ARG, bad
    # the E8M0 buffer holds the smoothing pass's fp32 per-channel statistics (4 bytes per
    # head and channel) until the conversion overwrites it
    for B, H, S, D in [(1, 1, 1, 64), (2, 3, 300, 128)]:
        assert qa.sage_v_fp4_buffer_sizes(B, H, S, D)["v_e8m0"] >= 4 * B * H * D


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful on a host without a GPU")
def test_valid_fp4_pv_arguments_without_a_device_report_no_device():
    assert qa.sage_quant_v_fp4(*GOOD_V4.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_quant_v_fp4_varlen(*GOOD_V4_VL.values()) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(pv_mode=2) == qa.SAGE_ERR_NO_DEVICE
    assert _call_attn(pv_mode=2, v_mean=P) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_varlen(*{**GOOD_ATTN_VL, "pv_mode": 2}.values()) == qa.SAGE_ERR_NO_DEVICE


# ---- Q quantised in the attention kernel (sage_attn_fwd_q16 and the Q/K passes without Q)
NO_Q = dict(q=None, q_i8=None, q_scale=None)
GOOD_Q16 = dict(q=P, k_i8=P, k_scale=P, v=P, v_scale=P, v_mean=None, out=P, dtype=0, B=1, H=4, H_kv=2, S=100, D=64,
                layout=0, is_causal=0, sm_scale=0.125, pv_mode=0, stream=None)
BAD_Q16 = [dict(q=None), dict(q=P + 2), dict(k_i8=None), dict(k_scale=None), dict(out=P + 4), dict(v_scale=None),
           dict(pv_mode=3), dict(is_causal=2), dict(sm_scale=0.0), dict(H_kv=3), dict(D=96), dict(S=0)]
GOOD_Q16_VL = dict(q=P, k_i8=P, k_scale=P, v=P, v_scale=P, v_mean=None, out=P, dtype=1, cu_q=P, cu_k=P, B=3, H=4,
                   H_kv=2, total_q=100, total_k=200, max_q=50, max_k=90, D=128, is_causal=1, sm_scale=0.1, pv_mode=0,
                   stream=None)
BAD_Q16_VL = [dict(q=None), dict(q=P + 8), dict(cu_q=None), dict(cu_k=P + 2), dict(k_i8=None), dict(max_q=0),
              dict(pv_mode=1, v_scale=None, v_mean=P), dict(B=0)]
# the Q/K passes may omit Q only as a whole, with INT8 per-block scales and unsmoothed Q
BAD_NO_Q = [dict(NO_Q, qk_quant=1), dict(NO_Q, qk_quant=2), dict(NO_Q, qk_quant=3), dict(NO_Q, qk_quant=4),
            dict(NO_Q, q_mean=P), dict(q=None), dict(q_i8=None), dict(q_scale=None), dict(q=None, q_i8=None),
            dict(NO_Q, k_i8=None), dict(NO_Q, k_mean=None)]


@pytest.mark.parametrize("bad", BAD_Q16, ids=[str(b) for b in BAD_Q16])
def test_attn_fwd_q16_rejects(bad):
    assert qa.sage_attn_fwd_q16(*{**GOOD_Q16, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_Q16_VL, ids=[str(b) for b in BAD_Q16_VL])
def test_attn_fwd_varlen_q16_rejects(bad):
    assert qa.sage_attn_fwd_varlen_q16(*{**GOOD_Q16_VL, **bad}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_NO_Q, ids=[str(b) for b in BAD_NO_Q])
def test_qk_passes_omit_q_only_as_a_whole(bad):
    assert _call_qk(**bad) == qa.SAGE_ERR_INVALID_ARG
    assert _call_qkv(**bad) == qa.SAGE_ERR_INVALID_ARG
    vl = {k: v for k, v in bad.items()}
    assert qa.sage_smooth_quant_qk_varlen(*{**GOOD_QK_VL, "qk_quant": 0, **vl}.values()) == qa.SAGE_ERR_INVALID_ARG


@pytest.mark.skipif(not _no_gpu(), reason="only meaningful on a host without a GPU")
def test_valid_q16_arguments_without_a_device_report_no_device():
    assert qa.sage_attn_fwd_q16(*GOOD_Q16.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_q16(*{**GOOD_Q16, "pv_mode": 1, "v_scale": None}.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_q16(*{**GOOD_Q16, "pv_mode": 2, "v_mean": P}.values()) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_attn_fwd_varlen_q16(*GOOD_Q16_VL.values()) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qk(**NO_Q) == qa.SAGE_ERR_NO_DEVICE
    assert _call_qkv(**NO_Q) == qa.SAGE_ERR_NO_DEVICE
    assert qa.sage_smooth_quant_qk_varlen(*{**GOOD_QK_VL, "qk_quant": 0, **NO_Q}.values()) == qa.SAGE_ERR_NO_DEVICE
