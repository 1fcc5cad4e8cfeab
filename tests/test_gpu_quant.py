"""GPU quantisation passes vs the oracle: INT8 codes, scales, K means and FP8 V
codes/scales must be bit-identical (same fp32 decisions on both sides)."""
import numpy as np
import pytest

import oracle as O
from quantized_attention_02_amd import synth

import gpu_util as G

pytestmark = pytest.mark.gpu

SMALL = [synth.WORKLOADS["tiny_b1h2s256d64"], synth.WORKLOADS["snippet_b1h16s512d64"]]
EDGE = [
    synth.custom(1, 2, 1, 64, seed=101),
    synth.custom(1, 1, 31, 128, dtype="bf16", seed=102),
    synth.custom(2, 3, 100, 64, layout="NHD", seed=103),
    synth.custom(1, 2, 257, 128, dtype="bf16", layout="NHD", outlier_p=0.01, seed=104),
    synth.custom(1, 3, 1000, 128, token_norm=True, seed=105),
    # grouped-query attention: K / V have fewer heads than Q
    synth.custom(2, 6, 300, 64, Hkv=2, seed=106),
    synth.custom(1, 8, 257, 128, dtype="bf16", layout="NHD", Hkv=1, seed=107),
]
FULL = [synth.WORKLOADS[n] for n in ("snippet_b2h32s4096d128", "prefill_b1h32s32768d128", "dit_b1h20s16384d128",
                                     "gqa_b1h32kv8s8192d128")]


def _heads(B, H, full):
    if not full:
        return [(b, h) for b in range(B) for h in range(H)]
    return sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)})


def _check_quant(w, full):
    q, k, v = G.inputs(w)
    bufs, _, _ = G.run(w)
    dt = O.DTYPES[w.dtype]
    q8 = bufs.q_i8.cpu().numpy()
    k8 = bufs.k_i8.cpu().numpy()
    qs, ks, km = bufs.q_scale.cpu().numpy(), bufs.k_scale.cpu().numpy(), bufs.k_mean.cpu().numpy()
    v8 = G.v8_logical(bufs.v_fp8, w.S)
    vs = bufs.v_scale.cpu().numpy()
    S = w.S
    assert q8.shape[1] == w.H and k8.shape[1] == w.kv_heads and bufs.v_fp8.shape[1] == w.kv_heads
    for (b, h) in _heads(w.B, w.H, full):
        qf = O.decode16(O.head(q, w.layout, b, h), dt)
        rq8, rqs = O.quant_q_head(qf, 32)
        assert np.array_equal(qs[b, h].view(np.uint32), rqs.view(np.uint32)), (b, h)
        assert np.array_equal(q8[b, h, :S], rq8), (b, h, int((q8[b, h, :S] != rq8).sum()))
    for (b, h) in _heads(w.B, w.kv_heads, full):
        kf = O.decode16(O.head(k, w.layout, b, h), dt)
        vf = O.decode16(O.head(v, w.layout, b, h), dt)
        rk8, rks, rkm = O.quant_k_head(kf, 64, True)
        rv8, rvs = O.quant_v_head(vf)
        assert np.array_equal(km[b, h].view(np.uint32), rkm.view(np.uint32)), (b, h)
        nkb = rks.size  # blocks that hold real keys; the rest pad the buffer to whole 128-key tiles
        assert np.array_equal(ks[b, h, :nkb].view(np.uint32), rks.view(np.uint32)), (b, h)
        assert not ks[b, h, nkb:].any()
        assert np.array_equal(k8[b, h, :S], rk8), (b, h, int((k8[b, h, :S] != rk8).sum()))
        assert np.array_equal(vs[b, h].view(np.uint32), rvs.view(np.uint32)), (b, h)
        assert np.array_equal(v8[b, h], rv8), (b, h, int((v8[b, h] != rv8).sum()))
    # padding rows / keys are zero
    assert not q8[:, :, S:].any() and not k8[:, :, S:].any()
    nk = bufs.v_fp8.shape[2]
    if nk * 64 > S:
        pad = G.v8_logical(bufs.v_fp8, nk * 64)[:, :, S:]
        assert not pad.any()


@pytest.mark.parametrize("w", SMALL + EDGE, ids=[w.name for w in SMALL + EDGE])
def test_quant_bit_exact_small(w):
    _check_quant(w, full=False)


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_quant_bit_exact_full_size_sampled_heads(w):
    _check_quant(w, full=True)


def test_quant_all_zero_inputs():
    """Degenerate case: all-zero Q/K/V give scale 0 and codes 0 (no NaN)."""
    import torch

    import quantized_attention_02_amd as qa

    z = torch.zeros((1, 2, 96, 64), dtype=torch.float16, device="cuda")
    bufs = qa.quantize(z, z, z, "HND", "fp8")
    torch.cuda.synchronize()
    for t in (bufs.q_scale, bufs.k_scale, bufs.k_mean, bufs.v_scale):
        assert not t.any() and torch.isfinite(t).all()
    for t in (bufs.q_i8, bufs.k_i8, bufs.v_fp8):
        assert not t.any()


FUSED_CASES = [
    (synth.custom(1, 2, 256, 64, seed=1401), "int8", False, False),
    (synth.custom(2, 6, 300, 128, layout="NHD", Hkv=2, seed=1402), "int8", True, False),
    (synth.custom(1, 4, 257, 128, dtype="bf16", layout="NHD", seed=1403), "int8_lane", False, True),
    (synth.custom(2, 3, 100, 64, dtype="bf16", seed=1404), "mxfp4", True, False),
    (synth.custom(1, 8, 1000, 128, Hkv=4, token_norm=True, q_bias_sigma=3.0, seed=1405), "int8", True, True),
    (synth.custom(1, 2, 1, 64, seed=1406), "int8_lane", True, True),
    (synth.WORKLOADS["snippet_b2h32s4096d128"], "int8", False, False),
    (synth.custom(2, 4, 130, 128, layout="NHD", Hkv=2, q_bias_sigma=3.0, seed=1407), "mxfp4", True, True),
    (synth.custom(2, 4, 300, 64, Hkv=2, token_norm=True, seed=1408), "int8_token", True, False),
    (synth.custom(1, 2, 129, 128, dtype="bf16", layout="NHD", q_bias_sigma=3.0, seed=1409), "int8_token", False, True),
    (synth.custom(2, 4, 300, 64, Hkv=2, token_norm=True, seed=1410), "int8_head", True, False),
    (synth.custom(1, 3, 1000, 128, dtype="bf16", layout="NHD", seed=1411), "int8_head", False, False),
]


@pytest.mark.parametrize("w,qk,smooth_v,smooth_q", FUSED_CASES,
                         ids=[f"{w.name}-{qk}-sv{int(sv)}-sq{int(sq)}" for w, qk, sv, sq in FUSED_CASES])
def test_quantize_qkv_equals_the_two_calls(w, qk, smooth_v, smooth_q):
    """sage_quantize_qkv (four launches) writes every buffer bit for bit as
    sage_smooth_quant_qk followed by sage_quant_v does."""
    import quantized_attention_02_amd as qa

    import torch

    q, k, v = (G.to_device(x, w.dtype) for x in G.inputs(w))
    res = []
    for fused in (True, False):
        # every buffer starts as the same byte pattern, so a byte that only one
        # of the two paths writes shows up as a difference
        bufs = qa.Quantized(w.B, w.H, w.S, w.D, q.device, w.kv_heads, qk)
        nq, sk = bufs.q_i8.shape[2] // qa.BLK_Q, bufs.k_i8.shape[2]
        bufs.q_mean = torch.empty((w.B, w.H, nq, w.D), dtype=torch.float32, device=q.device)
        bufs.delta_s = torch.empty((w.B, w.H, sk // qa.KV_PAD, nq, qa.KV_PAD), dtype=torch.float32, device=q.device)
        for n in ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_fp8", "v_scale", "v_mean", "q_mean", "delta_s"):
            getattr(bufs, n).view(torch.uint8).fill_(0xA5)
        qa.quantize(q, k, v, w.layout, "fp8", bufs, qk_quant=qk, smooth_v=smooth_v, smooth_q=smooth_q, fused=fused)
        torch.cuda.synchronize()
        names = ["q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_fp8", "v_scale"]
        names += ["v_mean"] if smooth_v else []
        names += ["q_mean", "delta_s"] if smooth_q else []
        res.append({n: getattr(bufs, n).cpu().numpy().view(np.uint8) for n in names})
    for n in res[0]:
        assert np.array_equal(res[0][n], res[1][n]), n
