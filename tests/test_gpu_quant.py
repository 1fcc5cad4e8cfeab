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
