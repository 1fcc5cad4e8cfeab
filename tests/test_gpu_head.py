"""GPU per-head INT8 granularity vs the oracle: one scale for all of a head's Q
tokens and one for all of its K - k_mean tokens, stored in every block slot of
the per-block scale layout.

Codes and scales bit-identical (fixed-length and packed batches); the int32
Q.K^T bit-identical; outputs within the attention bars (cosine >= 0.999, mean
relative L1 <= 1e-2) of the oracle run at the same granularity; smoothed Q is
rejected with this mode.
"""
import numpy as np
import pytest

import oracle as O
from quantized_attention_02_amd import synth

import gpu_util as G

pytestmark = pytest.mark.gpu

COS_MIN, REL_L1_MAX = G.COS_MIN, G.REL_L1_MAX
W = synth.WORKLOADS

QUANT_CASES = [
    W["tiny_b1h2s256d64"],
    synth.custom(1, 2, 1, 64, seed=1601),
    synth.custom(2, 3, 100, 64, layout="NHD", seed=1602),
    synth.custom(1, 2, 257, 128, dtype="bf16", layout="NHD", outlier_p=0.01, seed=1603),
    synth.custom(2, 6, 300, 128, Hkv=2, token_norm=True, seed=1604),
    synth.custom(1, 2, 9000, 64, seed=1605),  # more than 32 chunks' worth: 512-token chunks
]


def _check_head_quant(q8, qs, k8, ks, km, q, k, w, dt):
    S = w.S
    for b in range(w.B):
        for h in range(w.H):
            rq8, rqs = O.quant_q_head(O.decode16(O.head(q, w.layout, b, h), dt), S)
            assert np.array_equal(q8[b, h, :S], rq8), (b, h)
            assert (qs[b, h].view(np.uint32) == rqs.view(np.uint32)[0]).all(), (b, h)
        for h in range(w.kv_heads):
            rk8, rks, rkm = O.quant_k_head(O.decode16(O.head(k, w.layout, b, h), dt), S, True)
            assert np.array_equal(k8[b, h, :S], rk8), (b, h)
            assert not k8[b, h, S:].any()
            assert (ks[b, h].view(np.uint32) == rks.view(np.uint32)[0]).all(), (b, h)
            assert np.array_equal(km[b, h].view(np.uint32), rkm.view(np.uint32)), (b, h)


@pytest.mark.parametrize("w", QUANT_CASES, ids=[w.name for w in QUANT_CASES])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "two_calls"])
def test_head_quant_bit_exact(w, fused):
    import quantized_attention_02_amd as qa

    q, k, v = G.inputs(w)
    qd, kd, vd = (G.to_device(x, w.dtype) for x in (q, k, v))
    bufs = qa.quantize(qd, kd, vd, w.layout, "fp8", qk_quant="int8_head", fused=fused)
    import torch

    torch.cuda.synchronize()
    assert bufs.q_scale.shape[-1] == bufs.q_i8.shape[2] // 32 and bufs.k_scale.shape[-1] == bufs.k_i8.shape[2] // 64
    _check_head_quant(bufs.q_i8.cpu().numpy(), bufs.q_scale.cpu().numpy(), bufs.k_i8.cpu().numpy(),
                      bufs.k_scale.cpu().numpy(), bufs.k_mean.cpu().numpy(), q, k, w, O.DTYPES[w.dtype])


ATTN_CASES = [
    (W["tiny_b1h2s256d64"], False, "fp8"),
    (W["snippet_b1h16s512d64"], True, "fp8"),
    (W["snippet_b1h16s512d64"], False, "fp16"),
    (synth.custom(1, 2, 1, 64, seed=1611), False, "fp8"),
    (synth.custom(1, 1, 31, 128, dtype="bf16", seed=1612), True, "fp16"),
    (synth.custom(2, 3, 100, 64, layout="NHD", seed=1613), True, "fp8"),
    (synth.custom(1, 2, 257, 128, dtype="bf16", layout="NHD", seed=1614), False, "fp8"),
    (synth.custom(2, 6, 300, 128, Hkv=2, seed=1615), True, "fp8"),
]


def _ids(cases):
    return [f"{w.name}-{'causal' if c else 'full'}-{pv}" for w, c, pv in cases]


@pytest.mark.parametrize("w,causal,pv", ATTN_CASES, ids=_ids(ATTN_CASES))
def test_head_attn_matches_oracle(w, causal, pv):
    _, out, _ = G.run(w, causal=causal, pv=pv, qk_quant="int8_head")
    got = G.out_logical(out, w)
    q, k, v = G.inputs(w)
    ref = O.attn(q, k, v, O.DTYPES[w.dtype], w.layout, is_causal=causal,
                 pv_mode=O.PV_FP8 if pv == "fp8" else O.PV_FP16, tile_k=G.TILE_K[pv], gran="head")
    ref = np.stack([np.stack([ref[(b, h)] for h in range(w.H)]) for b in range(w.B)])
    assert np.isfinite(got).all()
    G.assert_parity(got, ref, f"{w.name} causal={causal} pv={pv} head")


def test_head_qk_int32_dump_bit_exact():
    w = synth.custom(2, 4, 300, 128, Hkv=2, seed=1631)
    b, h = 1, 3
    _, _, dump = G.run(w, causal=True, dump_head=(b, h), qk_quant="int8_head")
    q, k, _ = G.inputs(w)
    dt = O.DTYPES[w.dtype]
    rq8, _ = O.quant_q_head(O.decode16(O.head(q, w.layout, b, h), dt), w.S)
    rk8, _, _ = O.quant_k_head(O.decode16(O.head(k, w.layout, b, O.kv_head(h, w.H, w.kv_heads)), dt), w.S, True)
    got = dump.cpu().numpy()
    assert np.array_equal(np.tril(got), np.tril(O.qk_int32_head(rq8, rk8)))


def test_head_full_size_sampled():
    """The headline shape with per-head scales (benchmark launch configuration)."""
    w = W["snippet_b2h32s4096d128"]
    _, out, _ = G.run(w, qk_quant="int8_head")
    got = G.out_logical(out, w)
    assert np.isfinite(got).all()
    q, k, v = G.inputs(w)
    for (b, h) in ((0, 0), (1, 31)):
        # every row of the first head, sampled rows of the others
        rows = np.arange(w.S, dtype=np.int32) if (b, h) == (0, 0) else G.sample_rows(w.S, 24, seed=b * 100 + h)
        ref = O.attn(q, k, v, O.DTYPES[w.dtype], w.layout, heads=[(b, h)], rows=rows, gran="head")[(b, h)]
        g = got[b, h, rows]
        G.assert_parity(g, ref, f"head {w.name} head {(b, h)}")


def test_head_rejects_smoothed_q():
    import quantized_attention_02_amd as qa

    w = synth.custom(1, 2, 64, 64, seed=1641)
    with pytest.raises(qa.SageError):
        G.run(w, qk_quant="int8_head", smooth_q=True)
