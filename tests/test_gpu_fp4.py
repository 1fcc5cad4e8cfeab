"""GPU MXFP4 Q K^T (FP4 micro-scaled) vs the oracle.

E2M1 codes (unpacked from the nibble pairs) and E8M0 scale bytes are
bit-identical to the oracle's; outputs meet the attention bars (cosine >=
0.999, mean relative L1 <= 1e-2) against the oracle run with the FP4 product;
and, as the oracle's own pin states, the FP4 output stays within cos >= 0.98 of
exact attention on N(0, 1) inputs.
"""
import numpy as np
import pytest

import oracle as O
from quantized_attention_02_amd import synth

import gpu_util as G

pytestmark = pytest.mark.gpu

COS_MIN, REL_L1_MAX = G.COS_MIN, G.REL_L1_MAX
W = synth.WORKLOADS


def unpack(packed: np.ndarray) -> np.ndarray:
    """[..., D/2] bytes -> [..., D] E2M1 codes (channel 2j in the low nibble of byte j)."""
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


QUANT_CASES = [
    W["tiny_b1h2s256d64"],
    synth.custom(1, 2, 1, 64, seed=1101),
    synth.custom(2, 3, 100, 128, layout="NHD", seed=1102),
    synth.custom(1, 2, 257, 128, dtype="bf16", layout="NHD", outlier_p=0.01, seed=1103),
    synth.custom(2, 6, 300, 64, Hkv=2, token_norm=True, seed=1104),
]


@pytest.mark.parametrize("w", QUANT_CASES, ids=[w.name for w in QUANT_CASES])
def test_fp4_quant_bit_exact(w):
    q, k, _ = G.inputs(w)
    bufs, _, _ = G.run(w, qk_quant="mxfp4")
    dt = O.DTYPES[w.dtype]
    q4, qe = unpack(bufs.q_i8.cpu().numpy()), bufs.q_scale.cpu().numpy()
    k4, ke, km = unpack(bufs.k_i8.cpu().numpy()), bufs.k_scale.cpu().numpy(), bufs.k_mean.cpu().numpy()
    S = w.S
    for b in range(w.B):
        for h in range(w.H):
            r4, re = O.quant_mxfp4_rows(O.decode16(O.head(q, w.layout, b, h), dt))
            assert np.array_equal(q4[b, h, :S], r4), (b, h, int((q4[b, h, :S] != r4).sum()))
            assert np.array_equal(qe[b, h, :S], re), (b, h)
            assert not q4[b, h, S:].any() and not qe[b, h, S:].any()
        for h in range(w.kv_heads):
            r4, re, rm = O.quant_k_head_mxfp4(O.decode16(O.head(k, w.layout, b, h), dt), True)
            assert np.array_equal(km[b, h].view(np.uint32), rm.view(np.uint32)), (b, h)
            assert np.array_equal(k4[b, h, :S], r4), (b, h, int((k4[b, h, :S] != r4).sum()))
            assert np.array_equal(ke[b, h, :S], re), (b, h)
            assert not k4[b, h, S:].any() and not ke[b, h, S:].any()


ATTN_CASES = [
    (W["tiny_b1h2s256d64"], False, "fp8"),
    (W["snippet_b1h16s512d64"], True, "fp8"),
    (W["snippet_b1h16s512d64"], False, "fp16"),
    (synth.custom(1, 2, 1, 64, seed=1111), False, "fp8"),
    (synth.custom(1, 1, 31, 128, dtype="bf16", seed=1112), True, "fp16"),
    (synth.custom(2, 3, 100, 128, layout="NHD", seed=1113), True, "fp8"),
    (synth.custom(1, 2, 257, 128, dtype="bf16", layout="NHD", seed=1114), False, "fp8"),
    (synth.custom(2, 6, 300, 128, Hkv=2, seed=1115), True, "fp8"),
    (synth.custom(1, 3, 1000, 128, seed=1116), False, "fp16"),
]


def _ids(cases):
    return [f"{w.name}-{'causal' if c else 'full'}-{pv}" for w, c, pv in cases]


@pytest.mark.parametrize("w,causal,pv", ATTN_CASES, ids=_ids(ATTN_CASES))
def test_fp4_attn_matches_oracle(w, causal, pv):
    _, out, _ = G.run(w, causal=causal, pv=pv, qk_quant="mxfp4")
    got = G.out_logical(out, w)
    q, k, v = G.inputs(w)
    ref = O.attn(q, k, v, O.DTYPES[w.dtype], w.layout, is_causal=causal,
                 pv_mode=O.PV_FP8 if pv == "fp8" else O.PV_FP16, tile_k=G.TILE_K[pv], qk_format="fp4")
    ref = np.stack([np.stack([ref[(b, h)] for h in range(w.H)]) for b in range(w.B)])
    assert np.isfinite(got).all()
    G.assert_parity(got, ref, f"{w.name} causal={causal} pv={pv} mxfp4")


def test_fp4_full_size_sampled():
    """The headline shape with the FP4 product in the benchmark's launch configuration."""
    w = W["snippet_b2h32s4096d128"]
    _, out, _ = G.run(w, qk_quant="mxfp4")
    got = G.out_logical(out, w)
    assert np.isfinite(got).all()
    q, k, v = G.inputs(w)
    for (b, h) in ((0, 0), (1, 31), (1, 10)):
        # every row of the first head, sampled rows of the others
        rows = np.arange(w.S, dtype=np.int32) if (b, h) == (0, 0) else G.sample_rows(w.S, 24, seed=b * 100 + h)
        ref = O.attn(q, k, v, O.DTYPES[w.dtype], w.layout, heads=[(b, h)], rows=rows, qk_format="fp4")[(b, h)]
        g = got[b, h, rows]
        G.assert_parity(g, ref, f"mxfp4 {w.name} head {(b, h)}")


def test_fp4_tracks_exact_attention():
    w = synth.custom(1, 4, 512, 128, seed=1121)
    q, k, v = G.inputs(w)
    ex = O.attn_exact(q, k, v, O.DTYPES[w.dtype], w.layout)
    ex = np.stack([ex[(0, h)] for h in range(w.H)])[None]
    _, out, _ = G.run(w, qk_quant="mxfp4")
    c = G.cos(G.out_logical(out, w), ex)
    print("mxfp4 vs exact attention: cos", c)
    assert c >= 0.98, c


def test_fp4_varlen():
    import torch

    import quantized_attention_02_amd as qa

    w = synth.varlen("vl_fp4", 8, 2, 128, [300, 17, 129, 0, 64], seed=1131)
    q, k, v = synth.make_qkv_varlen(w)
    cq, ck = w.cu_seqlens()
    qd, kd, vd = (G.to_device(x, w.dtype) for x in (q, k, v))
    cud = [torch.from_numpy(c).cuda() for c in (cq, ck)]
    out = qa.sageattn_varlen(qd, kd, vd, cud[0], cud[1], max(w.seqlens_q), max(w.seqlens_k), is_causal=True,
                             qk_quant="mxfp4")
    torch.cuda.synchronize()
    got = O.decode16(G.to_u16(out), O.F16)
    ref = O.attn_varlen(q, k, v, cq, ck, O.F16, is_causal=True, qk_format="fp4")
    g = np.concatenate([got[cq[b]:cq[b + 1], h] for b in range(w.B) for h in range(w.H)])
    r = np.concatenate([ref[(b, h)] for b in range(w.B) for h in range(w.H)])
    G.assert_parity(g, r, "gpu_fp4")
