"""GPU V smoothing vs the oracle: V minus its channel mean is quantised to FP8
and the mean is added back to the output.

The means, codes and scales are bit-identical to the oracle's; outputs meet
the attention bars (cosine >= 0.999, mean relative L1 <= 1e-2) against the
oracle with smoothing; with per-channel V offsets the smoothed output is closer
to exact attention than the plain one.
"""
import numpy as np
import pytest

import oracle as O
from quantized_attention_02_amd import synth

import gpu_util as G

pytestmark = pytest.mark.gpu

COS_MIN, REL_L1_MAX = G.COS_MIN, G.REL_L1_MAX
W = synth.WORKLOADS

CASES = [
    synth.custom(1, 2, 256, 64, v_bias_sigma=4.0, seed=1001),
    synth.custom(1, 2, 1, 64, v_bias_sigma=4.0, seed=1002),
    synth.custom(2, 3, 100, 64, layout="NHD", v_bias_sigma=2.0, seed=1003),
    synth.custom(1, 2, 257, 128, dtype="bf16", layout="NHD", v_bias_sigma=6.0, seed=1004),
    synth.custom(2, 6, 700, 128, Hkv=2, token_norm=True, v_bias_sigma=3.0, seed=1005),
    synth.custom(1, 3, 9000, 64, v_bias_sigma=1.0, seed=1006),  # more than 32 chunks of 256 tokens
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_smooth_v_quant_bit_exact(w):
    _, _, v = G.inputs(w)
    bufs, _, _ = G.run(w, smooth_v=True)
    dt = O.DTYPES[w.dtype]
    v8 = G.v8_logical(bufs.v_fp8, w.S)
    vs, vm = bufs.v_scale.cpu().numpy(), bufs.v_mean.cpu().numpy()
    for b in range(w.B):
        for h in range(w.kv_heads):
            r8, rs, rm = O.quant_v_head(O.decode16(O.head(v, w.layout, b, h), dt), True)
            assert np.array_equal(vm[b, h].view(np.uint32), rm.view(np.uint32)), (b, h)
            assert np.array_equal(vs[b, h].view(np.uint32), rs.view(np.uint32)), (b, h)
            assert np.array_equal(v8[b, h], r8), (b, h, int((v8[b, h] != r8).sum()))


@pytest.mark.parametrize("w,causal", [(w, c) for w in CASES[:5] for c in (False, True)],
                         ids=[f"{w.name}-{c}" for w in CASES[:5] for c in (False, True)])
def test_smooth_v_attn_matches_oracle(w, causal):
    _, out, _ = G.run(w, causal=causal, smooth_v=True)
    got = G.out_logical(out, w)
    q, k, v = G.inputs(w)
    ref = O.attn(q, k, v, O.DTYPES[w.dtype], w.layout, is_causal=causal, tile_k=G.TILE_K["fp8"], smooth_v=True)
    ref = np.stack([np.stack([ref[(b, h)] for h in range(w.H)]) for b in range(w.B)])
    assert np.isfinite(got).all()
    G.assert_parity(got, ref, f"{w.name} causal={causal} smooth_v")


def test_smooth_v_with_lane_granularity_and_varlen():
    """Smoothing combines with lane scales and with packed batches."""
    import torch

    import quantized_attention_02_amd as qa

    w = synth.varlen("vl_smooth", 4, 2, 128, [300, 17, 129, 64], seed=1011)
    q, k, v = synth.make_qkv_varlen(w)
    v = O.encode16(O.decode16(v, O.F16) + np.float32(2.5), O.F16)  # a common V offset
    cq, ck = w.cu_seqlens()
    qd, kd, vd = (G.to_device(x, w.dtype) for x in (q, k, v))
    cud = [torch.from_numpy(c).cuda() for c in (cq, ck)]
    out = qa.sageattn_varlen(qd, kd, vd, cud[0], cud[1], max(w.seqlens_q), max(w.seqlens_k), is_causal=True,
                             qk_quant="int8_lane", smooth_v=True)
    torch.cuda.synchronize()
    got = O.decode16(G.to_u16(out), O.F16)
    ref = O.attn_varlen(q, k, v, cq, ck, O.F16, is_causal=True, gran="lane", smooth_v=True)
    g = np.concatenate([got[cq[b]:cq[b + 1], h] for b in range(w.B) for h in range(w.H)])
    r = np.concatenate([ref[(b, h)] for b in range(w.B) for h in range(w.H)])
    G.assert_parity(g, r, "gpu_smooth_v")


def test_smooth_v_closer_to_exact_with_v_offsets():
    w = synth.custom(1, 4, 1024, 128, v_bias_sigma=6.0, seed=1021)
    q, k, v = G.inputs(w)
    ex = O.attn_exact(q, k, v, O.DTYPES[w.dtype], w.layout)
    ex = np.stack([ex[(0, h)] for h in range(w.H)])[None]
    errs = {}
    for sv in (False, True):
        _, out, _ = G.run(w, smooth_v=sv)
        errs[sv] = G.rel_l1(G.out_logical(out, w), ex)
    print("rel L1 vs exact (smooth_v False/True):", errs)
    assert errs[True] < 0.5 * errs[False], errs


def test_smooth_v_full_size_sampled():
    """The headline shape with V smoothing in the benchmark's configuration."""
    w = W["snippet_b2h32s4096d128"]
    _, out, _ = G.run(w, smooth_v=True)
    got = G.out_logical(out, w)
    assert np.isfinite(got).all()
    q, k, v = G.inputs(w)
    for (b, h) in ((0, 0), (1, 31)):
        # every row of the first head, sampled rows of the others
        rows = np.arange(w.S, dtype=np.int32) if (b, h) == (0, 0) else G.sample_rows(w.S, 24, seed=7 + h)
        ref = O.attn(q, k, v, O.DTYPES[w.dtype], w.layout, heads=[(b, h)], rows=rows, smooth_v=True)[(b, h)]
        g = got[b, h, rows]
        G.assert_parity(g, ref, "gpu_smooth_v")
