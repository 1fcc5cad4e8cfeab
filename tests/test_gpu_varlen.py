"""GPU packed variable-length batches vs the oracle.

Quantised codes, scales and means are bit-identical to the oracle run on each
sequence alone; outputs reach the attention bars of test_gpu_attn (cosine >=
0.999, mean relative L1 <= 1e-2); each sequence's output is bit-identical to
the fixed-length path run on that sequence alone; sequences without queries or
keys are handled (zero rows for queries that see no key).
"""
import numpy as np
import pytest

import oracle as O
from quantized_attention_02_amd import synth

import gpu_util as G

pytestmark = pytest.mark.gpu

COS_MIN, REL_L1_MAX = G.COS_MIN, G.REL_L1_MAX

SMALL = [
    synth.varlen("vl_mixed_d64", 4, 2, 64, [200, 7, 64, 129, 1, 300], seed=801),
    synth.varlen("vl_bf16_d128", 6, 3, 128, [31, 33, 256, 0, 95], dtype="bf16", seed=802),
    synth.varlen("vl_cross_d128", 4, 4, 128, [40, 150, 5, 77], [150, 40, 64, 0], seed=803),
    synth.varlen("vl_single_d64", 2, 1, 64, [513], seed=804),
    # H a multiple of 8: the XCD mapping that splits every sequence's heads over the XCDs
    synth.varlen("vl_h8_d128", 8, 2, 128, [100, 380, 17, 250, 0, 129], seed=805),
]
CASES = [(w, c, pv) for w in SMALL for c in (False, True) for pv in ("fp8", "fp16")]


def _ids(cases):
    return [f"{w.name}-{'causal' if c else 'full'}-{pv}" for w, c, pv in cases]


def _inputs(w):
    import torch

    q, k, v = synth.make_qkv_varlen(w)
    cq, ck = w.cu_seqlens()
    dev = [G.to_device(x, w.dtype) for x in (q, k, v)]
    cud = [torch.from_numpy(c).cuda() for c in (cq, ck)]
    return (q, k, v, cq, ck), dev, cud


def _run(w, causal, pv, dev, cud, qk_quant="int8", smooth_q=False):
    import torch

    import quantized_attention_02_amd as qa

    qd, kd, vd = dev
    bufs = qa.quantize_varlen(qd, kd, vd, cud[0], cud[1], max(w.seqlens_q), max(max(w.seqlens_k), 1), pv,
                              qk_quant=qk_quant, smooth_q=smooth_q, is_causal=causal)
    out = torch.full_like(qd, float("nan"))
    qa.attn_fwd_varlen(bufs, vd, out, cud[0], cud[1], causal, None, pv)
    torch.cuda.synchronize()
    return bufs, out


def _v_logical(tiles, S):
    """[ntiles, D, 64] tiled codes -> [S, D]."""
    nt, D, _ = tiles.shape
    out = np.zeros((nt * 64, D), np.uint8)
    for p in range(64):
        out[G.VPOS_KEY[p]::64][:nt] = tiles[:, :, p]
    return out[:S]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_varlen_quant_bit_exact(w):
    import quantized_attention_02_amd as qa

    (q, k, v, cq, ck), dev, cud = _inputs(w)
    bufs, _ = _run(w, False, "fp8", dev, cud)
    q8, qs = bufs.q_i8.cpu().numpy(), bufs.q_scale.cpu().numpy()
    k8, ks, km = bufs.k_i8.cpu().numpy(), bufs.k_scale.cpu().numpy(), bufs.k_mean.cpu().numpy()
    v8, vs = bufs.v_fp8.cpu().numpy(), bufs.v_scale.cpu().numpy()
    dt = O.DTYPES[w.dtype]
    for b in range(w.B):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        rq, rk = qa.varlen_row0(q0, b, 32), qa.varlen_row0(k0, b, 128)
        nq, nkr = -(-(q1 - q0) // 32) * 32, -(-(k1 - k0) // 128) * 128
        for h in range(w.H):
            rq8, rqs = O.quant_q_head(O.decode16(q[q0:q1, h], dt), 32)
            assert np.array_equal(q8[h, rq:rq + q1 - q0], rq8), (b, h)
            assert not q8[h, rq + q1 - q0:rq + nq].any()
            assert np.array_equal(qs[h, rq // 32:rq // 32 + rqs.size].view(np.uint32), rqs.view(np.uint32)), (b, h)
        for h in range(w.Hkv):
            rk8, rks, rkm = O.quant_k_head(O.decode16(k[k0:k1, h], dt), 64, True)
            rv8, rvs = O.quant_v_head(O.decode16(v[k0:k1, h], dt))
            assert np.array_equal(k8[h, rk:rk + k1 - k0], rk8), (b, h)
            assert not k8[h, rk + k1 - k0:rk + nkr].any()
            assert np.array_equal(ks[h, rk // 64:rk // 64 + rks.size].view(np.uint32), rks.view(np.uint32)), (b, h)
            assert not ks[h, rk // 64 + rks.size:(rk + nkr) // 64].any()
            assert np.array_equal(km[b, h].view(np.uint32), rkm.view(np.uint32)), (b, h)
            assert np.array_equal(vs[b, h].view(np.uint32), rvs.view(np.uint32)), (b, h)
            tiles = v8[h, rk // 64:(rk + nkr) // 64]
            got = _v_logical(tiles, nkr)
            assert np.array_equal(got[:k1 - k0], rv8), (b, h)
            assert not got[k1 - k0:].any()


@pytest.mark.parametrize("w,causal,pv", CASES, ids=_ids(CASES))
def test_varlen_attn_matches_oracle(w, causal, pv):
    (q, k, v, cq, ck), dev, cud = _inputs(w)
    _, out = _run(w, causal, pv, dev, cud)
    got = O.decode16(G.to_u16(out), O.DTYPES[w.dtype])
    assert np.isfinite(got).all()  # every row of every sequence was written
    ref = O.attn_varlen(q, k, v, cq, ck, O.DTYPES[w.dtype], is_causal=causal,
                        pv_mode=O.PV_FP8 if pv == "fp8" else O.PV_FP16, tile_k=G.TILE_K[pv])
    g_all, r_all = [], []
    for b in range(w.B):
        for h in range(w.H):
            g = got[cq[b]:cq[b + 1], h]
            if ck[b + 1] == ck[b]:
                assert not g.any(), (b, h)  # no keys: zero rows
                continue
            g_all.append(g)
            r_all.append(ref[(b, h)])
    g_all, r_all = np.concatenate(g_all), np.concatenate(r_all)
    G.assert_parity(g_all, r_all, f"{w.name} causal={causal} pv={pv}")


@pytest.mark.parametrize("causal,pv", [(False, "fp8"), (True, "fp8"), (True, "fp16")])
def test_varlen_equals_fixed_length_per_sequence_bitwise(causal, pv):
    """Each sequence of a packed batch gives bit for bit what the fixed-length
    entry points give on that sequence alone (a batch of one, NHD)."""
    import torch

    import quantized_attention_02_amd as qa

    w = SMALL[0]
    (q, k, v, cq, ck), dev, cud = _inputs(w)
    _, out = _run(w, causal, pv, dev, cud)
    for b in range(w.B):
        if cq[b + 1] == cq[b]:
            continue
        qb, kb, vb = (x[None, c[b]:c[b + 1]].contiguous() for x, c in zip(dev, (cq, ck, ck)))
        ref = qa.sageattn(qb, kb, vb, tensor_layout="NHD", is_causal=causal, pv_mode=pv)
        torch.cuda.synchronize()
        assert torch.equal(out[cq[b]:cq[b + 1]].view(torch.int16), ref[0].view(torch.int16)), b


FULL = synth.VARLEN_WORKLOADS["varlen_h32kv8t32768d128"]


FULL_CASES = [(pv, False) for pv in FULL.pv_modes] + [("fp8", True)]


@pytest.mark.parametrize("pv,smooth_q", FULL_CASES, ids=[f"{pv}{'-sq' if sq else ''}" for pv, sq in FULL_CASES])
def test_varlen_full_size_sampled(pv, smooth_q):
    """The packed prefill workload in the benchmark's launch configuration:
    sampled rows of the longest, the shortest and a middle sequence (with and
    without smoothed Q)."""
    w = FULL
    (q, k, v, cq, ck), dev, cud = _inputs(w)
    causal = w.causal[0]
    _, out = _run(w, causal, pv, dev, cud, smooth_q=smooth_q)
    got = O.decode16(G.to_u16(out), O.DTYPES[w.dtype])
    assert np.isfinite(got).all()
    vmax = np.abs(O.decode16(v, O.DTYPES[w.dtype])).max()
    assert np.abs(got).max() <= vmax * (1 + 2.0 ** -4) + 1e-3
    lens = np.array(w.seqlens_q)
    seqs = sorted({int(lens.argmax()), int(lens.argmin()), w.B // 2})
    for b in seqs:
        S = int(lens[b])
        rows = G.sample_rows(S, 16, seed=b)
        for h in (0, w.H - 1, 13):
            ref = O.attn_varlen(q, k, v, cq, ck, O.DTYPES[w.dtype], is_causal=causal,
                                pv_mode=O.PV_FP8 if pv == "fp8" else O.PV_FP16, heads=[(b, h)], rows=rows,
                                tile_k=G.TILE_K[pv], smooth_q=smooth_q)[(b, h)]
            g = got[cq[b] + rows, h]
            G.assert_parity(g, ref, f"{w.name} seq {b} (S={S}) head {h}")


@pytest.mark.parametrize("w", [SMALL[2], SMALL[4]], ids=[SMALL[2].name, SMALL[4].name])
def test_varlen_lane_granularity(w):
    """Packed batches with lane granularity: codes bit-exact per sequence, output
    within the bars of the oracle at the same granularity."""
    import quantized_attention_02_amd as qa

    (q, k, v, cq, ck), dev, cud = _inputs(w)
    bufs, out = _run(w, True, "fp8", dev, cud, qk_quant="int8_lane")
    dt = O.DTYPES[w.dtype]
    qs, ks = bufs.q_scale.cpu().numpy(), bufs.k_scale.cpu().numpy()
    for b in range(w.B):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        rq, rk = qa.varlen_row0(q0, b, 32), qa.varlen_row0(k0, b, 128)
        for h in range(w.H):
            _, rqs = O.quant_q_head(O.decode16(q[q0:q1, h], dt), 1)
            assert np.array_equal(qs[h, rq:rq + q1 - q0].view(np.uint32), rqs.view(np.uint32)), (b, h)
        for h in range(w.Hkv):
            _, rks, _ = O.quant_k_head_lane(O.decode16(k[k0:k1, h], dt), True)
            assert np.array_equal(ks[h, rk // 16:rk // 16 + rks.size].view(np.uint32), rks.view(np.uint32)), (b, h)
    got = O.decode16(G.to_u16(out), dt)
    ref = O.attn_varlen(q, k, v, cq, ck, dt, is_causal=True, tile_k=G.TILE_K["fp8"], gran="lane")
    g_all, r_all = [], []
    for b in range(w.B):
        if ck[b + 1] == ck[b]:
            continue
        for h in range(w.H):
            g_all.append(got[cq[b]:cq[b + 1], h])
            r_all.append(ref[(b, h)])
    g_all, r_all = np.concatenate(g_all), np.concatenate(r_all)
    G.assert_parity(g_all, r_all, f"{w.name} lane")


@pytest.mark.parametrize("w", [SMALL[2], SMALL[4]], ids=[SMALL[2].name, SMALL[4].name])
def test_varlen_token_granularity(w):
    """Packed batches with per-token scales: scales bit-exact per sequence (one
    per Q row and per K row of the sequence's buffer rows), output within the
    bars of the oracle at the same granularity."""
    import quantized_attention_02_amd as qa

    (q, k, v, cq, ck), dev, cud = _inputs(w)
    bufs, out = _run(w, False, "fp16", dev, cud, qk_quant="int8_token")
    dt = O.DTYPES[w.dtype]
    q8, qs = bufs.q_i8.cpu().numpy(), bufs.q_scale.cpu().numpy()
    k8, ks = bufs.k_i8.cpu().numpy(), bufs.k_scale.cpu().numpy()
    for b in range(w.B):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        rq, rk = qa.varlen_row0(q0, b, 32), qa.varlen_row0(k0, b, 128)
        for h in range(w.H):
            rq8, rqs = O.quant_q_head(O.decode16(q[q0:q1, h], dt), 1)
            assert np.array_equal(q8[h, rq:rq + q1 - q0], rq8), (b, h)
            assert np.array_equal(qs[h, rq:rq + q1 - q0].view(np.uint32), rqs.view(np.uint32)), (b, h)
        for h in range(w.Hkv):
            rk8, rks, _ = O.quant_k_head(O.decode16(k[k0:k1, h], dt), 1, True)
            assert np.array_equal(k8[h, rk:rk + k1 - k0], rk8), (b, h)
            assert np.array_equal(ks[h, rk:rk + k1 - k0].view(np.uint32), rks.view(np.uint32)), (b, h)
    got = O.decode16(G.to_u16(out), dt)
    ref = O.attn_varlen(q, k, v, cq, ck, dt, is_causal=False, pv_mode=O.PV_FP16, tile_k=G.TILE_K["fp16"],
                        gran="token")
    g_all, r_all = [], []
    for b in range(w.B):
        if ck[b + 1] == ck[b]:
            continue
        for h in range(w.H):
            g_all.append(got[cq[b]:cq[b + 1], h])
            r_all.append(ref[(b, h)])
    g_all, r_all = np.concatenate(g_all), np.concatenate(r_all)
    G.assert_parity(g_all, r_all, f"{w.name} token")


@pytest.mark.parametrize("w", [SMALL[0], SMALL[2]], ids=[SMALL[0].name, SMALL[2].name])
def test_varlen_head_granularity(w):
    """Packed batches with one scale per sequence-head: codes bit-exact, every
    block slot of the sequence holding its head scale, output within the bars
    of the oracle at the same granularity."""
    import quantized_attention_02_amd as qa

    (q, k, v, cq, ck), dev, cud = _inputs(w)
    bufs, out = _run(w, True, "fp8", dev, cud, qk_quant="int8_head")
    dt = O.DTYPES[w.dtype]
    q8, qs = bufs.q_i8.cpu().numpy(), bufs.q_scale.cpu().numpy()
    k8, ks = bufs.k_i8.cpu().numpy(), bufs.k_scale.cpu().numpy()
    for b in range(w.B):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        rq, rk = qa.varlen_row0(q0, b, 32), qa.varlen_row0(k0, b, 128)
        if q1 > q0:
            for h in range(w.H):
                rq8, rqs = O.quant_q_head(O.decode16(q[q0:q1, h], dt), int(q1 - q0))
                assert np.array_equal(q8[h, rq:rq + q1 - q0], rq8), (b, h)
                sl = qs[h, rq // 32:rq // 32 + (q1 - q0 + 31) // 32]
                assert (sl.view(np.uint32) == rqs.view(np.uint32)[0]).all(), (b, h)
        if k1 > k0:
            for h in range(w.Hkv):
                rk8, rks, _ = O.quant_k_head(O.decode16(k[k0:k1, h], dt), int(k1 - k0), True)
                assert np.array_equal(k8[h, rk:rk + k1 - k0], rk8), (b, h)
                sl = ks[h, rk // 64:rk // 64 + 2 * ((k1 - k0 + 127) // 128)]
                assert (sl.view(np.uint32) == rks.view(np.uint32)[0]).all(), (b, h)
    got = O.decode16(G.to_u16(out), dt)
    ref = O.attn_varlen(q, k, v, cq, ck, dt, is_causal=True, tile_k=G.TILE_K["fp8"], gran="head")
    g_all, r_all = [], []
    for b in range(w.B):
        if ck[b + 1] == ck[b]:
            continue
        for h in range(w.H):
            g_all.append(got[cq[b]:cq[b + 1], h])
            r_all.append(ref[(b, h)])
    g_all, r_all = np.concatenate(g_all), np.concatenate(r_all)
    G.assert_parity(g_all, r_all, f"{w.name} head")


SMOOTH_Q = [
    synth.varlen("vl_sq_d64", 4, 2, 64, [200, 7, 64, 129, 1, 300], q_bias_sigma=4.0, seed=811),
    synth.varlen("vl_sq_cross_bf16_d128", 4, 4, 128, [40, 150, 5, 0, 77, 64], [150, 40, 64, 30, 0, 64],
                 dtype="bf16", q_bias_sigma=3.0, seed=812),
]
SQ_CASES = [(SMOOTH_Q[0], True, "fp8", "int8"), (SMOOTH_Q[0], False, "fp16", "int8_lane"),
            (SMOOTH_Q[0], True, "fp4", "mxfp4"), (SMOOTH_Q[1], True, "fp8", "int8"),
            (SMOOTH_Q[1], False, "fp8", "int8_token"), (SMOOTH_Q[1], True, "fp4", "int8")]
GRAN = {"int8": "block", "int8_lane": "lane", "int8_token": "token"}
PV_ORACLE = {"fp8": O.PV_FP8, "fp16": O.PV_FP16, "fp4": O.PV_FP4}


@pytest.mark.parametrize("w,causal,pv,qk", SQ_CASES,
                         ids=[f"{w.name}-{'causal' if c else 'full'}-{pv}-{qk}" for w, c, pv, qk in SQ_CASES])
def test_varlen_smooth_q(w, causal, pv, qk):
    """Smoothed Q on a packed batch: each sequence's block means (32 tokens from
    its first token) bit-identical to the oracle's, the output within the bars of
    the oracle with smoothed Q, and each sequence whose query and key counts agree
    bit-identical to the fixed-length entry points on that sequence alone."""
    import torch

    import quantized_attention_02_amd as qa

    (q, k, v, cq, ck), dev, cud = _inputs(w)
    qd, kd, vd = dev
    max_q, max_k = max(w.seqlens_q), max(max(w.seqlens_k), 1)
    bufs = qa.quantize_varlen(qd, kd, vd, cud[0], cud[1], max_q, max_k, pv, qk_quant=qk, smooth_q=True,
                              is_causal=causal)
    out = torch.full_like(qd, float("nan"))
    qa.attn_fwd_varlen(bufs, vd, out, cud[0], cud[1], causal, None, pv)
    torch.cuda.synchronize()
    dt = O.DTYPES[w.dtype]
    qm = bufs.q_mean.cpu().numpy()
    for b in range(w.B):
        q0, q1 = cq[b], cq[b + 1]
        if q1 == q0:
            continue
        r0 = qa.varlen_row0(q0, b, 32) // 32
        for h in range(w.H):
            _, _, rm = O.quant_q_head_smooth(O.decode16(q[q0:q1, h], dt), 32)
            assert np.array_equal(qm[h, r0:r0 + rm.shape[0]].view(np.uint32), rm.view(np.uint32)), (b, h)
    got = O.decode16(G.to_u16(out), dt)
    kw = dict(qk_format="fp4") if qk == "mxfp4" else dict(gran=GRAN[qk])
    ref = O.attn_varlen(q, k, v, cq, ck, dt, is_causal=causal, pv_mode=PV_ORACLE[pv], tile_k=G.TILE_K[pv],
                        smooth_q=True, **kw)
    g_all, r_all = [], []
    for b in range(w.B):
        g = got[cq[b]:cq[b + 1]]
        if ck[b + 1] == ck[b]:
            assert not g.any(), b  # no keys: zero rows
            continue
        for h in range(w.H):
            g_all.append(g[:, h])
            r_all.append(ref[(b, h)])
    G.assert_parity(np.concatenate(g_all), np.concatenate(r_all), f"{w.name} causal={causal} pv={pv} qk={qk} smooth_q")
    for b in range(w.B):
        if cq[b + 1] == cq[b] or w.seqlens_q[b] != w.seqlens_k[b]:
            continue
        qb, kb, vb = (x[None, c[b]:c[b + 1]].contiguous() for x, c in zip(dev, (cq, ck, ck)))
        one = qa.sageattn(qb, kb, vb, tensor_layout="NHD", is_causal=causal, pv_mode=pv, qk_quant=qk, smooth_q=True)
        torch.cuda.synchronize()
        assert torch.equal(out[cq[b]:cq[b + 1]].view(torch.int16), one[0].view(torch.int16)), b
