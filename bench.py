"""Benchmark of the quantized-attention hot path on one MI355X.

A step = one pass of the whole path over one batch of synthetic input already
resident in HBM: sage_quantize_qkv (K mean, INT8 Q/K, FP8 V; in pv fp16 mode
sage_smooth_quant_qk alone; in pv fp4 mode sage_smooth_quant_qk and
sage_quant_v_fp4; packed batches: the varlen calls) and sage_attn_fwd (INT8
QK^T, online softmax, FP8 / FP16 / MXFP4 PV), all on one stream.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--causal 0|1] [--pv fp8|fp16|fp4]

Prints one JSON line.  `value` is attention TOPS of the whole step
(4*B*H*S^2*D per step, halved when causal); the attention kernel alone is
reported in `roofline` (MFMA bound: INT8 and FP8 dense peak 5.0 POP/s), timed
with HIP events around each launch on the launch stream.  `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TOPS = 5000.0  # MI355X dense INT8 (POP/s) = dense FP8 (PFLOP/s) = 5.0 P
CPU_SAMPLE_S = 12.0  # seconds of oracle work in the CPU baseline sample
FP16_PEAK_TOPS = 2500.0  # MI355X dense FP16 (PFLOP/s) = 2.5 P
FP4_PEAK_TOPS = 10100.0  # MI355X dense FP4 / FP6 (PFLOP/s) = 10.1 P


def mfma_peak(pv, qk="int8"):
    """Peak of the attention kernel's contraction mix: half its operations are
    the Q.K^T product (INT8, or FP4 with MXFP4) and half the P.V product (FP8,
    or FP16 in pv fp16 mode), so the peak is the harmonic combination of the
    two dense peaks."""
    qk_peak = FP4_PEAK_TOPS if qk == "mxfp4" else MFMA_PEAK_TOPS
    pv_peak = {"fp8": MFMA_PEAK_TOPS, "fp16": FP16_PEAK_TOPS, "fp4": FP4_PEAK_TOPS}[pv]
    return 2.0 / (1.0 / qk_peak + 1.0 / pv_peak)
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_traffic.json")
ATTN_SRC = os.path.join(ROOT, "quantized_attention_02_amd", "csrc", "attn.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # the shader clock settles over the first ~0.1 s of back-to-back launches
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default=None)
    p.add_argument("--causal", type=int, default=None)
    p.add_argument("--pv", default="fp8", choices=["fp8", "fp16", "fp4"])
    p.add_argument("--smooth-v", action="store_true", help="V smoothing (pv fp8): quantise V minus its channel mean")
    p.add_argument("--smooth-q", action="store_true",
                   help="Q smoothing: quantise Q minus its 32-token block means")
    p.add_argument("--qk-quant", default="int8", choices=["int8", "int8_lane", "int8_token", "int8_head", "mxfp4"],
                   help="Q/K quantisation: INT8 per block, per Q token / 16-key lane group, per token or per head, or MXFP4")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=0,
                   help="heads in the CPU-oracle sample (0: as many as take about 12 s; with --oracle-timing: all)")
    p.add_argument("--oracle-timing", action="store_true",
                   help="only time the CPU oracle on the workload (all heads, or --cpu-heads of them scaled to "
                        "all) on the host cores, median of --oracle-repeats runs; no GPU use")
    p.add_argument("--oracle-repeats", type=int, default=1)
    p.add_argument("--q-pass", action="store_true",
                   help="INT8 per-block Q/K without Q smoothing: quantise Q in the Q/K pass and read its codes "
                        "(default: the attention kernel quantises Q itself, sage_attn_fwd_q16)")
    p.add_argument("--seq-sweep", action="store_true",
                   help="attention TOPS against sequence length (S = 1K .. 32K, B * S = 32K tokens, H 32, D 128, fp16, "
                        "HND, non-causal and causal, pv fp8), one JSON line; not the headline measurement")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 512 MiB device-to-device copy (calibrates the HBM byte counters)")
    return p.parse_args()


def seq_sweep():
    """Attention throughput against sequence length, in the form of the pages' kernel
    bench ("SageAttention量化加速框架完整指南", 性能调优实战: TOPS at S = 4096, 8192,
    16384 for head_dim 128): for each S, B = 32768 / S sequences of 32 heads, D = 128,
    fp16 HND inputs of the headline recipe, quantised once (sage_quantize_qkv), then
    sage_attn_fwd_q16 timed with HIP events (the mean of the timed calls after the
    warm-up calls)."""
    import numpy as np
    import torch

    import quantized_attention_02_amd as qa
    from quantized_attention_02_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    points = []
    for S in (1024, 2048, 4096, 8192, 16384, 32768):
        B = 32768 // S
        w = synth.custom(B, 32, S, 128, "fp16", "HND", bias_sigma=3.0, outlier_p=1e-3, seed=900 + S // 1024)
        q, k, v = synth.make_qkv(w)
        qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(torch.float16).to(dev) for x in (q, k, v))
        out = torch.empty_like(qd)
        for causal in (False, True):
            bufs = qa.Quantized(w.B, w.H, w.S, w.D, dev, w.kv_heads, "int8")
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            nq = 10
            for _ in range(2):  # (the first calls of a process include one-time set-up)
                qa.quantize(qd, kd, vd, w.layout, "fp8", bufs, is_causal=causal, q_in_attn=True)
            e[0].record()
            for _ in range(nq):
                qa.quantize(qd, kd, vd, w.layout, "fp8", bufs, is_causal=causal, q_in_attn=True)
            e[1].record()
            ops = w.ops(causal)
            n = max(5, min(100, int(2e13 / ops)))
            for _ in range(n):
                qa.attn_fwd(bufs, vd, out, w.layout, causal, None, "fp8", q=qd)
            e[2].record()
            for _ in range(n):
                qa.attn_fwd(bufs, vd, out, w.layout, causal, None, "fp8", q=qd)
            e[3].record()
            torch.cuda.synchronize()
            if not torch.isfinite(out.float()).all():
                raise RuntimeError(f"non-finite attention output at S={S}, causal={causal}")
            attn_us = e[2].elapsed_time(e[3]) * 1e3 / n
            quant_us = e[0].elapsed_time(e[1]) * 1e3 / nq
            points.append({"S": S, "B": B, "causal": causal, "attn_us": round(attn_us, 1),
                           "attn_tops": round(ops / attn_us / 1e6, 1),
                           "frac_of_5000": round(ops / attn_us / 1e6 / 5000.0, 4),
                           "quant_us": round(quant_us, 1),
                           "step_tops": round(ops / (attn_us + quant_us) / 1e6, 1)})
            print(f"seq sweep: S={S} causal={causal} {points[-1]['attn_tops']} TOPS", file=sys.stderr, flush=True)
        del qd, kd, vd, out
    print(json.dumps({"seq_sweep": {"H": 32, "D": 128, "tokens": 32768, "input_dtype": "fp16", "layout": "HND",
                                    "pv_mode": "fp8", "qk_quant": "int8", "q_quantised_in": "attention",
                                    "points": points}}))


def copy_calibration():
    """A plain copy of known size: 512 MiB read + 512 MiB written per launch."""
    import torch

    n = 512 * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}))


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_record(kernel_hash, workload, pv, causal, qk="int8", smooth_v=False, smooth_q=False, q_in_attn=False):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summaries, if one was taken on the current kernel source for this workload
    and mode."""
    try:
        recs = json.load(open(TRAFFIC_FILE))["records"]
    except (OSError, ValueError, KeyError, TypeError):
        return None
    for rec in recs:
        if (rec.get("attn_src_sha256_16") == kernel_hash and rec.get("workload") == workload
                and rec.get("pv_mode") == pv and rec.get("causal") == causal and rec.get("qk_quant", "int8") == qk
                and rec.get("smooth_v", False) == smooth_v and rec.get("smooth_q", False) == smooth_q
                and rec.get("q_in_attn", False) == q_in_attn):
            return rec
    return None


def oracle_qk(qk):
    """The oracle's keyword arguments for a Q/K quantisation mode."""
    return {"int8": {}, "int8_lane": {"gran": "lane"}, "int8_token": {"gran": "token"}, "int8_head": {"gran": "head"}, "mxfp4": {"qk_format": "fp4"}}[qk]


def cpu_model():
    """The host CPU's model name and logical core count."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(w, causal, pv, nheads, qk="int8", smooth_v=False, smooth_q=False, repeats=1, all_heads_ok=False):
    """The CPU oracle (quantisation + attention, every query row) timed on a
    sample of the workload's heads: nheads of them (0: as many as take about
    CPU_SAMPLE_S seconds, or all of them with all_heads_ok), median of `repeats`
    runs, scaled to TOPS."""
    import numpy as np

    import oracle as O
    from quantized_attention_02_amd import synth

    pvm = {"fp8": O.PV_FP8, "fp16": O.PV_FP16, "fp4": O.PV_FP4}[pv]
    if isinstance(w, synth.VarlenWorkload):
        q, k, v = synth.make_qkv_varlen(w)
        cq, ck = w.cu_seqlens()
        # sequences in a seeded random order, so that the sample mixes lengths
        order = np.random.default_rng(0).permutation(w.B)
        all_heads = [(int(b), h) for b in order for h in range(w.H)]

        def head_ops(b, h):
            one = synth.varlen("x", 1, 1, w.D, [w.seqlens_q[b]], [w.seqlens_k[b]])
            return one.ops(causal)

        def run(heads):
            t0 = time.perf_counter()
            O.attn_varlen(q, k, v, cq, ck, O.DTYPES[w.dtype], is_causal=bool(causal), pv_mode=pvm, heads=heads,
                          smooth_v=smooth_v, smooth_q=smooth_q, **oracle_qk(qk))
            return time.perf_counter() - t0
        what = "sequence-heads"
    else:
        q, k, v = synth.make_qkv(w)
        all_heads = [(b, h) for b in range(w.B) for h in range(w.H)]

        def head_ops(b, h):
            return 4.0 * w.S * w.S * w.D / (2 if causal else 1)

        def run(heads):
            t0 = time.perf_counter()
            O.attn(q, k, v, O.DTYPES[w.dtype], w.layout, is_causal=bool(causal), pv_mode=pvm, heads=heads,
                   smooth_v=smooth_v, smooth_q=smooth_q, **oracle_qk(qk))
            return time.perf_counter() - t0
        what = "heads"

    if nheads <= 0 and all_heads_ok:
        nheads = len(all_heads)
    if nheads <= 0:  # size the sample to about CPU_SAMPLE_S seconds from a one-head probe
        t1 = run(all_heads[-1:])
        per_op = t1 / head_ops(*all_heads[-1])
        nheads, acc = 0, 0.0
        for hd in all_heads:
            if nheads and acc + head_ops(*hd) * per_op > CPU_SAMPLE_S:
                break
            acc += head_ops(*hd) * per_op
            nheads += 1
    heads = all_heads[:min(nheads, len(all_heads))]

    def run_chunked(heads):
        # long samples run in chunks of about 30 s of work, reporting progress
        # on stderr; the chunk times add up to the sample's time
        per = max(1, int(30.0 / max(per_head_s, 1e-9)))
        total = 0.0
        for i in range(0, len(heads), per):
            total += run(heads[i:i + per])
            if len(heads) > per:
                print(f"oracle: {min(i + per, len(heads))}/{len(heads)} {what}, {total:.1f} s", file=sys.stderr,
                      flush=True)
        return total

    per_head_s = run(heads[:1]) if len(heads) > 1 else 0.0
    times = sorted(run_chunked(heads) for _ in range(max(1, repeats)))
    dt = times[len(times) // 2]
    ops = sum(head_ops(*hd) for hd in heads)
    model, ncpu = cpu_model()
    scale = sum(head_ops(*hd) for hd in all_heads) / ops
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": O.num_threads(), "kind": "oracle",
            "cpu": model, "host_logical_cpus": ncpu,
            "sample": f"{len(heads)} of {len(all_heads)} {what} of {w.name}, all query rows "
                      f"(quantisation of Q/K/V + attention), {dt:.2f} s wall"
                      + (f" (median of {len(times)}: {', '.join(f'{t:.2f}' for t in times)})" if len(times) > 1 else ""),
            "seconds": round(dt, 3), "whole_workload_seconds": round(dt * scale, 2),
            "whole_workload_scaled": len(heads) < len(all_heads)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the path has no multi-GPU part (one process drives one GPU)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.seq_sweep:
        seq_sweep()
        return
    if args.oracle_timing:
        from quantized_attention_02_amd import synth

        name = args.workload or synth.HEADLINE
        w = synth.VARLEN_WORKLOADS[name] if name in synth.VARLEN_WORKLOADS else synth.WORKLOADS[name]
        causal = w.causal[0] if args.causal is None else bool(args.causal)
        print(json.dumps({"oracle_timing": {"workload": name, "causal": causal, "pv_mode": args.pv,
                                            "ops": w.ops(causal),
                                            **cpu_baseline(w, causal, args.pv, args.cpu_heads, args.qk_quant,
                                                           args.smooth_v, args.smooth_q, args.oracle_repeats,
                                                           all_heads_ok=True)}}))
        return

    import numpy as np
    import torch

    import quantized_attention_02_amd as qa
    from quantized_attention_02_amd import synth

    name = args.workload or synth.HEADLINE
    varlen = name in synth.VARLEN_WORKLOADS
    if args.smooth_v and args.pv == "fp16":
        sys.exit("--smooth-v applies to pv fp8 and fp4")
    w = synth.VARLEN_WORKLOADS[name] if varlen else synth.WORKLOADS[name]
    causal = w.causal[0] if args.causal is None else bool(args.causal)
    ops = w.ops(causal)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = synth.make_qkv_varlen(w) if varlen else synth.make_qkv(w)
    tdt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev) for x in (q, k, v))
    out = torch.empty_like(qd)
    # INT8 per-block Q/K, unsmoothed Q: the attention kernel quantises Q itself
    q_in_attn = args.qk_quant == "int8" and not args.smooth_q and not args.q_pass
    if varlen:
        cq, ck = (torch.from_numpy(c).to(dev) for c in w.cu_seqlens())
        mq, mk = max(w.seqlens_q), max(w.seqlens_k)
        bufs = qa.QuantizedVarlen(w.B, w.H, w.Hkv, w.total_q, w.total_k, w.D, dev, args.qk_quant)

        def quant(cz):
            qa.quantize_varlen(qd, kd, vd, cq, ck, mq, mk, args.pv, bufs, qk_quant=args.qk_quant, smooth_v=args.smooth_v,
                               smooth_q=args.smooth_q, is_causal=bool(cz), q_in_attn=q_in_attn)

        def attn(cz):
            qa.attn_fwd_varlen(bufs, vd, out, cq, ck, cz, None, args.pv, q=qd)
    else:
        bufs = qa.Quantized(w.B, w.H, w.S, w.D, dev, w.kv_heads, args.qk_quant)

        def quant(cz):
            qa.quantize(qd, kd, vd, w.layout, args.pv, bufs, qk_quant=args.qk_quant, smooth_v=args.smooth_v,
                        smooth_q=args.smooth_q, is_causal=bool(cz), q_in_attn=q_in_attn)

        def attn(cz):
            qa.attn_fwd(bufs, vd, out, w.layout, cz, None, args.pv, q=qd)

    def run_steps(cz):
        """W untimed steps, then K timed steps between device synchronisations;
        returns (ms per step by the host clock, mean attention ms, mean
        quantisation ms by HIP events on the launch stream)."""
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

        def step(e=None):
            if e is not None:
                e[0].record()
            quant(cz)
            if e is not None:
                e[1].record()
            attn(cz)
            if e is not None:
                e[2].record()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(ev[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if not torch.isfinite(out.float()).all():
            raise RuntimeError("non-finite attention output")
        return ((t1 - t0) * 1e3 / args.steps, float(np.mean([e[1].elapsed_time(e[2]) for e in ev])),
                float(np.mean([e[0].elapsed_time(e[1]) for e in ev])))

    ms_step, attn_ms, quant_ms = run_steps(causal)
    attn_tops = ops / (attn_ms * 1e-3) / 1e12
    # the metric names the causal form of the same shape too: measured after the
    # headline steps, reported beside them (not part of `value`)
    companion = None
    if not causal and not varlen and args.pv == "fp8" and args.qk_quant == "int8" and not args.smooth_q:
        c_step, c_attn, c_quant = run_steps(True)
        c_ops = w.ops(True)
        companion = {"causal": True, "ms_per_step": round(c_step, 4), "value": round(c_ops / (c_step * 1e-3) / 1e12, 2),
                     "kernels_ms": {"quant_qk_plus_quant_v": round(c_quant, 4), "attn_fwd": round(c_attn, 4)},
                     "attn_fwd_tops": round(c_ops / (c_attn * 1e-3) / 1e12, 2),
                     "frac": round(c_ops / (c_attn * 1e-3) / 1e12 / mfma_peak(args.pv, args.qk_quant), 4)}
    khash = source_hash(ATTN_SRC)
    trec = traffic_record(khash, name, args.pv, bool(causal), args.qk_quant, args.smooth_v, args.smooth_q, q_in_attn)
    traffic = None if trec is None else trec["hbm_bytes_per_launch"]

    res = {
        "metric": "attention TOPS (4*B*H*S^2*D per step, halved if causal): smooth+quantise Q/K, quantise V, "
                  "fused INT8-QK/FP8-PV attention",
        "value": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8": "i8", "int8_lane": "i8", "int8_token": "i8", "int8_head": "i8", "mxfp4": "mxfp4"}[args.qk_quant] + {"fp8": "+fp8", "fp16": "+f16", "fp4": "+mxfp4"}[args.pv],
        "data": "synthetic",
        "config": ({"workload": name, "B": w.B, "H": w.H, "H_kv": w.Hkv, "total_q": w.total_q,
                    "total_k": w.total_k, "max_seqlen": max(w.seqlens_q), "D": w.D, "input_dtype": w.dtype,
                    "layout": "packed [T, H, D]", "causal": causal, "pv_mode": args.pv,
                    "qk_quant": args.qk_quant, "smooth_v": args.smooth_v, "smooth_q": args.smooth_q,
                    "q_quantised_in": "attention" if q_in_attn else "q/k pass"} if varlen else
                   {"workload": name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "S": w.S, "D": w.D,
                    "input_dtype": w.dtype, "layout": w.layout, "causal": causal, "pv_mode": args.pv,
                    "qk_quant": args.qk_quant, "smooth_v": args.smooth_v, "smooth_q": args.smooth_q,
                    "q_quantised_in": "attention" if q_in_attn else "q/k pass"}),
        "kernels_ms": {"quant_qk_plus_quant_v": round(quant_ms, 4), "attn_fwd": round(attn_ms, 4)},
        "attn_fwd_tops": round(attn_tops, 2),
        "roofline": {"bound": "mfma", "achieved": round(attn_tops, 2), "peak": round(mfma_peak(args.pv, args.qk_quant), 1), "unit": "TFLOP/s",
                     "frac": round(attn_tops / mfma_peak(args.pv, args.qk_quant), 4), "traffic": traffic,
                     "kernel": "k_attn (sage_attn_fwd)", "algorithmic_ops_per_launch": ops,
                     "limiter": "VALU issue of the fp32 online softmax (per score: int->fp32 convert, FMA, exp2, "
                                "half an FP8 pack; 64-multiply O rescale on most tiles; the row sum runs on the "
                                "matrix core), not the MFMAs",
                     "attn_src_sha256_16": khash},
    }
    if companion is not None:
        res["causal_companion"] = companion
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, causal, args.pv, args.cpu_heads, args.qk_quant, args.smooth_v,
                                           args.smooth_q)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
