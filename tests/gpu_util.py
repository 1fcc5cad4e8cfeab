"""Helpers for the GPU parity tests: upload the seeded host arrays, run the
library through its C ABI, and bring results back in the oracle's logical
[B, H, S, D] layout."""
from __future__ import annotations

import functools

import numpy as np

import oracle as O
import quantized_attention_02_amd as qa
from quantized_attention_02_amd import synth

# Method parameters of the attention kernel (include/sage.h): keys per online-
# softmax tile in each pv mode; the oracle is run with the same tiling.
TILE_K = {"fp8": 128, "fp16": 128}
VPOS_KEY = np.array([32 * ((p & 31) >> 4) + 8 * ((p & 15) >> 2) + 4 * (p >> 5) + (p & 3) for p in range(64)])


def torch_dtype(dt: str):
    import torch

    return {"fp16": torch.float16, "bf16": torch.bfloat16}[dt]


def to_device(u16: np.ndarray, dt: str):
    import torch

    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch_dtype(dt)).cuda()


def to_u16(t) -> np.ndarray:
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=3)
def inputs(w: synth.Workload):
    return synth.make_qkv(w)


def run(w: synth.Workload, *, causal=False, pv="fp8", sm_scale=None, dump_head=None, qk_quant="int8", smooth_v=False,
        smooth_q=False):
    """Quantise and run attention on the GPU. Returns (bufs, out tensor, dump or None)."""
    import torch

    q, k, v = inputs(w)
    qd, kd, vd = (to_device(x, w.dtype) for x in (q, k, v))
    bufs = qa.quantize(qd, kd, vd, w.layout, pv, qk_quant=qk_quant, smooth_v=smooth_v, smooth_q=smooth_q)
    out = torch.empty_like(qd)
    dump = None
    if dump_head is not None:
        dump = torch.full((w.S, w.S), -(2 ** 31), dtype=torch.int32, device="cuda")
    qa.attn_fwd(bufs, vd, out, w.layout, causal, sm_scale, pv, dump_head=dump_head, dump=dump)
    torch.cuda.synchronize()
    return bufs, out, dump


def out_logical(out, w: synth.Workload) -> np.ndarray:
    """GPU output -> fp32 numpy [B, H, S, D]."""
    x = O.decode16(to_u16(out), O.DTYPES[w.dtype])
    if w.layout == "NHD":
        x = x.transpose(0, 2, 1, 3)
    return np.ascontiguousarray(x)


def v8_logical(v_fp8, S: int) -> np.ndarray:
    """[B, H, nk, D, 64] tiled/permuted codes -> [B, H, S, D]."""
    t = v_fp8.cpu().numpy()
    B, H, nk, D, _ = t.shape
    out = np.zeros((B, H, nk * 64, D), np.uint8)
    for p in range(64):
        out[:, :, VPOS_KEY[p]::64, :][:, :, :nk, :] = t[:, :, :, :, p]
    return out[:, :, :S, :]


def sample_rows(S: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, S // 2, S - 2, S - 1]
    rows = set(r for r in fixed if 0 <= r < S)
    rows |= set(rng.integers(0, S, size=n).tolist())
    return np.array(sorted(rows), np.int32)


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def rel_l1(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(np.abs(a - b).sum() / np.abs(b).sum())


def row_cos_min(a, b):
    a = np.asarray(a, np.float64).reshape(-1, a.shape[-1])
    b = np.asarray(b, np.float64).reshape(-1, b.shape[-1])
    c = (a * b).sum(1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))
    return float(c.min())
