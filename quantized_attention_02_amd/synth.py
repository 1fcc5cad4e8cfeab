"""Seeded synthetic attention inputs (Q, K, V) -- no part of the method's arithmetic.

Both the GPU library and the CPU oracle are fed from here; this module only
draws random numbers and casts them to the 16-bit input dtype.  Shapes and
value recipes model the workloads the SageAttention pages talk about:

* the two usage snippets ("完整指南" page, section 五分钟跑通第一个加速样例:
  B=2, H=32, S=4096, D=128, fp16, HND; "Thư viện" page, section Dùng
  SageAttention trong code của bạn: B=1, H=16, S=512, D=64, fp16, HND);
* long-context LLM prefill (causal, NHD, bf16) and a video-DiT shape
  (model dim 2560 = 20 heads x 128, "Kairos" page section 四);
* K carries a per-channel bias shared by all tokens -- the outlier structure
  that K smoothing removes ("SageAttention2" page, section SageAttention2方法).

Recipe (one ``numpy.random.default_rng(seed)`` per workload, draws in this order):
  1. Q, K, V base values ~ N(0, 1), float32, logical [B, H, S, D] (K, V: [B, Hkv, S, D]);
  2. the K bias c[h, d] ~ N(0, bias_sigma^2) per K head, shared over b and s;
  3. (outlier_p > 0) Bernoulli(outlier_p) masks for Q, then K;
  4. (token_norm) per-token factors r ~ U(0.5, 2) drawn per (b, s) for Q, K, V;
  5. (v_bias_sigma > 0) a V bias c_v[h, d] ~ N(0, v_bias_sigma^2) per V head;
  6. (q_bias_sigma > 0) a Q bias c_q[h, d] ~ N(0, q_bias_sigma^2) per Q head.
Application: x *= r (token norm), K += c, V += c_v, Q += c_q, then masked
entries of Q and K *= 20.
Then cast round-to-nearest-even to fp16 (numpy) or bf16 (torch CPU) and, for
NHD, permute to [B, S, H, D].  Returned arrays are the raw uint16 codes.

Packed variable-length batches (``VarlenWorkload``): Q is the recipe above
with B = 1, S = total query tokens, NHD, seed s; K and V the same with S =
total key tokens, Hkv heads, seed s + 1; the batch axis is dropped, giving
token-major [T, H, D].  Sequence lengths come from ``mixed_lengths``: draws
log-uniform in [lo, hi] (rounded) until the total is reached, the last one cut
to fit -- a serving-style mix of short and long prompts.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str  # "fp16" | "bf16"
    layout: str  # "HND" | "NHD"
    bias_sigma: float
    outlier_p: float = 0.0
    token_norm: bool = False
    causal: tuple = (False,)
    pv_modes: tuple = ("fp8",)
    seed: int = 42
    Hkv: int = 0  # K/V heads (grouped-query attention); 0: as many as Q
    v_bias_sigma: float = 0.0  # per-channel V offset shared by all tokens (drawn after the rest)
    q_bias_sigma: float = 0.0  # per-channel Q offset shared by all tokens (drawn last)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    def ops(self, causal: bool) -> float:
        """Attention operations per call: 4*B*H*S^2*D, halved for causal."""
        n = 4.0 * self.B * self.H * self.S * self.S * self.D
        return n / 2 if causal else n

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_b1h2s256d64", 1, 2, 256, 64, "fp16", "HND", 2.0, seed=42),
        Workload("snippet_b1h16s512d64", 1, 16, 512, 64, "fp16", "HND", 2.0, causal=(False, True), seed=43),
        Workload("snippet_b2h32s4096d128", 2, 32, 4096, 128, "fp16", "HND", 3.0, outlier_p=1e-3,
                 pv_modes=("fp8", "fp16"), seed=44),
        Workload("prefill_b1h32s32768d128", 1, 32, 32768, 128, "bf16", "NHD", 3.0, causal=(True,), seed=45),
        Workload("dit_b1h20s16384d128", 1, 20, 16384, 128, "bf16", "NHD", 3.0, token_norm=True, seed=46),
        # grouped-query attention (4 query heads per K/V head), LLM prefill layout
        Workload("gqa_b1h32kv8s8192d128", 1, 32, 8192, 128, "bf16", "NHD", 3.0, causal=(True,), seed=47, Hkv=8),
    ]
}
HEADLINE = "snippet_b2h32s4096d128"


def _cast16(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def make_qkv(w: Workload, seed: int | None = None):
    """Return (q, k, v) as uint16 codes in the workload's physical layout."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.S, w.D)
    kv_shape = (w.B, w.kv_heads, w.S, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(kv_shape, dtype=np.float32)
    v = rng.standard_normal(kv_shape, dtype=np.float32)
    c = (rng.standard_normal((w.kv_heads, w.D), dtype=np.float32) * np.float32(w.bias_sigma)).astype(np.float32)
    if w.outlier_p > 0:
        mq = rng.random(shape) < w.outlier_p
        mk = rng.random(kv_shape) < w.outlier_p
    if w.token_norm:
        for x in (q, k, v):
            r = rng.uniform(0.5, 2.0, size=(w.B, w.S)).astype(np.float32)
            x *= r[:, None, :, None]
    k += c[None, :, None, :]
    if w.v_bias_sigma > 0:
        cv = (rng.standard_normal((w.kv_heads, w.D), dtype=np.float32) * np.float32(w.v_bias_sigma)).astype(np.float32)
        v += cv[None, :, None, :]
    if w.q_bias_sigma > 0:
        cq = (rng.standard_normal((w.H, w.D), dtype=np.float32) * np.float32(w.q_bias_sigma)).astype(np.float32)
        q += cq[None, :, None, :]
    if w.outlier_p > 0:
        q[mq] *= np.float32(20.0)
        k[mk] *= np.float32(20.0)
    out = []
    for x in (q, k, v):
        if w.layout == "NHD":
            x = np.ascontiguousarray(x.transpose(0, 2, 1, 3))
        out.append(_cast16(x, w.dtype))
    return tuple(out)


def custom(B, H, S, D, dtype="fp16", layout="HND", bias_sigma=2.0, outlier_p=0.0, token_norm=False, seed=0, Hkv=0,
           v_bias_sigma=0.0, q_bias_sigma=0.0):
    """An ad-hoc workload (edge shapes in tests)."""
    kv = f"kv{Hkv}" if Hkv else ""
    return Workload(f"custom_b{B}h{H}{kv}s{S}d{D}", B, H, S, D, dtype, layout, bias_sigma, outlier_p, token_norm,
                    seed=seed, Hkv=Hkv, v_bias_sigma=v_bias_sigma, q_bias_sigma=q_bias_sigma)


def mixed_lengths(total: int, lo: int, hi: int, seed: int) -> tuple:
    """Sequence lengths summing to `total`, log-uniform in [lo, hi]."""
    rng = np.random.default_rng(seed)
    out, left = [], total
    while left > 0:
        n = int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi))))))
        n = max(1, min(n, left))
        out.append(n)
        left -= n
    return tuple(out)


@dataclass(frozen=True)
class VarlenWorkload:
    name: str
    H: int
    Hkv: int
    D: int
    dtype: str
    seqlens_q: tuple
    seqlens_k: tuple
    bias_sigma: float = 3.0
    causal: tuple = (True,)
    pv_modes: tuple = ("fp8",)
    seed: int = 0
    q_bias_sigma: float = 0.0  # per-channel Q offset shared by all tokens (as Workload)

    @property
    def B(self) -> int:
        return len(self.seqlens_q)

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.seqlens_k))

    def cu_seqlens(self):
        """(cu_q, cu_k): int32 prefix sums [B + 1]."""
        cq = np.concatenate([[0], np.cumsum(self.seqlens_q)]).astype(np.int32)
        ck = np.concatenate([[0], np.cumsum(self.seqlens_k)]).astype(np.int32)
        return cq, ck

    def ops(self, causal: bool) -> float:
        """Attention operations per call: 4*H*D*sum(Sq*Sk), the causal mask keeping
        about half (sum of min(i + 1, Sk) over the query rows i)."""
        n = 0.0
        for sq, sk in zip(self.seqlens_q, self.seqlens_k):
            if causal:
                m = min(sq, sk)
                n += m * (m + 1) / 2 + (sq - m) * sk
            else:
                n += sq * sk
        return 4.0 * self.H * self.D * n


def varlen(name, H, Hkv, D, seqlens_q, seqlens_k=None, dtype="fp16", bias_sigma=2.0, causal=(False,),
           pv_modes=("fp8",), seed=0, q_bias_sigma=0.0) -> VarlenWorkload:
    return VarlenWorkload(name, H, Hkv, D, dtype, tuple(seqlens_q), tuple(seqlens_k or seqlens_q), bias_sigma,
                          causal, pv_modes, seed, q_bias_sigma)


def make_qkv_varlen(w: VarlenWorkload):
    """(q [Tq, H, D], k [Tk, Hkv, D], v [Tk, Hkv, D]) uint16 codes, token-major."""
    wq = Workload(w.name + "_q", 1, w.H, w.total_q, w.D, w.dtype, "NHD", w.bias_sigma, seed=w.seed,
                  q_bias_sigma=w.q_bias_sigma)
    wk = Workload(w.name + "_kv", 1, w.H, w.total_k, w.D, w.dtype, "NHD", w.bias_sigma, seed=w.seed + 1, Hkv=w.Hkv)
    q = make_qkv(wq)[0][0]
    _, k, v = make_qkv(wk)
    return q, k[0], v[0]


VARLEN_WORKLOADS = {
    w.name: w
    for w in [
        # LLM prefill of a batch of prompts of mixed lengths, 32768 tokens in all, GQA 32/8
        varlen("varlen_h32kv8t32768d128", 32, 8, 128, mixed_lengths(32768, 128, 8192, seed=48), dtype="bf16",
               bias_sigma=3.0, causal=(True,), pv_modes=("fp8", "fp16"), seed=48),
    ]
}
