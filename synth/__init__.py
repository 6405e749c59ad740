"""Seeded synthetic inputs for gated block-sparse attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no pooling, scoring, gating, selection or attention).  Both
the HIP path's tests/benchmark and the CPU oracle's tests take their inputs from
here, so the two sides read the same bits.

Recipe (seed = workload number, draws in the fixed order q, k, v, dO, s):
  * values are drawn in fp32 from a normal distribution and, for bf16
    workloads, rounded once to bf16 (round-to-nearest-even, torch's conversion);
  * "N(0, 2)" means variance 2 (standard deviation sqrt 2); "N(0,1)/sqrt(2)"
    means standard deviation 1/sqrt(2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one synthetic workload."""
    number: int
    name: str
    mode: str            # "train" (fwd + bwd over a sequence) or "decode"
    batch: int
    hq: int
    hkv: int
    seqlen: int          # N for training, L (valid cache length incl. new token) for decode
    head_dim: int
    block: int
    topk: int            # K history blocks (budget = (K + 1) * block tokens)
    dtype: str           # "f32" or "bf16"
    scores: str          # "given" (s drawn), "standin" (pooled q . pooled k), "pooled-keys"
    qkv_std: float = 1.0
    s_std: float = math.sqrt(2.0)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def nblocks(self) -> int:
        return -(-self.seqlen // self.block)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workloads.  Shapes follow the Qwen3 attention geometries the pages
# evaluate (picx.dev summary 'Decode Efficiency' / Figure 7: batch 1 up to 512K
# context and batch 8 at 64K; evolve.pub review 'Summary': budgets 1024-4096).
WORKLOADS = {
    1: Workload(1, "tiny-fp32", "train", 1, 1, 1, 256, 64, 16, 4, "f32", "given",
                qkv_std=1.0 / math.sqrt(2.0)),
    2: Workload(2, "qwen3-4b-8k-train", "train", 1, 32, 8, 8192, 128, 64, 31, "bf16",
                "standin"),
    3: Workload(3, "qwen3-8b-32k-train", "train", 1, 32, 8, 32768, 128, 64, 15, "bf16",
                "given"),
    4: Workload(4, "batched-decode-8x64k", "decode", 8, 32, 8, 65536, 128, 64, 63, "bf16",
                "pooled-keys"),
    5: Workload(5, "qwen3-14b-512k-decode", "decode", 1, 40, 8, 524288, 128, 64, 31, "bf16",
                "pooled-keys"),
}


def workload(number: int, **overrides) -> Workload:
    w = WORKLOADS[number]
    return replace(w, **overrides) if overrides else w


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, gen, device, dtype):
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def train_inputs(w: Workload, seed: Optional[int] = None, device="cpu",
                 poison_invalid_scores: bool = True) -> dict:
    """q [b,hq,N,d], k/v [b,hkv,N,d], dout [b,hq,N,d] in the workload dtype and,
    for workloads whose scores are given, s fp32 [b,hkv,T,T].

    With ``poison_invalid_scores`` the entries of s that no row may read (history
    index m >= query block t) are set to NaN, so a reader of them is caught.
    """
    seed = w.number if seed is None else seed
    gen = _gen(seed, device)
    b, hq, hkv, n, d = w.batch, w.hq, w.hkv, w.seqlen, w.head_dim
    dt = w.torch_dtype
    out = {
        "q": _normal((b, hq, n, d), w.qkv_std, gen, device, dt),
        "k": _normal((b, hkv, n, d), w.qkv_std, gen, device, dt),
        "v": _normal((b, hkv, n, d), w.qkv_std, gen, device, dt),
        "dout": _normal((b, hq, n, d), 1.0, gen, device, dt),
        "s": None,
    }
    if w.scores == "given":
        t = w.nblocks
        s = _normal((b, hkv, t, t), w.s_std, gen, device, torch.float32)
        if poison_invalid_scores:
            upper = torch.ones(t, t, dtype=torch.bool, device=device).triu()
            s[..., upper] = float("nan")
        out["s"] = s
    return out


def decode_inputs(w: Workload, seed: Optional[int] = None, device="cpu",
                  cache_len: Optional[int] = None) -> dict:
    """q [b,hq,d]; kcache/vcache [b,hkv,cache_len,d] (cache_len >= L; the
    positions past L hold draws too, which no reader may use)."""
    seed = w.number if seed is None else seed
    gen = _gen(seed, device)
    b, hq, hkv, L, d = w.batch, w.hq, w.hkv, w.seqlen, w.head_dim
    cl = L if cache_len is None else cache_len
    dt = w.torch_dtype
    return {
        "q": _normal((b, hq, d), w.qkv_std, gen, device, dt),
        "kcache": _normal((b, hkv, cl, d), w.qkv_std, gen, device, dt),
        "vcache": _normal((b, hkv, cl, d), w.qkv_std, gen, device, dt),
    }


def random_scores(shape, seed: int, std: float = math.sqrt(2.0), device="cpu"):
    """i.i.d. N(0, std^2) fp32 selector scores of any shape."""
    gen = _gen(seed, device)
    return _normal(shape, std, gen, device, torch.float32)


def random_selection(b: int, hkv: int, T: int, K: int, seed: int) -> torch.Tensor:
    """int32 [b,hkv,T,K]: for query block t, min(K, t) distinct history blocks
    m < t drawn uniformly, in ascending order, then -1 padding (the layout of a
    Top-K selection, without the scores behind it)."""
    gen = _gen(seed, "cpu")
    out = torch.full((b, hkv, T, K), -1, dtype=torch.int32)
    for bb in range(b):
        for kv in range(hkv):
            for t in range(1, T):
                k = min(K, t)
                pick = torch.randperm(t, generator=gen)[:k].sort().values
                out[bb, kv, t, :k] = pick.to(torch.int32)
    return out


def random_log_gates(shape, seed: int) -> torch.Tensor:
    """fp32 log gates in (-4, 0]: log g of the selected blocks of any shape."""
    gen = _gen(seed, "cpu")
    return -4.0 * torch.rand(*shape, generator=gen, dtype=torch.float32)
