"""Shared helpers of the GPU parity tests: tolerances, comparisons, runners.

Tolerances (max-abs for o / LSE, relative L2 for gradients) are the required
agreement for this method: Top-K indices bit-exact; o and LSE within 1e-5
(fp32 tensors) or 2e-2 (bf16 tensors, fp32 accumulation); dq/dk/dv/ds within
3e-2 relative L2 for bf16 and 1e-5 for fp32.  Gate values (logg, lse_s) are
fp32 on both sides of the comparison and are held to 1e-5.
"""
import sys

import numpy as np
import torch

from oracle import sas_oracle as O

ATOL_F32 = 1e-5
ATOL_BF16 = 2e-2
REL_F32 = 1e-5
REL_BF16 = 3e-2
GATE_ATOL = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t):
    return O._np64(t)


def _arr(x):
    return np64(x) if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)


def rel_l2(a, b):
    a, b = _arr(a), _arr(b)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


def max_abs(a, b):
    a, b = _arr(a), _arr(b)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def block_err(got, ref, rms):
    """L2 error of one sampled block over the larger of its own norm and the
    RMS norm of that quantity's sampled blocks: a dlogg row (or ds row) can be
    a near-zero sum of cancelling terms, whose own norm says nothing about the
    size of the rounding it carries."""
    got, ref = _arr(got), _arr(ref)
    return float(np.sqrt(np.sum((got - ref) ** 2)) / max(np.sqrt(np.sum(ref ** 2)), rms))


def worst_block_errs(rows):
    """{name: [(got, ref), ...]} -> {name: largest block_err over its blocks}."""
    out = {}
    for name, pairs in rows.items():
        rms = float(np.sqrt(sum(float(np.sum(_arr(r_) ** 2)) for _, r_ in pairs) / len(pairs)))
        out[name] = max(block_err(got, ref, rms) for got, ref in pairs)
    return out


def tols(dtype):
    return (ATOL_F32, REL_F32) if dtype == torch.float32 else (ATOL_BF16, REL_BF16)


def gpu_select_given(s_gpu, K, row_offset=0, C=None):
    from gated_block_sparse_scores_amd import ops
    b, hkv, T, Cs = s_gpu.shape
    C = Cs if C is None else C
    idx, logg, lse_s, _ = ops.select_topk(b, hkv, T, C, K, row_offset=row_offset, s=s_gpu)
    return idx, logg, lse_s
