"""GPU parity of the stand-in selector backward (C ABI sas_selector_bwd): ds to
the pooled summaries and through the mean pools into dq / dk, against the
oracle; and the whole stand-in training chain (pool, select, forward, backward,
selector backward) against the oracle's."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import rel_l2, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def selector_inputs(seed, b, hq, hkv, n, d, bs, dtype):
    gen = torch.Generator().manual_seed(seed)
    T = O.n_blocks(n, bs)
    ds = torch.randn(b, hkv, T, T, generator=gen) * 0.05
    ds[..., torch.ones(T, T, dtype=torch.bool).triu()] = float("nan")   # never read
    qbar = torch.randn(b, hkv, T, d, generator=gen) * 0.2
    kbar = torch.randn(b, hkv, T, d, generator=gen) * 0.2
    dq = torch.randn(b, hq, n, d, generator=gen).to(dtype)
    dk = torch.randn(b, hkv, n, d, generator=gen).to(dtype)
    return ds, qbar, kbar, dq, dk


CASES = [
    # b, hq, hkv, n,    d,   bs, dtype
    (1, 2, 1, 256, 64, 16, torch.float32),
    (2, 8, 2, 1000, 128, 64, torch.bfloat16),     # ragged last block
    (1, 4, 4, 17, 64, 16, torch.float32),         # T = 2, one-token tail
    (1, 32, 8, 8192, 128, 64, torch.bfloat16),    # 8K training shape (T 128)
    (1, 32, 8, 32768, 128, 64, torch.bfloat16),   # 32K training shape (T 512)
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:6]) for c in CASES])
def test_selector_bwd_vs_oracle(case):
    from gated_block_sparse_scores_amd import ops
    b, hq, hkv, n, d, bs, dtype = case
    say(f"selector_bwd {case}")
    ds, qbar, kbar, dq0, dk0 = selector_inputs(sum(case[:6]), b, hq, hkv, n, d, bs, dtype)
    dq, dk = dq0.to(DEV), dk0.to(DEV)
    dqb, dkb = ops.selector_bwd(ds.to(DEV), qbar.to(DEV), kbar.to(DEV), bs, n, hq, dq=dq, dk=dk)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    rq, rk = O.selector_bwd(ds.nan_to_num(0.0), qbar, kbar, scale)
    # fp32 accumulation over up to T terms
    eq, ek = rel_l2(dqb.cpu(), rq), rel_l2(dkb.cpu(), rk)
    say(f"  dqbar {eq:.2e} dkbar {ek:.2e}")
    assert eq <= 1e-5 and ek <= 1e-5
    # the spread: one rounding to the output dtype on top of the given values
    ref_q = O._np64(dq0) + O.pool_queries_bwd(rq, hq, n, bs)
    ref_k = O._np64(dk0) + O.pool_keys_bwd(rk, n, bs)
    ulp = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -22
    for got, ref in ((dq.cpu(), ref_q), (dk.cpu(), ref_k)):
        err = np.abs(O._np64(got) - ref)
        assert np.all(err <= ulp * np.abs(ref) + 1e-6), float(err.max())


@pytest.mark.parametrize("dtype,shape", [
    (torch.float32, (1, 2, 1, 96, 64, 16, 2)),
    (torch.bfloat16, (1, 8, 2, 640, 128, 64, 3)),
], ids=["f32", "bf16"])
def test_standin_training_chain(dtype, shape):
    """Pool q and k, stand-in scores + Top-K, forward, backward (ds), selector
    backward into dq / dk: every gradient against the oracle's chain."""
    from gated_block_sparse_scores_amd import ops
    b, hq, hkv, n, d, bs, K = shape
    w = synth.workload(2, batch=b, hq=hq, hkv=hkv, seqlen=n, head_dim=d, block=bs, topk=K,
                       dtype="f32" if dtype == torch.float32 else "bf16")
    x = synth.train_inputs(w, seed=42)
    xd = {k_: v_.to(DEV) for k_, v_ in x.items() if v_ is not None}
    T = O.n_blocks(n, bs)
    qb = ops.block_pool(xd["q"], bs, hq // hkv)
    kb = ops.block_pool(xd["k"], bs, 1)
    idx, logg, lse_s, s = ops.select_topk(b, hkv, T, T, K, qbar=qb, kbar=kb)
    o, lse = ops.attn_fwd(xd["q"], xd["k"], xd["v"], idx, logg, bs)
    gr = ops.attn_bwd(xd["q"], xd["k"], xd["v"], o, xd["dout"], lse, idx, logg, s, lse_s, bs)
    dqb, dkb = ops.selector_bwd(gr["ds"], qb, kb, bs, n, hq, dq=gr["dq"], dk=gr["dk"])
    torch.cuda.synchronize()
    # oracle chain
    qo = O.to_f32(O.pool_queries(x["q"], hkv, bs))
    ko = O.to_f32(O.pool_keys(x["k"], bs))
    so = O.standin_scores(qo, ko, O.default_scale(d), T)
    oi, ol, ols = O.select_topk(so, K)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    ref = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], oi, ol, so, ols, bs)
    rq, rk = O.selector_bwd(ref["ds"], qo, ko, O.default_scale(d))
    ref_dq = ref["dq"] + O.pool_queries_bwd(rq, hq, n, bs)
    ref_dk = ref["dk"] + O.pool_keys_bwd(rk, n, bs)
    tol = 1e-5 if dtype == torch.float32 else 3e-2
    e = {"dq": rel_l2(gr["dq"].cpu(), ref_dq), "dk": rel_l2(gr["dk"].cpu(), ref_dk),
         "dv": rel_l2(gr["dv"].cpu(), ref["dv"]), "ds": rel_l2(gr["ds"].cpu(), ref["ds"]),
         "dqbar": rel_l2(dqb.cpu(), rq), "dkbar": rel_l2(dkb.cpu(), rk)}
    say("  " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in e.items()))
    assert all(v_ <= tol for v_ in e.values()), e
    if dtype == torch.float32:
        # here the selector's share of dq is far above the tolerance, so the
        # dq check above sees it (at bf16 it is below the rounding of dq, and
        # dqbar / dkbar carry the check)
        spread = O.pool_queries_bwd(rq, hq, n, bs)
        assert np.linalg.norm(spread) > 1e-3 * np.linalg.norm(ref["dq"])
