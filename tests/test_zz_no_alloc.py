"""GPU check of sas_decode_step_noalloc (the decode step with no workspace
argument, for callers that cannot allocate): through the C ABI, two calls in a
row, the second with a smaller input, each equal to sas_decode_step with an
allocated workspace (same kernels and the same reductions, so bitwise), and the
first also within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import GATE_ATOL, max_abs, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed, b, hq, hkv, L, K):
    w = synth.workload(4, batch=b, hq=hq, hkv=hkv, seqlen=L, head_dim=128, block=64, topk=K)
    x = synth.decode_inputs(w, seed=seed)
    C = (L - 1) // 64
    kbar = torch.from_numpy(O.to_f32(O.pool_keys(x["kcache"][:, :, :C * 64], 64))).to(
        torch.bfloat16)
    return x, kbar


def _outputs(q, kcache):
    b, hq, _ = q.shape
    hkv = kcache.shape[1]
    return (torch.empty_like(q), torch.empty((b, hq), dtype=torch.float32, device=DEV))


def _run(x, kbar, L, K, noalloc):
    from gated_block_sparse_scores_amd import _lib as Lb
    from gated_block_sparse_scores_amd import ops
    q, kc, vc = (x[k].to(DEV) for k in ("q", "kcache", "vcache"))
    kb = kbar.to(DEV)
    b, hkv = kc.shape[:2]
    sh = ops.shape_of(q, kc, 64, seqlen=L)
    o, lse = _outputs(q, kc)
    idx = torch.empty((b, hkv, K), dtype=torch.int32, device=DEV)
    logg = torch.empty((b, hkv, K), dtype=torch.float32, device=DEV)
    lse_s = torch.empty((b, hkv), dtype=torch.float32, device=DEV)
    if noalloc:
        Lb.sas_decode_step_noalloc(sh, kc.shape[2], K, q, kb, Lb.SAS_DTYPE_BF16, kb.shape[2], kc,
                                   vc, True, o, lse, idx, logg, lse_s)
    else:
        n = Lb.sas_decode_step_workspace_size(sh, K)
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)
        Lb.sas_decode_step(sh, kc.shape[2], K, q, kb, Lb.SAS_DTYPE_BF16, kb.shape[2], kc, vc,
                           True, o, lse, idx, logg, lse_s, ws, n)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "idx": idx, "logg": logg, "lse_s": lse_s}


def test_noalloc_step_equals_allocated_step_twice():
    from gated_block_sparse_scores_amd import _lib as Lb
    cases = [(5, 4, 32, 8, 64 * 600 + 37, 31),   # larger first
             (6, 2, 16, 4, 64 * 90 + 1, 16)]     # then a smaller input
    for seed, b, hq, hkv, L, K in cases:
        say(f"decode_step_noalloc b={b} hq={hq} hkv={hkv} L={L} K={K}")
        sh = Lb.Shape(b, hq, hkv, L, 128, 64, Lb.SAS_DTYPE_BF16)
        assert Lb.sas_decode_step_workspace_size(sh, K) <= Lb.SAS_STATIC_SCRATCH_BYTES
        x, kbar = _case(seed, b, hq, hkv, L, K)
        a = _run(x, kbar, L, K, noalloc=True)
        r = _run(x, kbar, L, K, noalloc=False)
        for key in a:
            assert torch.equal(a[key], r[key]), key
        if seed == 5:   # and the result itself, against the oracle
            C = (L - 1) // 64
            qb = O.to_f32(O.decode_qbar(x["q"], hkv))
            s = O.standin_scores(qb, kbar.float().numpy(), O.default_scale(128), C, row_offset=C)
            oi, ol, ols = O.select_topk(s, K, row_offset=C, C=C)
            np.testing.assert_array_equal(a["idx"].cpu().numpy(), oi[:, :, 0])
            assert max_abs(a["logg"].cpu(), ol[:, :, 0]) <= GATE_ATOL
            oo, olse = O.decode(x["q"], x["kcache"], x["vcache"], L, oi[:, :, 0], ol[:, :, 0], 64)
            assert max_abs(a["o"].cpu(), oo) <= 2e-2 and max_abs(a["lse"].cpu(), olse) <= 2e-2


def test_noalloc_step_at_the_batched_decode_size():
    """Batch 8 x 64K tokens, 32 / 8 heads, K 63 (the batched-decode workload,
    4.4 MB of the 16 MiB scratch): the no-alloc step equals the allocated one
    bitwise.  Library against library, so the caches and the pooled-key cache
    are drawn on the device."""
    from gated_block_sparse_scores_amd import _lib as Lb
    b, hq, hkv, L, K = 8, 32, 8, 65536, 63
    say(f"decode_step_noalloc b={b} hq={hq} hkv={hkv} L={L} K={K}")
    sh = Lb.Shape(b, hq, hkv, L, 128, 64, Lb.SAS_DTYPE_BF16)
    assert Lb.sas_decode_step_workspace_size(sh, K) <= Lb.SAS_STATIC_SCRATCH_BYTES
    w = synth.workload(4, batch=b, hq=hq, hkv=hkv, seqlen=L, head_dim=128, block=64, topk=K)
    x = synth.decode_inputs(w, seed=9, device=DEV)
    C = (L - 1) // 64
    kbar = synth.random_scores((b, hkv, C, 128), seed=10, std=0.1, device=DEV).to(torch.bfloat16)
    a = _run(x, kbar, L, K, noalloc=True)
    r = _run(x, kbar, L, K, noalloc=False)
    for key in a:
        assert torch.equal(a[key], r[key]), key
    del x
    torch.cuda.empty_cache()
