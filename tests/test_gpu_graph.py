"""The serving and training paths captured in a HIP graph and replayed.

Every entry point launches its kernels on the caller's stream, allocates
nothing and records no memset, so a caller can capture it (torch.cuda.graph
captures on torch's current stream, which the binding passes down).  The
backward's second stream joins the capture through its fork / join events.
Each graph is replayed several times with new inputs copied into its static
input tensors, with eager work and a synchronisation between the replays, and
every replay must equal an eager call on the same inputs bit for bit (the
kernels are deterministic).  The eager decode result of the first replay's
inputs is also held to the oracle.
"""
import numpy as np
import pytest
import torch

import synth
from tests._gpu_helpers import max_abs, say, tols
from tests.test_gpu_decode_step import oracle_step, step_case

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _assert_same(a, b, what):
    assert a.shape == b.shape and a.dtype == b.dtype, what
    assert torch.equal(_bits(a), _bits(b)), what


def test_decode_step_graph_replays():
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops
    # bf16, d 128, block 64, G 4: the MFMA decode with the in-kernel candidate merge
    b, hq, hkv, Lc, d, bs, K = 2, 8, 2, 4000, 128, 64, 15
    say(f"graph: decode step b={b} hq={hq} hkv={hkv} L={Lc} K={K}")
    x, kbar = step_case(11, b, hq, hkv, Lc, d, bs, K, torch.bfloat16)
    kc, vc, kb = x["kcache"].to(DEV), x["vcache"].to(DEV), kbar.to(DEV)
    sh = ops.shape_of(x["q"].to(DEV), kc, bs, seqlen=Lc)
    ws = torch.empty(L.sas_decode_step_workspace_size(sh, K), dtype=torch.uint8, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(5)
    qs = [torch.randn((b, hq, d), generator=gen, device=DEV).to(torch.bfloat16)
          for _ in range(4)]
    q_static = qs[0].clone()

    def step(q):
        return ops.decode_step(q, kb, kc, vc, Lc, K, bs, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        step(q_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_static = step(q_static)
    for i, q in enumerate(qs):
        q_static.copy_(q)
        graph.replay()
        torch.cuda.synchronize()
        ref = step(q.clone())               # eager, between the replays
        torch.cuda.synchronize()
        for name, a, r in zip(("o", "lse", "idx", "logg", "lse_s"), out_static, ref):
            _assert_same(a, r, f"replay {i}: {name}")
        if i == 0:
            xo = dict(x, q=q.cpu())
            idx_o, logg_o, lse_s_o, o_o, lse_o = oracle_step(xo, kbar, Lc, bs, K, True)
            np.testing.assert_array_equal(ref[2].cpu().numpy(), idx_o)
            atol, _ = tols(torch.bfloat16)
            assert max_abs(ref[0].cpu(), o_o) <= atol and max_abs(ref[1].cpu(), lse_o) <= atol
    say("  4 replays equal the eager step; the first also the oracle")


def test_training_step_graph_replays():
    from gated_block_sparse_scores_amd import ops
    # bf16 MFMA kernels; the dK/dV grid is small, so dQ runs on the second stream
    b, hq, hkv, n, d, bs, K = 1, 8, 2, 1024, 128, 64, 7
    say(f"graph: training step b={b} hq={hq} hkv={hkv} n={n} K={K}")
    w = synth.workload(2, batch=b, hq=hq, hkv=hkv, seqlen=n, head_dim=d, block=bs, topk=K)
    x = synth.train_inputs(w, seed=21, device=DEV)
    T = w.nblocks
    gen = torch.Generator(device=DEV).manual_seed(9)
    douts = [torch.randn(x["dout"].shape, generator=gen, device=DEV).to(torch.bfloat16)
             for _ in range(3)]
    dout_static = douts[0].clone()

    def step(dout):
        qb = ops.block_pool(x["q"], bs, w.group)
        kb = ops.block_pool(x["k"], bs, 1)
        idx, logg, lse_s, s = ops.select_topk(b, hkv, T, T, K, qbar=qb, kbar=kb)
        o, lse = ops.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
        gr = ops.attn_bwd(x["q"], x["k"], x["v"], o, dout, lse, idx, logg, s, lse_s, bs)
        return [o, lse, gr["dq"], gr["dk"], gr["dv"], gr["dlogg"], gr["ds"]]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(dout_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_static = step(dout_static)
    names = ("o", "lse", "dq", "dk", "dv", "dlogg", "ds")
    for i, dout in enumerate(douts):
        dout_static.copy_(dout)
        graph.replay()
        torch.cuda.synchronize()
        ref = step(dout.clone())
        torch.cuda.synchronize()
        for name, a, r in zip(names, out_static, ref):
            _assert_same(a, r, f"replay {i}: {name}")
    say("  3 replays equal the eager step")
