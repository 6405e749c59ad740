"""GPU parity of ragged batches (sas_shape.seq_lens) against the oracle: the
training chain (pooling, selection, forward, backward, selector backward) where
each sequence is the method on its own tokens, and decode / the fused step
where each sequence has its own cache length."""
import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import GATE_ATOL, max_abs, rel_l2, say, tols, worst_block_errs

pytestmark = pytest.mark.gpu
DEV = "cuda"
JUNK = 7.5   # finite padding value: must never reach a result


def ragged_inputs(seed, b, hq, hkv, n, d, bs, K, dtype, lens):
    w = synth.workload(1, batch=b, hq=hq, hkv=hkv, seqlen=n, head_dim=d, block=bs, topk=K,
                       dtype="f32" if dtype == torch.float32 else "bf16")
    x = synth.train_inputs(w, seed=seed, poison_invalid_scores=False)
    T = O.n_blocks(n, bs)
    x["s"] = synth.random_scores((b, hkv, T, T), seed=seed + 1)
    for bb, nb in enumerate(lens):
        for key in ("q", "k", "v", "dout"):
            x[key][bb, :, nb:] = JUNK
    return x


CASES = [
    # b, hq, hkv, n,   d,   bs, K, dtype,          lens
    (4, 8, 2, 640, 128, 64, 3, torch.bfloat16, [640, 200, 1, 0]),
    (3, 2, 1, 96, 64, 16, 2, torch.float32, [96, 50, 17]),
]


@pytest.mark.parametrize("standin", [True, False], ids=["standin", "given-s"])
@pytest.mark.parametrize("case", CASES, ids=[str(c[8]) for c in CASES])
def test_ragged_training(case, standin):
    from gated_block_sparse_scores_amd import ops
    b, hq, hkv, n, d, bs, K, dtype, lens = case
    say(f"ragged training {lens} standin={standin}")
    x = ragged_inputs(sum(lens) + K, b, hq, hkv, n, d, bs, K, dtype, lens)
    T = O.n_blocks(n, bs)
    xd = {k_: v_.to(DEV) for k_, v_ in x.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    if standin:
        qb = ops.block_pool(xd["q"], bs, hq // hkv, seq_lens=sl)
        kb = ops.block_pool(xd["k"], bs, 1, seq_lens=sl)
        idx, logg, lse_s, s = ops.select_topk(b, hkv, T, T, K, qbar=qb, kbar=kb, seq_lens=sl,
                                              seqlen=n, block=bs)
    else:
        idx, logg, lse_s, s = ops.select_topk(b, hkv, T, T, K, s=xd["s"], seq_lens=sl,
                                              seqlen=n, block=bs)
    o, lse = ops.attn_fwd(xd["q"], xd["k"], xd["v"], idx, logg, bs, seq_lens=sl)
    gr = ops.attn_bwd(xd["q"], xd["k"], xd["v"], o, xd["dout"], lse, idx, logg, s, lse_s, bs,
                      seq_lens=sl)
    if standin:
        dq_attn = gr["dq"].clone()
        dqb, dkb = ops.selector_bwd(gr["ds"], qb, kb, bs, n, hq, dq=gr["dq"], dk=gr["dk"],
                                    seq_lens=sl)
    torch.cuda.synchronize()
    ref = O.ragged_train(x["q"], x["k"], x["v"], x["dout"], lens, K, bs, s=x["s"].numpy(),
                         standin=standin)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    assert max_abs(logg.cpu(), ref["logg"]) <= GATE_ATOL
    np.testing.assert_allclose(lse_s.cpu().numpy(), ref["lse_s"], rtol=0, atol=GATE_ATOL)
    atol, rtol = tols(dtype)
    oc, lc = o.cpu(), lse.cpu()
    for bb, nb in enumerate(lens):
        assert torch.all(oc[bb, :, nb:] == 0) and torch.all(torch.isinf(lc[bb, :, nb:]))
        if nb:
            assert max_abs(oc[bb, :, :nb], ref["o"][bb, :, :nb]) <= atol
            assert max_abs(lc[bb, :, :nb], ref["lse"][bb, :, :nb]) <= atol
    grads = {"dk": gr["dk"], "dv": gr["dv"], "dlogg": gr["dlogg"], "ds": gr["ds"]}
    ref_dq, ref_dk = ref["dq"], ref["dk"].copy()
    if standin:
        # the selector's part, per sequence (oracle), on top of the attention's
        ref_dq = ref_dq.copy()
        for bb, nb in enumerate(lens):
            if nb == 0:
                continue
            Tb = O.n_blocks(nb, bs)
            rq, rk = O.selector_bwd(ref["ds"][bb:bb + 1, :, :Tb, :Tb],
                                    ref["qbar"][bb:bb + 1, :, :Tb], ref["kbar"][bb:bb + 1, :, :Tb],
                                    O.default_scale(d))
            ref_dq[bb, :, :nb] += O.pool_queries_bwd(rq, hq, nb, bs)[0]
            ref_dk[bb, :, :nb] += O.pool_keys_bwd(rk, nb, bs)[0]
        assert rel_l2(dq_attn.cpu(), ref["dq"]) <= rtol
    errs = {"dq": rel_l2(gr["dq"].cpu(), ref_dq), "dk": rel_l2(gr["dk"].cpu(), ref_dk)}
    errs.update({k_: rel_l2(grads[k_].cpu(), ref[k_]) for k_ in ("dv", "dlogg", "ds")})
    say("  " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= rtol, k_
    for bb, nb in enumerate(lens):
        for key in ("dq", "dk", "dv"):
            assert torch.all(gr[key][bb, :, nb:].cpu() == 0), (key, bb)


DECODE = [
    # lens,                      hq, hkv, d,   bs, K, dtype
    ([1000, 64, 3000, 4097], 8, 2, 128, 64, 8, torch.bfloat16),
    ([300, 17, 129], 4, 4, 64, 16, 4, torch.float32),
]


@pytest.mark.parametrize("case", DECODE, ids=[str(c[0]) for c in DECODE])
def test_ragged_decode_dense_cache(case):
    """sas_decode and sas_decode_step with per-sequence lengths over a dense
    cache: each sequence decodes at its own length (oracle: per sequence)."""
    from gated_block_sparse_scores_amd import ops
    lens, hq, hkv, d, bs, K, dtype = case
    b, Lmax = len(lens), max(lens)
    say(f"ragged decode {lens}")
    w = synth.workload(4, batch=b, hq=hq, hkv=hkv, seqlen=Lmax, head_dim=d, block=bs, topk=K,
                       dtype="f32" if dtype == torch.float32 else "bf16")
    x = synth.decode_inputs(w, seed=Lmax + K)
    for bb, L in enumerate(lens):
        x["kcache"][bb, :, L:] = JUNK
        x["vcache"][bb, :, L:] = JUNK
    maxC = (Lmax - 1) // bs
    kbar = torch.zeros((b, hkv, max(maxC, 1), d), dtype=torch.bfloat16)
    ridx = np.full((b, hkv, K), -1, dtype=np.int64)
    rlogg = np.zeros((b, hkv, K))
    qbar32 = O.to_f32(O.decode_qbar(x["q"], hkv))
    for bb, L in enumerate(lens):
        C = (L - 1) // bs
        if C == 0:
            continue
        kbar[bb, :, :C] = torch.from_numpy(
            O.to_f32(O.pool_keys(x["kcache"][bb:bb + 1, :, :C * bs], bs)))[0].to(torch.bfloat16)
        so = O.standin_scores(qbar32[bb:bb + 1], kbar[bb:bb + 1].float().numpy(),
                              O.default_scale(d), C, row_offset=C)
        i, lg, _ = O.select_topk(so, K, row_offset=C, C=C)
        ridx[bb], rlogg[bb] = i[0, :, 0], lg[0, :, 0]
    oo = np.zeros((b, hq, d))
    ol = np.zeros((b, hq))
    for bb, L in enumerate(lens):
        ob, lb = O.decode(x["q"][bb:bb + 1], x["kcache"][bb:bb + 1], x["vcache"][bb:bb + 1], L,
                          ridx[bb:bb + 1], rlogg[bb:bb + 1], bs)
        oo[bb], ol[bb] = ob[0], lb[0]
    xd = {k_: v_.to(DEV) for k_, v_ in x.items()}
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    atol, _ = tols(dtype)
    o, lse = ops.decode(xd["q"], xd["kcache"], xd["vcache"], Lmax,
                        torch.from_numpy(ridx.astype(np.int32)).to(DEV),
                        torch.from_numpy(rlogg.astype(np.float32)).to(DEV), bs, seq_lens=sl)
    fo, flse, fidx, flogg, _ = ops.decode_step(xd["q"], kbar.to(DEV), xd["kcache"], xd["vcache"],
                                               Lmax, K, bs, seq_lens=sl)
    torch.cuda.synchronize()
    assert max_abs(o.cpu(), oo) <= atol and max_abs(lse.cpu(), ol) <= atol
    np.testing.assert_array_equal(fidx.cpu().numpy().astype(np.int64), ridx)
    assert max_abs(flogg.cpu(), rlogg) <= GATE_ATOL
    say(f"  decode o {max_abs(o.cpu(), oo):.2e}; step o {max_abs(fo.cpu(), oo):.2e}")
    assert max_abs(fo.cpu(), oo) <= atol and max_abs(flse.cpu(), ol) <= atol


def test_full_lengths_equal_dense_bitwise():
    """A ragged batch whose lengths are all full gives bitwise the results of
    the plain batch (the ragged backward runs dQ and dK/dV one after the other,
    the plain one at this size concurrently; both use the same D)."""
    from gated_block_sparse_scores_amd import ops
    w = synth.workload(2, seqlen=2048)
    x = {k_: v_.to(DEV) for k_, v_ in synth.train_inputs(w, seed=5).items() if v_ is not None}
    T = w.nblocks
    sl = torch.full((w.batch,), w.seqlen, dtype=torch.int32, device=DEV)
    outs = []
    for lens in (None, sl):
        kw = {} if lens is None else {"seq_lens": lens, "seqlen": w.seqlen, "block": w.block}
        qb = ops.block_pool(x["q"], w.block, w.group, seq_lens=lens)
        kb = ops.block_pool(x["k"], w.block, 1, seq_lens=lens)
        idx, logg, lse_s, s = ops.select_topk(w.batch, w.hkv, T, T, w.topk, qbar=qb, kbar=kb, **kw)
        o, lse = ops.attn_fwd(x["q"], x["k"], x["v"], idx, logg, w.block, seq_lens=lens)
        gr = ops.attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg, s, lse_s, w.block,
                          seq_lens=lens)
        outs.append((o, lse, gr))
    torch.cuda.synchronize()
    (o1, l1, g1), (o2, l2, g2) = outs
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for key in ("dq", "dk", "dv", "dlogg", "ds"):
        assert torch.equal(g1[key], g2[key]), key


@pytest.mark.timeout(300)
def test_ragged_batch_of_the_benchmark():
    """The ragged training batch the benchmark times: sequences of 8192, 6177,
    3077 and 1024 tokens padded to 8192, 32/8 heads, d 128, block 64, Top-31,
    stand-in selector.  Per sequence (the oracle on that sequence's own tokens):
    its pooled scores (fp64 dot products rounded once, so equal but for an
    fp32 rounding boundary), the Top-K of the device's scores, and for two KV
    heads the o, LSE, dq, dlogg and ds of sampled query blocks (the last one
    partial) and the dk, dv of the key block with the longest inverse list;
    padding rows stay zero."""
    from gated_block_sparse_scores_amd import ops
    lens = [8192, 6177, 3077, 1024]
    w = synth.workload(2, batch=len(lens))
    x = synth.train_inputs(w, seed=77)
    for bb, nb in enumerate(lens):
        for key in ("q", "k", "v", "dout"):
            x[key][bb, :, nb:] = JUNK
    say(f"ragged batch {lens}")
    xd = {k_: x[k_].to(DEV) for k_ in ("q", "k", "v", "dout")}
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    T, bs, K, g = w.nblocks, w.block, w.topk, w.group
    qb = ops.block_pool(xd["q"], bs, g, seq_lens=sl)
    kb = ops.block_pool(xd["k"], bs, 1, seq_lens=sl)
    idx, logg, lse_s, s = ops.select_topk(w.batch, w.hkv, T, T, K, qbar=qb, kbar=kb, seq_lens=sl,
                                          seqlen=w.seqlen, block=bs)
    o, lse = ops.attn_fwd(xd["q"], xd["k"], xd["v"], idx, logg, bs, seq_lens=sl)
    gr = ops.attn_bwd(xd["q"], xd["k"], xd["v"], o, xd["dout"], lse, idx, logg, s, lse_s, bs,
                      seq_lens=sl)
    torch.cuda.synchronize()
    scale = O.default_scale(w.head_dim)
    s_c, idx_c, logg_c = s.cpu().numpy(), idx.cpu().numpy(), logg.cpu().numpy()
    o_c, lse_c, dq_c = o.cpu(), lse.cpu(), gr["dq"].cpu()
    dl_c, ds_c = gr["dlogg"].cpu().numpy(), gr["ds"].cpu().numpy()
    dk_c, dv_c = gr["dk"].cpu(), gr["dv"].cpu()
    worst = {"o": 0.0, "lse": 0.0}
    rows = {k_: [] for k_ in ("dq", "dlogg", "ds", "dk", "dv")}
    for bb, nb in enumerate(lens):
        Tb = O.n_blocks(nb, bs)
        xb = {k_: x[k_][bb:bb + 1, :, :nb] for k_ in ("q", "k", "v", "dout")}
        qo = O.to_f32(O.pool_queries(xb["q"], w.hkv, bs))
        ko = O.to_f32(O.pool_keys(xb["k"], bs))
        so = O.standin_scores(qo, ko, scale, Tb)
        valid = np.tril(np.ones((Tb, Tb), dtype=bool), -1)
        assert np.sum((s_c[bb:bb + 1, :, :Tb, :Tb] != so) & valid) <= 2, bb
        oi, ol, ols = O.select_topk(s_c[bb:bb + 1, :, :Tb, :Tb], K)
        np.testing.assert_array_equal(idx_c[bb:bb + 1, :, :Tb], oi)
        assert max_abs(logg_c[bb:bb + 1, :, :Tb], ol) <= GATE_ATOL
        assert torch.all(o_c[bb, :, nb:] == 0) and torch.all(dq_c[bb, :, nb:] == 0)
        assert torch.all(dk_c[bb, :, nb:] == 0) and torch.all(dv_c[bb, :, nb:] == 0)
        for kv in (0, w.hkv - 1):
            hs = slice(kv * g, (kv + 1) * g)
            for t in sorted({1, Tb // 2, Tb - 1}):
                lo, hi = O.block_span(t, bs, nb)
                ob, lb, _, _ = O.fwd_row_block(xb["q"], xb["k"], xb["v"], oi, ol, bs, scale, 0,
                                               kv, t)
                dqb, dlb, _ = O.bwd_row_block(xb["q"], xb["k"], xb["v"], xb["dout"], oi, ol, bs,
                                              scale, 0, kv, t)
                dsr = O.ds_row(s_c[bb, kv, t, :t], ols[0, kv, t], oi[0, kv, t], dlb)
                worst["o"] = max(worst["o"], max_abs(o_c[bb, hs, lo:hi], ob))
                worst["lse"] = max(worst["lse"], max_abs(lse_c[bb, hs, lo:hi], lb))
                rows["dq"].append((dq_c[bb, hs, lo:hi], dqb))
                rows["dlogg"].append((dl_c[bb, kv, t], dlb))
                rows["ds"].append((ds_c[bb, kv, t, :t], dsr))
            counts = np.bincount(oi[0, kv][oi[0, kv] >= 0], minlength=Tb)
            m = int(np.argmax(counts))
            dkb, dvb = O.bwd_key_block(xb["q"], xb["k"], xb["v"], xb["dout"], oi, ol, bs, scale,
                                       0, kv, m)
            lo, hi = O.block_span(m, bs, nb)
            rows["dk"].append((dk_c[bb, kv, lo:hi], dkb))
            rows["dv"].append((dv_c[bb, kv, lo:hi], dvb))
    # gradients: relative L2 per sampled block, over the larger of the block's
    # own norm and the RMS block norm (a one-block dlogg row can be a near-zero
    # sum of cancelling terms)
    worst.update(worst_block_errs(rows))
    say("  worst: " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in worst.items()))
    assert worst["o"] <= 2e-2 and worst["lse"] <= 2e-2
    for k_ in ("dq", "dlogg", "ds", "dk", "dv"):
        assert worst[k_] <= 3e-2, k_
