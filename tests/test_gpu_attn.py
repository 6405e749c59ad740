"""GPU parity of the fused gated block-sparse forward and backward (C ABI)."""
import math
import time

import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import (GATE_ATOL, max_abs, np64, rel_l2, say, tols)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_gpu(x, K, bs, gated=True, s_for_ds=True):
    """Select (given s) + forward + backward on the device."""
    from gated_block_sparse_scores_amd import ops
    g = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    b, hkv = g["k"].shape[:2]
    T = g["s"].shape[2]
    idx, logg, lse_s, _ = ops.select_topk(b, hkv, T, T, K, s=g["s"])
    lg = logg if gated else None
    o, lse = ops.attn_fwd(g["q"], g["k"], g["v"], idx, lg, bs)
    gr = ops.attn_bwd(g["q"], g["k"], g["v"], o, g["dout"], lse, idx, lg,
                      g["s"] if gated else None, lse_s if gated else None, bs,
                      want_ds=gated and s_for_ds)
    torch.cuda.synchronize()
    return dict(idx=idx, logg=logg, lse_s=lse_s, o=o, lse=lse, **gr)


def small_inputs(seed, b, hq, hkv, n, d, bs, K, dtype, std=1.0):
    w = synth.workload(1, batch=b, hq=hq, hkv=hkv, seqlen=n, head_dim=d, block=bs, topk=K,
                       dtype="f32" if dtype == torch.float32 else "bf16", qkv_std=std)
    x = synth.train_inputs(w, seed=seed, poison_invalid_scores=False)
    T = O.n_blocks(n, bs)
    s = synth.random_scores((b, hkv, T, T), seed=seed + 7)
    s[..., torch.ones(T, T, dtype=torch.bool).triu()] = float("nan")
    x["s"] = s
    return x


def compare_full(x, r, K, bs, dtype, gated=True):
    atol, rtol = tols(dtype)
    idx_o, logg_o, lse_s_o = O.select_topk(x["s"], K)
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), idx_o)
    lg = logg_o if gated else None
    o, lse = O.attn_fwd(x["q"], x["k"], x["v"], idx_o, lg, bs)
    eo, el = max_abs(r["o"].cpu(), o), max_abs(r["lse"].cpu(), lse)
    gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx_o, lg if gated else None,
                    x["s"], lse_s_o, bs) if gated else None
    if not gated:
        gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx_o, None, x["s"], lse_s_o, bs)
    errs = {"o": eo, "lse": el}
    for key in ("dq", "dk", "dv"):
        errs[key] = rel_l2(np64(r[key].cpu()), gr[key])
    if gated:
        errs["dlogg"] = rel_l2(np64(r["dlogg"].cpu()), gr["dlogg"])
        errs["ds"] = rel_l2(np64(r["ds"].cpu()), gr["ds"])
    say("  errors: " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    assert eo <= atol and el <= atol
    for key in ("dq", "dk", "dv", "dlogg", "ds"):
        if key in errs:
            assert errs[key] <= rtol, key
    return errs


def test_slot_map_past_4096_query_blocks():
    """T = 4100 query blocks: past the one-pass slot-map build (T <= 4096) the
    map is cleared, then marked entry by entry.  dK / dV of sampled key blocks
    and the gate gradients of the rows that selected them, against the oracle
    (fp32, block 16, a random selection of K = 3 per row)."""
    from gated_block_sparse_scores_amd import ops
    bs, T, K, d = 16, 4100, 3, 64
    say(f"slot map T={T}")
    w = synth.workload(1, batch=1, hq=1, hkv=1, seqlen=bs * T, head_dim=d, block=bs, topk=K,
                       dtype="f32")
    x = synth.train_inputs(w, seed=41, poison_invalid_scores=False)
    idx = synth.random_selection(1, 1, T, K, seed=42)
    logg = synth.random_log_gates((1, 1, T, K), seed=43)
    g = {k_: x[k_].to(DEV) for k_ in ("q", "k", "v", "dout")}
    idx_g, lg_g = idx.to(DEV), logg.to(DEV)
    o, lse = ops.attn_fwd(g["q"], g["k"], g["v"], idx_g, lg_g, bs)
    gr = ops.attn_bwd(g["q"], g["k"], g["v"], o, g["dout"], lse, idx_g, lg_g, None, None, bs,
                      want_ds=False)
    torch.cuda.synchronize()
    dk, dv, dl = gr["dk"].cpu(), gr["dv"].cpu(), gr["dlogg"].cpu()
    scale = 1.0 / math.sqrt(d)
    oi, ol = idx.numpy(), logg.numpy()
    counts = np.bincount(oi[0, 0][oi[0, 0] >= 0], minlength=T)
    _, rtol = tols(torch.float32)
    for m in sorted({int(np.argmax(counts)), T // 2, T - 2}):
        dkb, dvb = O.bwd_key_block(x["q"], x["k"], x["v"], x["dout"], oi, ol, bs, scale, 0, 0, m)
        lo, hi = O.block_span(m, bs, w.seqlen)
        ek, ev = rel_l2(np64(dk[0, 0, lo:hi]), dkb), rel_l2(np64(dv[0, 0, lo:hi]), dvb)
        say(f"  key block {m} ({int(counts[m])} selecting rows): dk {ek:.2e} dv {ev:.2e}")
        assert ek <= rtol and ev <= rtol, m
        for t in np.nonzero((oi[0, 0] == m).any(axis=1))[0][:4]:
            _, dlb, _ = O.bwd_row_block(x["q"], x["k"], x["v"], x["dout"], oi, ol, bs, scale, 0,
                                        0, int(t))
            assert rel_l2(np64(dl[0, 0, int(t)]), dlb) <= rtol, (m, int(t))


CASES = [
    # b, hq, hkv, n,   d,  bs, K
    (1, 1, 1, 256, 64, 16, 4),
    (1, 4, 2, 200, 64, 16, 3),
    (2, 4, 1, 130, 128, 32, 2),
    (1, 8, 2, 300, 128, 64, 3),
    (1, 5, 1, 257, 128, 64, 2),
    (1, 4, 4, 64, 128, 64, 1),
    (1, 2, 1, 1000, 64, 64, 64),
    # shapes served by the bf16 MFMA kernels (G even, d 128, block 64, N % 64 == 0)
    (1, 4, 1, 64, 128, 64, 2),
    (1, 4, 2, 384, 128, 64, 3),
    (1, 6, 1, 256, 128, 64, 2),
    (1, 8, 2, 512, 128, 64, 3),
    (2, 8, 1, 640, 128, 64, 5),
    (1, 16, 4, 1024, 128, 64, 16),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_fwd_bwd_small(case, dtype):
    b, hq, hkv, n, d, bs, K = case
    say(f"fwd+bwd {case} {dtype}")
    x = small_inputs(sum(case), b, hq, hkv, n, d, bs, K, dtype)
    r = run_gpu(x, K, bs)
    compare_full(x, r, K, bs, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_ungated_is_block_sparse_attention(dtype):
    """logg NULL computes picx Eq. 2 (no gates)."""
    x = small_inputs(3, 1, 4, 2, 192, 128, 64, 2, dtype)
    r = run_gpu(x, 2, 64, gated=False)
    compare_full(x, r, 2, 64, dtype, gated=False)


def test_tiny_fp32_workload():
    """seq 256, 1 head, d 64, block 16, K 4, fp32: the whole output and every
    gradient against the oracle."""
    w = synth.workload(1)
    x = synth.train_inputs(w)
    say("tiny fp32 workload")
    r = run_gpu(x, w.topk, w.block)
    compare_full(x, r, w.topk, w.block, torch.float32)


def test_repeat_runs_bitwise_equal():
    x = small_inputs(11, 1, 8, 2, 512, 128, 64, 3, torch.bfloat16)
    a = run_gpu(x, 3, 64)
    b_ = run_gpu(x, 3, 64)
    for key in ("o", "lse", "dq", "dk", "dv", "dlogg", "ds"):
        assert torch.equal(a[key], b_[key]), key


def test_ds_rows_sum_to_zero_and_empty_first_row():
    x = small_inputs(13, 1, 4, 2, 640, 128, 64, 3, torch.bfloat16)
    r = run_gpu(x, 3, 64)
    ds = np64(r["ds"].cpu())
    scale = np.abs(ds).max()
    assert np.abs(ds.sum(-1)).max() <= 1e-5 * scale
    assert np.all(ds[..., 0, :] == 0)
    T = ds.shape[-1]
    assert np.all(ds[..., np.triu(np.ones((T, T), dtype=bool))] == 0)


# ------------------------------------------------------------------ full-size workloads, sampled

def run_workload(wl):
    from gated_block_sparse_scores_amd import ops
    w = synth.workload(wl)
    x = synth.train_inputs(w, device=DEV)
    T = w.nblocks
    if w.scores == "standin":
        qb = ops.block_pool(x["q"], w.block, w.group)
        kb = ops.block_pool(x["k"], w.block, 1)
        idx, logg, lse_s, s = ops.select_topk(w.batch, w.hkv, T, T, w.topk, qbar=qb, kbar=kb)
    else:
        s = x["s"]
        idx, logg, lse_s, _ = ops.select_topk(w.batch, w.hkv, T, T, w.topk, s=s)
    o, lse = ops.attn_fwd(x["q"], x["k"], x["v"], idx, logg, w.block)
    gr = ops.attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg, s, lse_s, w.block)
    torch.cuda.synchronize()
    return w, x, dict(idx=idx, logg=logg, lse_s=lse_s, s=s, o=o, lse=lse, **gr)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("wl", [2, 3])
def test_training_workload_sampled(wl):
    """Full-size training workloads (8K tokens / 32K tokens, 32/8 heads, d 128,
    block 64).  For every KV head the oracle recomputes sampled query blocks
    (o, LSE, dq, dlogg, ds) and sampled key blocks (dk, dv; always including
    the key block with that head's longest inverse list) on the device's
    selection, which is itself checked against the oracle's Top-K of the same
    fp32 scores.  Each sampled block is held to the tolerance on its own, and
    the pooled errors too."""
    say(f"training workload {wl}")
    t_start = time.perf_counter()
    w, x, r = run_workload(wl)
    T = w.nblocks
    xc = {k_: x[k_].cpu() for k_ in ("q", "k", "v", "dout")}
    if w.scores == "standin":
        # the oracle's own stand-in scores from the inputs; the device's agree
        # with them except where the fp64 dot lands on an fp32 rounding boundary
        qo = O.to_f32(O.pool_queries(xc["q"], w.hkv, w.block))
        ko = O.to_f32(O.pool_keys(xc["k"], w.block))
        s_np = O.standin_scores(qo, ko, O.default_scale(w.head_dim), T)
        valid = np.tril(np.ones((T, T), dtype=bool), -1)
        assert np.sum((r["s"].cpu().numpy() != s_np) & valid) <= 2
    else:
        s_np = x["s"].cpu().numpy()
    oi, ol, ols = O.select_topk(s_np, w.topk)
    np.testing.assert_array_equal(r["idx"].cpu().numpy(), oi)
    assert max_abs(r["logg"].cpu().numpy(), ol) <= GATE_ATOL
    scale = O.default_scale(w.head_dim)
    rng = np.random.default_rng(wl)
    g = w.group
    o_gpu, lse_gpu, dq_gpu = r["o"].cpu(), r["lse"].cpu(), r["dq"].cpu()
    ds_gpu, dl_gpu = r["ds"].cpu().numpy(), r["dlogg"].cpu().numpy()
    dk_gpu, dv_gpu = r["dk"].cpu(), r["dv"].cpu()
    errs = {"o": 0.0, "lse": 0.0}
    blocks = {k_: [] for k_ in ("dq", "dlogg", "ds", "dk", "dv")}

    def acc(name, got, ref, where):
        blocks[name].append((float(np.sum((got - ref) ** 2)), float(np.sum(ref ** 2)), where))

    nblk = nkey = 0
    for kv in range(w.hkv):
        tsamp = sorted({0, 1, T // 2, T - 1, *rng.integers(0, T, 2).tolist()})
        for t in tsamp:
            lo, hi = O.block_span(t, w.block, w.seqlen)
            ob, lb, _, _ = O.fwd_row_block(xc["q"], xc["k"], xc["v"], oi, ol, w.block, scale, 0,
                                           kv, t)
            hs = slice(kv * g, (kv + 1) * g)
            errs["o"] = max(errs["o"], max_abs(o_gpu[0, hs, lo:hi], ob))
            errs["lse"] = max(errs["lse"], max_abs(lse_gpu[0, hs, lo:hi], lb))
            dqb, dlb, _ = O.bwd_row_block(xc["q"], xc["k"], xc["v"], xc["dout"], oi, ol, w.block,
                                          scale, 0, kv, t)
            acc("dq", np64(dq_gpu[0, hs, lo:hi]), dqb, (kv, t))
            if t > 0:
                acc("dlogg", dl_gpu[0, kv, t], dlb, (kv, t))
                dsr = O.ds_row(s_np[0, kv, t, :t], ols[0, kv, t], oi[0, kv, t], dlb)
                acc("ds", ds_gpu[0, kv, t, :t], dsr, (kv, t))
            nblk += 1
        # key blocks: the longest inverse list of this head (the most query
        # blocks folded into one dK / dV), the second to last block, and for
        # the first and last head a middle block
        counts = np.bincount(oi[0, kv][oi[0, kv] >= 0], minlength=T)
        msamp = {int(np.argmax(counts)), T - 2}
        if kv in (0, w.hkv - 1):
            msamp.add(int(rng.integers(T // 3, T - 2)))
        msamp = sorted(msamp)
        nkey += len(msamp)
        for m in msamp:
            dkb, dvb = O.bwd_key_block(xc["q"], xc["k"], xc["v"], xc["dout"], oi, ol, w.block,
                                       scale, 0, kv, m)
            lo, hi = O.block_span(m, w.block, w.seqlen)
            acc("dk", np64(dk_gpu[0, kv, lo:hi]), dkb, (kv, m, int(counts[m])))
            acc("dv", np64(dv_gpu[0, kv, lo:hi]), dvb, (kv, m, int(counts[m])))
    # Every sampled block on its own: its error over its own norm, or over the
    # RMS block norm of that quantity when larger (a dlogg row of one history
    # block, or a ds row, can be a near-zero sum of cancelling terms), and the
    # pooled relative L2 over all sampled blocks.
    worst = {}
    for name, rows in blocks.items():
        rms = math.sqrt(sum(d_ for _, d_, _ in rows) / len(rows))
        for num, den, where in rows:
            e = math.sqrt(num) / max(math.sqrt(den), rms)
            if e > worst.get(name, (0.0, None))[0]:
                worst[name] = (e, where)
            assert e <= 3e-2, f"{name} error {e:.3e} at {where}"
        errs[name] = math.sqrt(sum(n_ for n_, _, _ in rows) / sum(d_ for _, d_, _ in rows))
    say(f"  {nblk} query blocks and {nkey} key blocks over all {w.hkv} KV heads; "
        "pooled errors: " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    say("  worst block: " + ", ".join(f"{k_}={e:.2e} at {wh}" for k_, (e, wh) in worst.items()))
    say(f"  host time {time.perf_counter() - t_start:.1f} s")
    assert errs["o"] <= 2e-2 and errs["lse"] <= 2e-2
    for name in ("dq", "dlogg", "ds", "dk", "dv"):
        assert errs[name] <= 3e-2, name
    # invariants over every row
    ds_all = np64(r["ds"])
    assert np.abs(ds_all.sum(-1)).max() <= 1e-5 * np.abs(ds_all).max()
    assert torch.isfinite(r["dq"]).all() and torch.isfinite(r["dk"]).all()
