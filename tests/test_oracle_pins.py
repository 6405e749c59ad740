"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test names the pin it implements and the passage that fixes it (page
titles as in the oracle's header).  None of them compares the oracle with
itself: the references are textbook attention (torch's scaled_dot_product_attention
in float64), autograd, brute-force enumeration, finite differences, closed forms
and invariants.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import sas_oracle as O

F64 = torch.float64


def small(seed=0, b=1, hq=2, hkv=1, n=48, d=8, bs=8, K=2, s_std=math.sqrt(2.0)):
    w = synth.workload(1, batch=b, hq=hq, hkv=hkv, seqlen=n, head_dim=d, block=bs, topk=K)
    x = synth.train_inputs(w, seed=seed, poison_invalid_scores=False)
    t = O.n_blocks(n, bs)
    x["s"] = synth.random_scores((b, hkv, t, t), seed=seed + 1000, std=s_std)
    return w, x


def select(x, K):
    return O.select_topk(x["s"], K)


def sdpa(q, k, v, mask=None, causal=False, scale=None):
    """Textbook attention via torch (float64)."""
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask, is_causal=causal,
                                          scale=scale)


def expand_kv(x, g):
    return x.repeat_interleave(g, dim=1)


# ---------------------------------------------------------------- P1: one history block == dense causal

@pytest.mark.parametrize("n_blocks_", [1, 2])
@pytest.mark.parametrize("K", [1, 3])
def test_p1_single_history_block_is_dense_causal(n_blocks_, K):
    """picx 'Key Idea' Eq. 4 / Eq. 6: with one history block the gate softmax is
    exactly 1 (log g = 0), and the current block has g0 = 1, so gated sparse
    attention over N = 2*bs (or N = bs) tokens is plain causal attention."""
    bs = 8
    w, x = small(seed=3, hq=4, hkv=2, n=bs * n_blocks_, d=16, bs=bs, K=K)
    idx, logg, lse_s = select(x, K)
    assert np.all(logg[idx >= 0] == 0.0)
    o, lse = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    q, k, v = (x[n].to(F64).requires_grad_() for n in ("q", "k", "v"))
    ref = sdpa(q, expand_kv(k, 2), expand_kv(v, 2), causal=True)
    np.testing.assert_allclose(o, ref.detach().numpy(), atol=1e-13, rtol=0)
    # LSE against torch.logsumexp of the causal logits
    z = (q @ expand_kv(k, 2).transpose(-1, -2)) / math.sqrt(16)
    z = z.masked_fill(torch.ones(z.shape[-2:], dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(z, -1).detach().numpy(), atol=1e-13)
    # gradients against autograd, and ds == 0 exactly
    dout = x["dout"].to(F64)
    (ref * dout).sum().backward()
    gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx, logg, x["s"], lse_s, bs)
    np.testing.assert_allclose(gr["dq"], q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dk"], k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dv"], v.grad.numpy(), atol=1e-12)
    assert np.all(gr["ds"] == 0.0)


# ---------------------------------------------------------------- P2: shift invariance of s

def test_p2_score_shift_invariance():
    """picx Eq. 6: log g_m = s_m - LSE(s) is unchanged by s -> s + c per row, and
    Top-K by s is unchanged; so idx, gates, o, LSE and every gradient are too.
    Scores are quantised to 2^-10 so that s + c is exact in fp32 (and has ties)."""
    bs, K = 8, 3
    w, x = small(seed=5, hq=2, hkv=1, n=64, d=8, bs=bs, K=K)
    s = torch.round(x["s"] * 1024) / 1024
    c = torch.tensor([4.0, -2.0, 8.0, 0.5, 1.0, -4.0, 2.0, 16.0]).view(1, 1, 8, 1)
    s2 = s + c
    assert torch.equal(s2 - c, s)
    a = O.select_topk(s, K)
    b_ = O.select_topk(s2, K)
    np.testing.assert_array_equal(a[0], b_[0])
    np.testing.assert_allclose(a[1], b_[1], atol=1e-12)
    oa = O.attn_fwd(x["q"], x["k"], x["v"], a[0], a[1], bs)
    ob = O.attn_fwd(x["q"], x["k"], x["v"], b_[0], b_[1], bs)
    np.testing.assert_allclose(oa[0], ob[0], atol=1e-12)
    ga = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], a[0], a[1], s, a[2], bs)
    gb = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], b_[0], b_[1], s2, b_[2], bs)
    for key in ("dq", "dk", "dv", "ds", "dlogg"):
        np.testing.assert_allclose(ga[key], gb[key], atol=1e-11)


# ---------------------------------------------------------------- P3: sum of ds over the history is 0

def test_p3_ds_sums_to_zero():
    """The Jacobian of s -> s - LSE(s) annihilates the all-ones vector (picx Eq. 6),
    so every row of ds sums to zero."""
    bs, K = 8, 2
    w, x = small(seed=7, hq=4, hkv=2, n=80, d=8, bs=bs, K=K)
    idx, logg, lse_s = select(x, K)
    gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx, logg, x["s"], lse_s, bs)
    rows = gr["ds"].sum(axis=-1)
    scale = np.abs(gr["ds"]).max()
    assert scale > 0
    assert np.abs(rows).max() <= 1e-13 * max(1.0, scale)
    # and some unselected block gets a nonzero gradient (softmax over all history)
    unselected = np.ones_like(gr["ds"], dtype=bool)
    for t in range(gr["ds"].shape[2]):
        unselected[..., t, t:] = False
        for kv in range(2):
            for m in idx[0, kv, t]:
                if m >= 0:
                    unselected[0, kv, t, m] = False
    assert np.abs(gr["ds"][unselected]).max() > 0


# ---------------------------------------------------------------- P4: dense scope == library masked softmax

def _dense_scope_mask(s_leaf, n, bs):
    """Float attention bias of dense-scope SAS, built with torch ops:
    log_softmax(s_t[:t]) on history block m, 0 on the causal current block."""
    T = O.n_blocks(n, bs)
    rows = []
    for t in range(T):
        lo, hi = O.block_span(t, bs, n)
        r = hi - lo
        pieces = []
        if t > 0:
            ls = torch.log_softmax(s_leaf[t, :t], dim=0)
            for m in range(t):
                mlo, mhi = O.block_span(m, bs, n)
                pieces.append(ls[m].expand(r, mhi - mlo))
        causal = torch.zeros(r, r, dtype=F64).masked_fill(
            torch.ones(r, r, dtype=torch.bool).triu(1), -math.inf)
        pieces.append(causal)
        if hi < n:
            pieces.append(torch.full((r, n - hi), -math.inf, dtype=F64))
        rows.append(torch.cat(pieces, dim=1))
    return torch.cat(rows, dim=0)


def test_p4_dense_scope_matches_library_softmax_and_autograd():
    """K >= C_t for every row (dense scope, picx summary 'Overview'): no Top-K
    is active, so o is softmax(qK^T/sqrt(d) + log g)V with log g = log_softmax(s)
    (picx Eq. 6, Eq. 9) -- torch's scaled_dot_product_attention with a float mask --
    and dq/dk/dv/ds are torch autograd through it."""
    bs, n = 8, 44                        # ragged last block
    T = O.n_blocks(n, bs)
    w, x = small(seed=11, hq=4, hkv=2, n=n, d=8, bs=bs, K=T)
    idx, logg, lse_s = select(x, T)
    o, lse = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    g = 2
    q, k, v = (x[nm].to(F64).requires_grad_() for nm in ("q", "k", "v"))
    # torch reference per kv head (each kv head has its own s row set)
    outs = []
    s_leafs = []
    for kv in range(2):
        sl = x["s"][0, kv].to(F64).clone().requires_grad_()
        s_leafs.append(sl)
        mask = _dense_scope_mask(sl, n, bs)
        heads = slice(kv * g, (kv + 1) * g)
        outs.append(sdpa(q[:, heads], k[:, kv:kv + 1].expand(-1, g, -1, -1),
                         v[:, kv:kv + 1].expand(-1, g, -1, -1), mask=mask))
    ref = torch.cat(outs, dim=1)
    np.testing.assert_allclose(o, ref.detach().numpy(), atol=1e-13)
    dout = x["dout"].to(F64)
    (ref * dout).sum().backward()
    gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx, logg, x["s"], lse_s, bs)
    np.testing.assert_allclose(gr["dq"], q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dk"], k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dv"], v.grad.numpy(), atol=1e-12)
    for kv in range(2):
        ref_ds = s_leafs[kv].grad.numpy()
        ref_ds = np.tril(ref_ds, -1)              # only m < t is read
        np.testing.assert_allclose(gr["ds"][0, kv], ref_ds, atol=1e-12)


# ---------------------------------------------------------------- P5: brute-force Top-K with ties

def test_p5_topk_bruteforce_with_ties():
    """picx Eq. 3, ties to the lower block index: among all K-subsets of the
    history with the largest score sum, the lexicographically smallest sorted
    index list.  Integer-valued scores force many exact ties."""
    rng = np.random.default_rng(0)
    for trial in range(300):
        C = int(rng.integers(1, 12))
        s = rng.integers(-2, 3, size=C).astype(np.float32)
        K = int(rng.integers(1, C + 2))
        kk = min(K, C)
        best = None
        for comb in itertools.combinations(range(C), kk):
            key = (-float(s[list(comb)].sum()), comb)
            if best is None or key < best:
                best = key
        np.testing.assert_array_equal(O.topk_history(s, K), np.array(best[1]))


def test_p5_negative_zero_ties_with_zero():
    s = np.array([0.0, -0.0, 0.0, -1.0, -0.0], dtype=np.float32)
    np.testing.assert_array_equal(O.topk_history(s, 2), [0, 1])
    s = np.array([-0.0, 0.0], dtype=np.float32)
    np.testing.assert_array_equal(O.topk_history(s, 1), [0])


# ---------------------------------------------------------------- P6: finite differences

def _loss(x, s, K, bs):
    idx, logg, _ = O.select_topk(s, K)
    o, _ = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    return float((o * O._np64(x["dout"])).sum()), idx


def test_p6_finite_differences():
    """Central differences (eps = 1e-6, float64) of L = sum dO . o with respect to
    every valid score and every entry of q, k, v.  Top-K is piecewise constant
    (picx 'Theoretical Foundation'), so the selection must not move under +-eps;
    the test asserts it."""
    bs, n, K = 6, 20, 2                  # T = 4, ragged last block
    w, x = small(seed=13, hq=2, hkv=1, n=n, d=4, bs=bs, K=K)
    x = {k_: (v_.to(F64) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    s = x["s"].numpy().astype(np.float64)
    idx, logg, lse_s = O.select_topk(s.astype(np.float32), K)
    s32 = s.astype(np.float32).astype(np.float64)
    gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx, logg, s32, lse_s, bs)
    eps = 1e-6

    def fd_s(t, m):
        sp, sm = s32.copy(), s32.copy()
        sp[0, 0, t, m] += eps
        sm[0, 0, t, m] -= eps
        # the fp32 ranking of the perturbed rows must equal the unperturbed one
        lp, ip = _loss_s(x, sp, K, bs)
        lm, im = _loss_s(x, sm, K, bs)
        assert np.array_equal(ip, idx) and np.array_equal(im, idx)
        return (lp - lm) / (2 * eps)

    T = O.n_blocks(n, bs)
    for t in range(1, T):
        for m in range(t):
            fd = fd_s(t, m)
            assert abs(fd - gr["ds"][0, 0, t, m]) <= 1e-8 + 1e-6 * abs(fd), (t, m)

    for name, grad in (("q", gr["dq"]), ("k", gr["dk"]), ("v", gr["dv"])):
        base = x[name].clone()
        for pos in itertools.product(*[range(sz) for sz in base.shape]):
            xp = dict(x)
            tp = base.clone()
            tp[pos] += eps
            xp[name] = tp
            lp = _loss_s(xp, s32, K, bs)[0]
            tm = base.clone()
            tm[pos] -= eps
            xp[name] = tm
            lm = _loss_s(xp, s32, K, bs)[0]
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-8 + 1e-6 * abs(fd), (name, pos)


def _loss_s(x, s64, K, bs):
    """L for float64 scores: selection is decided on fp32 values, gates use the
    exact float64 score (as the derivative requires)."""
    s32 = s64.astype(np.float32)
    idx, _, _ = O.select_topk(s32, K)
    b, hkv, T, _ = s64.shape
    logg = np.zeros(idx.shape)
    for t in range(T):
        if t == 0:
            continue
        lse = O.gate_normaliser(s64[0, 0, t, :t])
        for sl, m in enumerate(idx[0, 0, t]):
            if m >= 0:
                logg[0, 0, t, sl] = s64[0, 0, t, m] - lse
    o, _ = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    return float((o * O._np64(x["dout"])).sum()), idx


# ---------------------------------------------------------------- P7: Eq. 5 closed form

def test_p7_inner_gate_gradient_closed_form():
    """picx 'Gradient Analysis' Eq. 5 (inner gating):
    dg_m = sum_{i in B_m} (p_i / g_m) dO^T (v_i - o), hence
    d(log g_m) = g_m dg_m = sum_{rows} sum_{j in B_m} p_ij dO_i . (v_j - o_i),
    evaluated here from the forward's probabilities, with no dS and no D."""
    bs, K = 8, 3
    w, x = small(seed=17, hq=4, hkv=2, n=72, d=8, bs=bs, K=K)
    idx, logg, lse_s = select(x, K)
    gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx, logg, x["s"], lse_s, bs)
    scale = O.default_scale(8)
    T = O.n_blocks(72, bs)
    for kv in range(2):
        for t in range(T):
            o, _, ps, (J, bias, slot, cur, kj, vj) = O.fwd_row_block(
                x["q"], x["k"], x["v"], idx, logg, bs, scale, 0, kv, t)
            for sl in range(K):
                if idx[0, kv, t, sl] < 0:
                    continue
                cols = np.nonzero(slot == sl)[0]
                total = 0.0
                for gi, h in enumerate(range(kv * 2, kv * 2 + 2)):
                    lo, hi = O.block_span(t, bs, 72)
                    do = O._np64(x["dout"][0, h, lo:hi])
                    for r in range(hi - lo):
                        for c in cols:
                            total += ps[gi][r, c] * do[r] @ (vj[c] - o[gi][r])
                assert abs(total - gr["dlogg"][0, kv, t, sl]) <= 1e-12


# ---------------------------------------------------------------- P8: decode == last row of forward

@pytest.mark.parametrize("L", [64, 61])
def test_p8_decode_equals_last_forward_row(L):
    """Decode at position L-1 with the selection of the last query block equals
    the forward's output row L-1 (same keys, same biases); GQA equals MHA with
    K/V repeated per group under the shared selection (picx 'Efficiency
    Benefits': GQA with per-group selection)."""
    bs, K = 8, 3
    w, x = small(seed=19, hq=4, hkv=2, n=L, d=8, bs=bs, K=K)
    idx, logg, lse_s = select(x, K)
    o, lse = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    t = (L - 1) // bs
    od, lsed = O.decode(x["q"][:, :, L - 1], x["k"], x["v"], L, idx[:, :, t], logg[:, :, t], bs)
    np.testing.assert_allclose(od, o[:, :, L - 1], atol=1e-13)
    np.testing.assert_allclose(lsed, lse[:, :, L - 1], atol=1e-13)
    # GQA == MHA with repeated K/V and the selection repeated per query head
    k4, v4 = expand_kv(x["k"], 2), expand_kv(x["v"], 2)
    om, lsem = O.decode(x["q"][:, :, L - 1], k4, v4, L, np.repeat(idx[:, :, t], 2, axis=1),
                        np.repeat(logg[:, :, t], 2, axis=1), bs)
    np.testing.assert_allclose(om, od, atol=1e-13)


def test_p8_decode_ungated_is_library_attention_over_selected_keys():
    """logg = None is picx Eq. 2 (gates dropped at inference, evolve 'Summary'):
    plain softmax attention over the selected blocks plus the current prefix."""
    bs, K, L = 8, 2, 53
    w, x = small(seed=23, hq=2, hkv=1, n=L, d=8, bs=bs, K=K)
    idx, _, _ = select(x, K)
    t = (L - 1) // bs
    od, _ = O.decode(x["q"][:, :, L - 1], x["k"], x["v"], L, idx[:, :, t], None, bs)
    keys = [j for m in idx[0, 0, t] if m >= 0 for j in range(m * bs, (m + 1) * bs)]
    keys += list(range(t * bs, L))
    q = x["q"][:, :, L - 1:L].to(F64)
    ref = sdpa(q, x["k"][:, :, keys].to(F64).expand(-1, 2, -1, -1),
               x["v"][:, :, keys].to(F64).expand(-1, 2, -1, -1))
    np.testing.assert_allclose(od, ref[:, :, 0].numpy(), atol=1e-13)


# ---------------------------------------------------------------- P9: gate limit

def test_p9_dominant_gate_limit():
    """Raising one history score by 40 drives every other history gate to
    ~e^-40 (picx Eq. 6) while the raised block's log-gate -> 0, so the output is
    plain attention over {that block, current block} up to e^-40-level terms."""
    bs, K, n = 8, 3, 64
    w, x = small(seed=29, hq=1, hkv=1, n=n, d=8, bs=bs, K=K, s_std=0.5)
    s = x["s"].clone()
    t, mstar = 7, 2
    s[0, 0, t, mstar] += 40.0
    idx, logg, _ = O.select_topk(s, K)
    assert mstar in idx[0, 0, t]
    o, _ = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    keys = list(range(mstar * bs, (mstar + 1) * bs))
    lo = t * bs
    q = x["q"][:, :, lo:lo + bs].to(F64)
    kk = torch.cat([x["k"][:, :, keys], x["k"][:, :, lo:lo + bs]], dim=2).to(F64)
    vv = torch.cat([x["v"][:, :, keys], x["v"][:, :, lo:lo + bs]], dim=2).to(F64)
    mask = torch.zeros(bs, 2 * bs, dtype=F64)
    mask[:, bs:] = mask[:, bs:].masked_fill(torch.ones(bs, bs, dtype=torch.bool).triu(1),
                                            -math.inf)
    ref = sdpa(q, kk, vv, mask=mask)
    np.testing.assert_allclose(o[0, 0, lo:lo + bs], ref[0, 0].numpy(), atol=1e-12)


# ---------------------------------------------------------------- P10: gathered == dense, sums, poisoning

def test_p10_gather_equals_dense_and_rows_normalise():
    """picx 'Kernel Design' (mask non-selected blocks) and daiwk 'Scope' (dense
    materialised reference): the masked N x N formulation and the gathered one
    agree; each probability row sums to one."""
    bs, K, n = 8, 2, 70
    w, x = small(seed=31, hq=4, hkv=2, n=n, d=8, bs=bs, K=K)
    idx, logg, _ = select(x, K)
    a = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    b_ = O.attn_fwd_dense(x["q"], x["k"], x["v"], idx, logg, bs)
    np.testing.assert_allclose(a[0], b_[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b_[1], atol=1e-13)
    for t in range(O.n_blocks(n, bs)):
        _, _, ps, _ = O.fwd_row_block(x["q"], x["k"], x["v"], idx, logg, bs,
                                      O.default_scale(8), 0, 1, t)
        for p in ps:
            np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)


def test_p10_invalid_scores_are_never_read():
    bs, K, n = 8, 2, 64
    w, x = small(seed=37, hq=2, hkv=1, n=n, d=8, bs=bs, K=K)
    s = x["s"].clone()
    poisoned = s.clone()
    T = O.n_blocks(n, bs)
    poisoned[..., torch.ones(T, T, dtype=torch.bool).triu()] = float("nan")
    a = O.select_topk(s, K)
    b_ = O.select_topk(poisoned, K)
    for u, v in zip(a, b_):
        np.testing.assert_array_equal(u, v)
    ga = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], a[0], a[1], s, a[2], bs)
    gb = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], b_[0], b_[1], poisoned, b_[2], bs)
    for key in ga:
        np.testing.assert_array_equal(ga[key], gb[key])


# ---------------------------------------------------------------- stand-in scorer pins

def test_pooling_matches_library_mean_and_ragged_tail():
    """Mean pooling of block summaries (evolve FAQ: pooling-based block
    summaries) equals torch.mean over the block's valid tokens (and group heads)."""
    bs, n = 8, 30
    w, x = small(seed=41, hq=6, hkv=2, n=n, d=4, bs=bs)
    kb = O.pool_keys(x["k"], bs)
    qb = O.pool_queries(x["q"], 2, bs)
    k64, q64 = x["k"].to(F64), x["q"].to(F64)
    for m in range(O.n_blocks(n, bs)):
        lo, hi = O.block_span(m, bs, n)
        np.testing.assert_allclose(kb[:, :, m], k64[:, :, lo:hi].mean(2).numpy(), atol=1e-15)
        for kv in range(2):
            ref = q64[:, kv * 3:(kv + 1) * 3, lo:hi].reshape(1, -1, 4).mean(1)
            np.testing.assert_allclose(qb[:, kv, m], ref.numpy(), atol=1e-15)


def test_standin_scores_library_matmul_and_validity():
    bs, n = 8, 64
    w, x = small(seed=43, hq=4, hkv=2, n=n, d=8, bs=bs)
    qb = O.to_f32(O.pool_queries(x["q"], 2, bs))
    kb = O.to_f32(O.pool_keys(x["k"], bs))
    T = 8
    s = O.standin_scores(qb, kb, O.default_scale(8), T)
    ref = (torch.from_numpy(qb).double() @ torch.from_numpy(kb).double().transpose(-1, -2)
           ) / math.sqrt(8)
    for t in range(T):
        np.testing.assert_array_equal(s[..., t, :t], ref[..., t, :t].float().numpy())
        assert np.all(s[..., t, t:] == 0)
    # decode mode: one row with row_offset = C sees the whole history
    sd = O.standin_scores(qb[:, :, :1], kb, O.default_scale(8), 7, row_offset=7)
    np.testing.assert_array_equal(sd[..., 0, :], ref[..., 0, :7].float().numpy())


def test_selected_pairs_counts_keys():
    bs, n, K = 8, 40, 2
    w, x = small(seed=47, hq=2, hkv=1, n=n, d=4, bs=bs, K=K)
    idx, logg, _ = select(x, K)
    count = 0
    for t in range(O.n_blocks(n, bs)):
        J, _, _, cur = O.key_set(t, idx[0, 0, t], None, bs, n)
        lo, hi = O.block_span(t, bs, n)
        for i in range(lo, hi):
            count += int(np.sum(~cur)) + int(np.sum(cur & (J <= i)))
    assert O.selected_pairs(idx, n, bs, 2) == 2 * count


# ---------------------------------------------------------------- P11-P13: selector backward (stand-in)

def _standin_loss(q, k, v, dout, K, bs, idx_fixed=None):
    """L = sum dO . o with s = scale * pooled(q) . pooled(k) in float64 (the
    stand-in selector), gates log g = s - LSE(s) over the history, selection
    decided on the fp32 scores.  Returns L, idx and the float64 scores."""
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    qb = O.pool_queries(q, hkv, bs)
    kb = O.pool_keys(k, bs)
    scale = 1.0 / math.sqrt(d)
    s64 = np.einsum("bktd,bkmd->bktm", qb, kb) * scale
    idx, _, _ = O.select_topk(s64.astype(np.float32), K)
    if idx_fixed is not None:
        assert np.array_equal(idx, idx_fixed), "selection moved under the perturbation"
    T = s64.shape[2]
    logg = np.zeros(idx.shape)
    lse = np.full(s64.shape[:3], -math.inf)
    for bb in range(b):
        for kv in range(hkv):
            for t in range(1, T):
                lse[bb, kv, t] = O.gate_normaliser(s64[bb, kv, t, :t])
                for sl, m in enumerate(idx[bb, kv, t]):
                    if m >= 0:
                        logg[bb, kv, t, sl] = s64[bb, kv, t, m] - lse[bb, kv, t]
    o, _ = O.attn_fwd(q, k, v, idx, logg, bs)
    return float((o * O._np64(dout)).sum()), idx, logg, s64, lse, qb, kb


def test_p11_standin_chain_finite_differences():
    """Central differences of L with respect to every entry of q and k, where q
    and k reach L both through attention and through the stand-in scores (mean
    pools, dot product, gate softmax).  The analytic gradient is the attention
    backward plus the selector backward spread through the pools' adjoints."""
    bs, n, K = 6, 20, 2                  # T = 4, ragged last block
    w, x = small(seed=21, hq=4, hkv=2, n=n, d=4, bs=bs, K=K)
    q, k, v, dout = (x[n_].to(F64) for n_ in ("q", "k", "v", "dout"))
    L0, idx, logg, s64, lse, qb, kb = _standin_loss(q, k, v, dout, K, bs)
    gr = O.attn_bwd(q, k, v, dout, idx, logg, s64, lse, bs)
    dqb, dkb = O.selector_bwd(gr["ds"], qb, kb, 1.0 / math.sqrt(4))
    dq = gr["dq"] + O.pool_queries_bwd(dqb, q.shape[1], n, bs)
    dk = gr["dk"] + O.pool_keys_bwd(dkb, n, bs)
    assert np.abs(O.pool_queries_bwd(dqb, q.shape[1], n, bs)).max() > 1e-4   # not vacuous
    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk)):
        base = q if name == "q" else k
        for pos in itertools.product(*[range(sz) for sz in base.shape]):
            tp, tm = base.clone(), base.clone()
            tp[pos] += eps
            tm[pos] -= eps
            args_p = (tp, k) if name == "q" else (q, tp)
            args_m = (tm, k) if name == "q" else (q, tm)
            lp = _standin_loss(*args_p, v, dout, K, bs, idx_fixed=idx)[0]
            lm = _standin_loss(*args_m, v, dout, K, bs, idx_fixed=idx)[0]
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-8 + 1e-6 * abs(fd), (name, pos, fd, grad[pos])


def test_p12_pool_adjoints():
    """<pool(x), y> == <x, pool_bwd(y)> for the query pool (heads and tokens)
    and the key pool, ragged last block included."""
    rng = np.random.default_rng(5)
    b, hq, hkv, n, d, bs = 2, 6, 2, 23, 3, 5
    q = rng.standard_normal((b, hq, n, d))
    k = rng.standard_normal((b, hkv, n, d))
    T = O.n_blocks(n, bs)
    y = rng.standard_normal((b, hkv, T, d))
    lhs = (O.pool_queries(q, hkv, bs) * y).sum()
    rhs = (q * O.pool_queries_bwd(y, hq, n, bs)).sum()
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    lhs = (O.pool_keys(k, bs) * y).sum()
    rhs = (k * O.pool_keys_bwd(y, n, bs)).sum()
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_p13_selector_bwd_matches_autograd():
    """torch float64 autograd of sum(ds * s) over the valid history, with s the
    pooled stand-in scores written with torch ops, against the oracle's selector
    backward and pool adjoints (training rows: C_t = t; decode-style rows with
    an offset: C_t = min(t + row_offset, C))."""
    gen = torch.Generator().manual_seed(8)
    b, hq, hkv, n, d, bs = 2, 4, 2, 29, 6, 6
    T = O.n_blocks(n, bs)
    for row_offset, C in ((0, T), (3, T + 2)):
        q = torch.randn(b, hq, n, d, generator=gen, dtype=F64, requires_grad=True)
        k = torch.randn(b, hkv, C * bs if C > T else n, d, generator=gen, dtype=F64,
                        requires_grad=True)
        nk = k.shape[2]
        ds = torch.randn(b, hkv, T, C, generator=gen, dtype=F64)
        # pooled q: mean over the G heads of each group and the block's tokens
        g = hq // hkv
        qg = q.reshape(b, hkv, g, n, d)
        qbar = torch.stack([qg[:, :, :, t * bs:min(n, (t + 1) * bs)].mean(dim=(2, 3))
                            for t in range(T)], dim=2)
        kbar = torch.stack([k[:, :, m * bs:min(nk, (m + 1) * bs)].mean(dim=2)
                            for m in range(C)], dim=2)
        s = torch.matmul(qbar, kbar.transpose(2, 3)) / math.sqrt(d)
        mask = torch.zeros(T, C, dtype=F64)
        for t in range(T):
            mask[t, :min(t + row_offset, C)] = 1.0
        (ds * mask * s).sum().backward()
        dqb, dkb = O.selector_bwd(ds.numpy(), qbar.detach().numpy(), kbar.detach().numpy(),
                                  1.0 / math.sqrt(d), row_offset=row_offset)
        assert torch.isfinite(q.grad).all() and torch.isfinite(k.grad).all()
        np.testing.assert_allclose(O.pool_queries_bwd(dqb, hq, n, bs), q.grad.numpy(),
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(O.pool_keys_bwd(dkb, nk, bs), k.grad.numpy(), rtol=1e-12,
                                   atol=1e-13)


# ---------------------------------------------------------------- P14-P17: gate variants

def test_p14_gate_activations_closed_forms():
    """log g under each activation of [picx] Eq. 4 equals its library form
    (torch log_softmax over the history, logsigmoid, identity); the Top-K set is
    the same for all three (phi is monotone)."""
    w, x = small(seed=31, n=64, bs=8, K=3)
    s32 = x["s"].numpy().astype(np.float32)
    base_idx = None
    for act, ref in (("softmax", None), ("sigmoid", F.logsigmoid), ("raw", lambda z: z)):
        idx, logg, lse = O.select_topk(s32, 3, act=act)
        if base_idx is None:
            base_idx = idx
        assert np.array_equal(idx, base_idx)
        T = s32.shape[2]
        for t in range(1, T):
            row = torch.from_numpy(s32[0, 0, t, :t].astype(np.float64))
            full = torch.log_softmax(row, 0) if act == "softmax" else ref(row)
            for sl, m in enumerate(idx[0, 0, t]):
                if m >= 0:
                    assert abs(logg[0, 0, t, sl] - float(full[m])) <= 1e-12


def _outer_reference(q, k, v, idx, logg, bs):
    """o = softmax(q K_J^T / sqrt(d), causal on the current block) @ (g * V_J),
    written with torch ops per query block and head (outer gating; query head h
    reads KV head h // G and that KV head's selection)."""
    b, hq, n, d = q.shape
    g_ = hq // k.shape[1]
    out = torch.zeros(b, hq, n, d, dtype=F64)
    for t in range(O.n_blocks(n, bs)):
        lo, hi = O.block_span(t, bs, n)
        for h in range(hq):
            kv = h // g_
            keys, gains = [], []
            for sl, m in enumerate(idx[0, kv, t].tolist()):
                if m >= 0:
                    mlo, mhi = O.block_span(m, bs, n)
                    keys += list(range(mlo, mhi))
                    gains += [math.exp(logg[0, kv, t, sl])] * (mhi - mlo)
            keys += list(range(lo, hi))
            gains += [1.0] * (hi - lo)
            J = torch.tensor(keys)
            z = q[0, h, lo:hi] @ k[0, kv, J].T / math.sqrt(d)
            future = (J[None, :] > torch.arange(lo, hi)[:, None]) & (J[None, :] >= lo)
            z = z.masked_fill(future, -math.inf)
            out[0, h, lo:hi] = torch.softmax(z, 1) @ (v[0, kv, J] *
                                                     torch.tensor(gains, dtype=F64)[:, None])
    return out


def test_p15_outer_gating_forward_and_eq5():
    """Outer gating: the forward equals softmax(qK^T)(g V) written with torch
    ops, and dlogg_m / g_m equals the right-hand side of [picx] Eq. 5,
    sum over the block's keys of p_i dO . v_i, evaluated from torch's softmax."""
    bs, n, K = 8, 40, 2
    w, x = small(seed=17, hq=2, hkv=1, n=n, d=6, bs=bs, K=K)
    q, k, v, dout = (x[n_].to(F64) for n_ in ("q", "k", "v", "dout"))
    idx, logg, lse_s = O.select_topk(x["s"].numpy().astype(np.float32), K)
    o, _ = O.attn_fwd(q, k, v, idx, logg, bs, outer=True)
    ref = _outer_reference(q, k, v, idx, logg, bs)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    gr = O.attn_bwd(q, k, v, dout, idx, logg, x["s"].numpy(), lse_s, bs, outer=True)
    T = O.n_blocks(n, bs)
    for t in range(1, T):
        lo, hi = O.block_span(t, bs, n)
        for sl, m in enumerate(idx[0, 0, t].tolist()):
            if m < 0:
                continue
            mlo, mhi = O.block_span(m, bs, n)
            # probabilities of the ungated softmax over the row's key set
            keys = [j for s2, m2 in enumerate(idx[0, 0, t].tolist()) if m2 >= 0
                    for j in range(*O.block_span(m2, bs, n))] + list(range(lo, hi))
            J = torch.tensor(keys)
            dg = 0.0
            for h in range(2):
                z = q[0, h, lo:hi] @ k[0, 0, J].T / math.sqrt(6)
                z = z.masked_fill((J[None, :] > torch.arange(lo, hi)[:, None]) & (J[None, :] >= lo),
                                  -math.inf)
                p = torch.softmax(z, 1)
                sel = (J >= mlo) & (J < mhi)
                dg += float((p[:, sel] * (dout[0, h, lo:hi] @ v[0, 0, J[sel]].T)).sum())
            assert abs(gr["dlogg"][0, 0, t, sl] / math.exp(logg[0, 0, t, sl]) - dg) <= \
                1e-10 * max(1.0, abs(dg))


def _variant_loss(x, s64, K, bs, act, outer):
    s32 = s64.astype(np.float32)
    idx, _, _ = O.select_topk(s32, K)
    T = s64.shape[2]
    logg = np.zeros(idx.shape)
    for t in range(1, T):
        lse = O.gate_normaliser(s64[0, 0, t, :t])
        for sl, m in enumerate(idx[0, 0, t]):
            if m >= 0:
                logg[0, 0, t, sl] = O.gate_log(s64[0, 0, t, m:m + 1], lse, act)[0]
    o, _ = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs, outer=outer)
    return float((o * O._np64(x["dout"])).sum()), idx, logg


@pytest.mark.parametrize("act,outer", [("sigmoid", False), ("raw", False), ("softmax", True),
                                       ("sigmoid", True)])
def test_p16_variant_finite_differences(act, outer):
    """Central differences of L in every valid score (and, for outer gating, in
    every entry of q, k, v) for the gate variants."""
    bs, n, K = 6, 20, 2
    w, x = small(seed=23, hq=2, hkv=1, n=n, d=4, bs=bs, K=K)
    x = {k_: (v_.to(F64) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in x.items()}
    s32 = x["s"].numpy().astype(np.float32).astype(np.float64)
    L0, idx, logg = _variant_loss(x, s32, K, bs, act, outer)
    lse = np.full(s32.shape[:3], -math.inf)
    for t in range(1, s32.shape[2]):
        lse[0, 0, t] = O.gate_normaliser(s32[0, 0, t, :t])
    gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx, logg, s32, lse, bs, act=act,
                    outer=outer)
    eps = 1e-6
    T = O.n_blocks(n, bs)
    for t in range(1, T):
        for m in range(t):
            sp, sm = s32.copy(), s32.copy()
            sp[0, 0, t, m] += eps
            sm[0, 0, t, m] -= eps
            lp, ip, _ = _variant_loss(x, sp, K, bs, act, outer)
            lm, im, _ = _variant_loss(x, sm, K, bs, act, outer)
            assert np.array_equal(ip, idx) and np.array_equal(im, idx)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gr["ds"][0, 0, t, m]) <= 1e-8 + 1e-6 * abs(fd), (t, m)
    if not outer:
        return
    for name in ("q", "k", "v"):
        base = x[name].clone()
        for pos in itertools.product(*[range(sz) for sz in base.shape]):
            xp = dict(x)
            tp, tm = base.clone(), base.clone()
            tp[pos] += eps
            tm[pos] -= eps
            xp[name] = tp
            lp = _variant_loss(xp, s32, K, bs, act, outer)[0]
            xp[name] = tm
            lm = _variant_loss(xp, s32, K, bs, act, outer)[0]
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gr["d" + name][pos]) <= 1e-8 + 1e-6 * abs(fd), (name, pos)


@pytest.mark.parametrize("act", ["softmax", "sigmoid", "raw"])
def test_p17_straight_through(act):
    """STE: the forward is the hard (ungated) one, and ds = J_phi(s)^T dL/dg with
    dL/dg taken by central differences of the hard forward's loss in each
    selected block's gate at g = 1, and J_phi from torch autograd."""
    bs, n, K = 6, 30, 2
    w, x = small(seed=29, hq=2, hkv=1, n=n, d=4, bs=bs, K=K)
    q, k, v, dout = (x[n_].to(F64) for n_ in ("q", "k", "v", "dout"))
    s32 = x["s"].numpy().astype(np.float32)
    idx, logg, lse_s = O.select_topk(s32, K, act=act)
    gr = O.attn_bwd(q, k, v, dout, idx, logg, s32, lse_s, bs, act=act, ste=True)
    do = O._np64(dout)
    eps = 1e-6
    phi = {"softmax": lambda z: torch.softmax(z, 0), "sigmoid": torch.sigmoid,
           "raw": torch.exp}[act]
    for t in range(1, O.n_blocks(n, bs)):
        dLdg = np.zeros(t)
        for sl, m in enumerate(idx[0, 0, t].tolist()):
            if m < 0:
                continue
            vals = []
            for sign in (1, -1):
                lg = np.zeros(idx.shape)
                lg[0, 0, t, sl] = math.log(1.0 + sign * eps)
                o, _ = O.attn_fwd(q, k, v, idx, lg, bs)
                vals.append(float((o * do).sum()))
            dLdg[m] = (vals[0] - vals[1]) / (2 * eps)
        row = torch.tensor(s32[0, 0, t, :t].astype(np.float64))
        Jm = torch.autograd.functional.jacobian(phi, row).numpy()    # [g_m, s_m']
        ref = Jm.T @ dLdg
        np.testing.assert_allclose(gr["ds"][0, 0, t, :t], ref, rtol=1e-6, atol=1e-9)
    # q, k, v gradients under ste are those of the hard forward: central
    # differences of the ungated loss in a few entries of q and v
    for name, base in (("q", q), ("v", v)):
        for pos in ((0, 0, 7, 1), (0, 1, 25, 3), (0, 0, 29, 0)):
            if name == "v":
                pos = (0, 0) + pos[2:]
            tp, tm = base.clone(), base.clone()
            tp[pos] += eps
            tm[pos] -= eps
            lp = float((O.attn_fwd(tp if name == "q" else q, k, tp if name == "v" else v, idx,
                                   None, bs)[0] * do).sum())
            lm = float((O.attn_fwd(tm if name == "q" else q, k, tm if name == "v" else v, idx,
                                   None, bs)[0] * do).sum())
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gr["d" + name][pos]) <= 1e-8 + 1e-6 * abs(fd), (name, pos)


# ---------------------------------------------------------------- P18: paged, ragged decode

def test_p18_paged_decode_equals_dense():
    """A dense cache scattered into randomly permuted pages and read back through
    its block table gives the dense cache and the dense decode, sequence by
    sequence, for a ragged batch (different lengths, one with no history)."""
    rng = np.random.default_rng(3)
    b, hq, hkv, d, bs, K = 3, 4, 2, 8, 4, 3
    lens = [29, 4, 17]
    maxb = O.n_blocks(max(lens), bs)
    q = rng.standard_normal((b, hq, d))
    kd = rng.standard_normal((b, hkv, maxb * bs, d))
    vd = rng.standard_normal((b, hkv, maxb * bs, d))
    npages = b * maxb + 5
    perm = rng.permutation(npages)[:b * maxb].reshape(b, maxb)
    kp = rng.standard_normal((npages, hkv, bs, d))    # unused pages hold other data
    vp = rng.standard_normal((npages, hkv, bs, d))
    for bb in range(b):
        for m in range(maxb):
            kp[perm[bb, m]] = kd[bb, :, m * bs:(m + 1) * bs]
            vp[perm[bb, m]] = vd[bb, :, m * bs:(m + 1) * bs]
    idx = np.full((b, hkv, K), -1)
    logg = rng.standard_normal((b, hkv, K)) - 2.0
    for bb, L in enumerate(lens):
        C = (L - 1) // bs
        for kv in range(hkv):
            sel = np.sort(rng.choice(C, size=min(K, C), replace=False)) if C else []
            idx[bb, kv, :len(sel)] = sel
    for bb, L in enumerate(lens):
        np.testing.assert_array_equal(O.gather_pages(kp, perm[bb], L, bs), kd[bb, :, :L])
    for outer in (False, True):
        o, lse = O.decode_paged(q, kp, vp, perm, lens, idx, logg, bs, outer=outer)
        for bb, L in enumerate(lens):
            od, ld = O.decode(q[bb:bb + 1], kd[bb:bb + 1, :, :L], vd[bb:bb + 1, :, :L], L,
                              idx[bb:bb + 1], logg[bb:bb + 1], bs, outer=outer)
            np.testing.assert_array_equal(o[bb], od[0])
            np.testing.assert_array_equal(lse[bb], ld[0])


# ---------------------------------------------------------------- P19: ragged training batch

def test_p19_ragged_batch():
    """A ragged batch whose sequences all have the full length is the dense
    batch, and a shorter sequence's results depend only on its own tokens:
    changing the padding (and every other sequence) leaves them unchanged, and
    its rows past the end carry no result."""
    bs, n, K = 8, 40, 2
    w, x = small(seed=41, b=2, hq=2, hkv=1, n=n, d=6, bs=bs, K=K)
    q, k, v, dout = (x[n_].to(F64) for n_ in ("q", "k", "v", "dout"))
    s = x["s"].numpy()
    full = O.ragged_train(q, k, v, dout, [n, n], K, bs, s=s)
    idx, logg, lse_s = O.select_topk(s, K)
    o, lse = O.attn_fwd(q, k, v, idx, logg, bs)
    gr = O.attn_bwd(q, k, v, dout, idx, logg, s, lse_s, bs)
    np.testing.assert_allclose(full["o"], o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(full["lse"], lse, rtol=0, atol=1e-13)
    for key in ("dq", "dk", "dv", "dlogg", "ds"):
        np.testing.assert_allclose(full[key], gr[key], rtol=0, atol=1e-12)
    lens = [n, 21]
    r1 = O.ragged_train(q, k, v, dout, lens, K, bs, standin=True)
    q2, k2, v2, d2 = (t.clone() for t in (q, k, v, dout))
    for t in (q2, k2, v2, d2):
        t[1, :, 21:] = 123.0
        t[0] = torch.randn(t[0].shape, dtype=F64)
    r2 = O.ragged_train(q2, k2, v2, d2, lens, K, bs, standin=True)
    for key in ("o", "dq", "dk", "dv"):
        np.testing.assert_array_equal(r1[key][1], r2[key][1])
    assert np.all(r1["o"][1, :, 21:] == 0) and np.all(np.isinf(r1["lse"][1, :, 21:]))
    assert np.all(r1["idx"][1, :, O.n_blocks(21, bs):] == -1)
    # and the short sequence alone is the dense method on its 21 tokens
    alone = O.ragged_train(q[1:], k[1:], v[1:], dout[1:], [21], K, bs, standin=True)
    np.testing.assert_array_equal(alone["o"][0], r1["o"][1])


# ---------------------------------------------------------------- P20: decode query pooling per KV head

def test_p20_decode_qbar_groups_the_heads_of_each_kv_head():
    """picx 'Efficiency Benefits' (GQA with per-group selection): in decode the
    selector's query summary of KV head kv is the mean of the one new token's
    G query heads that read kv, i.e. heads h with h // G == kv.  Checked with
    hkv = 3, G = 4 (a transposed grouping gives other heads) against an
    accumulation keyed by h // G, against torch's mean over each head slice,
    and against the training pool (pinned above) of a one-token sequence with
    block 1; the decode scores it gives equal the group mean of the per-head
    scores q_h . kbar (linearity)."""
    b, hkv, G, d, C = 2, 3, 4, 5, 6
    gen = torch.Generator().manual_seed(53)
    q = torch.randn(b, hkv * G, d, generator=gen, dtype=F64)
    kbar = torch.randn(b, hkv, C, d, generator=gen, dtype=F64)
    qb = O.decode_qbar(q, hkv)
    assert qb.shape == (b, hkv, 1, d)
    acc = np.zeros((b, hkv, d))
    cnt = np.zeros(hkv)
    for h in range(hkv * G):
        acc[:, h // G] += q[:, h].numpy()
        cnt[h // G] += 1
    np.testing.assert_allclose(qb[:, :, 0], acc / cnt[None, :, None], atol=1e-15)
    for kv in range(hkv):
        np.testing.assert_allclose(qb[:, kv, 0], q[:, kv * G:(kv + 1) * G].mean(dim=1).numpy(),
                                   atol=1e-15)
    np.testing.assert_allclose(qb, O.pool_queries(q[:, :, None, :], hkv, 1), atol=1e-15)
    per_head = torch.stack([(q[:, h][:, None, :] * kbar[:, h // G]).sum(-1)
                            for h in range(hkv * G)], dim=1)            # [b, hq, C]
    group_mean = per_head.reshape(b, hkv, G, C).mean(2) / math.sqrt(d)
    s = O.standin_scores(qb, kbar.numpy(), 1.0 / math.sqrt(d), C, row_offset=C)
    np.testing.assert_allclose(s[:, :, 0], group_mean.numpy(), rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- P21: outer-gated decode

@pytest.mark.parametrize("L", [64, 61])
def test_p21_outer_decode_equals_last_outer_forward_row(L):
    """Outer gating ([picx] 'Gradient Analysis' Eq. 5, right: the gate scales a
    block's values after an ungated softmax) in decode: the token at position
    L - 1 under its block's selection equals row L - 1 of the outer-gated
    forward (pinned by P15) and of the torch-written outer reference, for
    every head of two KV heads; its LSE is the ungated softmax's."""
    bs, K = 8, 3
    w, x = small(seed=59, hq=4, hkv=2, n=L, d=8, bs=bs, K=K)
    idx, logg, _ = select(x, K)
    t = (L - 1) // bs
    assert np.any(logg[:, :, t] < -1e-3)          # the gates really differ from 1
    o, lse = O.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs, outer=True)
    od, lsed = O.decode(x["q"][:, :, L - 1], x["k"], x["v"], L, idx[:, :, t], logg[:, :, t], bs,
                        outer=True)
    np.testing.assert_allclose(od, o[:, :, L - 1], atol=1e-13)
    np.testing.assert_allclose(lsed, lse[:, :, L - 1], atol=1e-13)
    q, k, v = (x[n_].to(F64) for n_ in ("q", "k", "v"))
    ref = _outer_reference(q, k, v, idx, logg, bs)
    np.testing.assert_allclose(od, ref[:, :, L - 1].numpy(), atol=1e-13)
    # the ungated LSE: torch.logsumexp over the row's selected and causal keys
    for h in range(4):
        keys = [j for m in idx[0, h // 2, t] if m >= 0 for j in range(m * bs, (m + 1) * bs)]
        keys += list(range(t * bs, L))
        z = q[0, h, L - 1] @ k[0, h // 2, keys].T / math.sqrt(8)
        assert abs(lsed[0, h] - float(torch.logsumexp(z, 0))) <= 1e-13


# ---------------------------------------------------------------- P22: per-key-block dk / dv

def test_p22_key_block_gradients_equal_the_full_backward():
    """dk, dv of one key block B_m are the sums over the row blocks whose key
    set holds B_m: the blocks that selected m and m itself on the diagonal
    ([picx] 'Gradient Analysis' Eq. 5, left; 'Kernel Design': key-side
    gradients gathered from the selecting rows).  For every key block of both
    KV heads they equal the full backward's dk, dv on that block's rows (the
    full backward is pinned by P1, P4 and P6), under inner and outer gating;
    block 1 is selected by every later row block and the last block is partial."""
    bs, K, n = 8, 2, 60
    w, x = small(seed=61, hq=4, hkv=2, n=n, d=8, bs=bs, K=K)
    T = O.n_blocks(n, bs)
    s = x["s"].clone()
    s[..., 1] += 6.0                               # block 1 wins every row that sees it
    idx, logg, lse_s = O.select_topk(s, K)
    for kv in range(2):
        assert all(1 in idx[0, kv, t].tolist() for t in range(2, T))
    scale = O.default_scale(8)
    for outer in (False, True):
        gr = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], idx, logg, s, lse_s, bs, outer=outer)
        for kv in range(2):
            for m in range(T):
                dk, dv = O.bwd_key_block(x["q"], x["k"], x["v"], x["dout"], idx, logg, bs, scale,
                                         0, kv, m, outer)
                lo, hi = O.block_span(m, bs, n)
                np.testing.assert_allclose(dk, gr["dk"][0, kv, lo:hi], atol=1e-12, rtol=0)
                np.testing.assert_allclose(dv, gr["dv"][0, kv, lo:hi], atol=1e-12, rtol=0)
