"""Plain, slow, fp64 CPU oracle for SAS gated block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP library and imports nothing from it.

What it computes, and where the pages define it (page titles, then section /
equation):

  [picx]  picx.dev summary of "SAS: Simple Attention Sparsification" --
          'Theoretical Foundation' Eq. 1-3, 'Key Idea: Differentiable Continuous
          Gating' Eq. 4 and 9, 'Gradient Analysis' Eq. 5 and 6, 'Kernel Design'.
  [daiwk] "SAS: End-to-end learning of sparse attention rankings from
          language-model loss" (reproduction README) -- 'Core equations',
          'Background and main changes' (flowchart), 'Scope'.
  [evolve] "SAS: Simple Attention Sparsification via End-to-End Optimization of
          Context Ranking" (evolve.pub review) -- 'Summary', FAQ.

Per row r = (batch b, KV head kv, query block t), with valid history length C_t:
  1. scores s_m for history blocks m < C_t (given, or the mean-pool stand-in:
     pooled query block . pooled key block / sqrt(d));
  2. gate normaliser lse_s = log sum_{m<C_t} exp(s_m); log g_m = s_m - lse_s
     ([picx] Eq. 6; the current block keeps g0 = 1, i.e. bias 0, Eq. 4);
  3. I = Top-K(s): the min(K, C_t) history blocks of largest s, equal scores
     going to the lower block index, emitted in ascending order ([picx] Eq. 3);
  4. keys J_i = union of the selected blocks and the causal prefix of the
     current block; bias log g_m on block m, 0 on the current block;
  5. o_i = softmax_j(q_i . k_j * scale + bias_j) v_j, scale = 1/sqrt(d)
     ([daiwk] 'Core equations'; [picx] Eq. 9);
  6. gradients of L = sum dO . o: dq, dk, dv, d(log g) summed per selected block
     ([picx] Eq. 5, inner gating), and ds through the gate softmax of step 2;
  7. decode: the same for a single query token at position L - 1;
  8. the selector's own backward for the stand-in scores: ds to the pooled
     summaries (dqbar, dkbar), and through the mean pools to dq and dk;
  9. ragged batches: each sequence of a padded batch is the dense method on
     its own tokens (training), or decodes at its own length over a paged cache.

Gate variants (the ablation axes of [alanhou] / [cctest] Table 1; [picx] Eq. 4
and 5): the activation phi of Eq. 4 is "softmax" (Eq. 6, the method), "sigmoid"
(g = sigmoid(s)) or "raw" (log g = s, the raw selector logit); "outer" gating
applies g after the softmax, o = sum_j p_j g_m(j) v_j with p ungated (the
gradient on the right of Eq. 5); "ste" is hard gating with a straight-through
backward: the forward is ungated (g = 1 on the selected blocks) and ds is the
soft phi's Jacobian applied to dL/dg taken at g = 1.

Readings taken where the pages leave a step open: the gate softmax runs over
all C_t history blocks of the row (not only the selected ones); the 1/sqrt(d)
scale multiplies q . k only, never the log gate; Top-K ranks s (ties to the
lower block index, -0.0 == +0.0) and takes all C_t blocks when K >= C_t; the
current block is token-causal and selected blocks are fully visible; one
selection per (batch, KV head, query block) is shared by the block's rows and
the KV head's G query heads; a decode query sits at position L - 1 of a cache
of valid length L, its current block being (L - 1) / bs.

Arithmetic: float64 throughout, except where a floating-point value decides an
integer (the Top-K ranking): that decision is taken on fp32 scores, the
precision the scores are stored in, exactly as the device library takes it.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch


# --------------------------------------------------------------------------- helpers

def _np64(x) -> np.ndarray:
    """Any torch tensor (incl. bf16) or array-like -> float64 numpy array."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _rows(x, J: np.ndarray) -> np.ndarray:
    """x[J] along the first axis as float64 (x a torch tensor or an array)."""
    if isinstance(x, torch.Tensor):
        return _np64(x[torch.from_numpy(np.asarray(J, dtype=np.int64))])
    return _np64(np.asarray(x)[J])


def _npint(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def n_blocks(n: int, bs: int) -> int:
    return -(-n // bs)


def block_span(m: int, bs: int, n: int):
    """Token range [lo, hi) of block B_m; the last block may be partial."""
    return m * bs, min((m + 1) * bs, n)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to fp32 (round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> torch.Tensor:
    """fp32 -> bf16 with round to nearest even (torch's conversion)."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)


# --------------------------------------------------------------------------- (1) scores

def pool_keys(k, bs: int) -> np.ndarray:
    """kbar[b,kv,m] = mean of k over the valid tokens of block B_m (float64).

    Stand-in for the pages' "pooling-based block summaries" ([evolve] FAQ)."""
    k = _np64(k)
    b, hkv, n, d = k.shape
    out = np.empty((b, hkv, n_blocks(n, bs), d))
    for m in range(out.shape[2]):
        lo, hi = block_span(m, bs, n)
        out[:, :, m] = k[:, :, lo:hi].mean(axis=2)
    return out


def pool_queries(q, hkv: int, bs: int) -> np.ndarray:
    """qbar[b,kv,t] = mean of q over the G query heads of KV head kv and over the
    valid tokens of query block t (float64)."""
    q = _np64(q)
    b, hq, n, d = q.shape
    g = hq // hkv
    out = np.empty((b, hkv, n_blocks(n, bs), d))
    for kv in range(hkv):
        heads = q[:, kv * g:(kv + 1) * g]
        for t in range(out.shape[2]):
            lo, hi = block_span(t, bs, n)
            out[:, kv, t] = heads[:, :, lo:hi].mean(axis=(1, 2))
    return out


def history_len(t: int, row_offset: int, C: int) -> int:
    """Valid history length of row t: C_t = min(t + row_offset, C)."""
    return min(t + row_offset, C)


def standin_scores(qbar32: np.ndarray, kbar32: np.ndarray, scale: float,
                   C: int, row_offset: int = 0) -> np.ndarray:
    """s[b,kv,t,m] = (qbar . kbar) * scale for m < C_t, rounded to fp32; 0 elsewhere.

    qbar32 [b,kv,T,d] and kbar32 [b,kv,>=C,d] are the fp32 pooled summaries; the
    dot product is evaluated in float64 and rounded once to fp32."""
    qb = np.asarray(qbar32, dtype=np.float64)
    kb = np.asarray(kbar32, dtype=np.float64)[:, :, :C]
    b, hkv, T, _ = qb.shape
    s = np.zeros((b, hkv, T, C), dtype=np.float32)
    for t in range(T):
        ct = history_len(t, row_offset, C)
        if ct == 0:
            continue
        dots = np.einsum("bkd,bkmd->bkm", qb[:, :, t], kb[:, :, :ct])
        s[:, :, t, :ct] = to_f32(dots * scale)
    return s


# --------------------------------------------------------------------------- (2)+(3) gates, Top-K

def gate_normaliser(s_row: np.ndarray) -> float:
    """lse_s = log sum_m exp(s_m) over the valid history, shifted by the max."""
    s_row = np.asarray(s_row, dtype=np.float64)
    if s_row.size == 0:
        return -math.inf
    if not np.all(np.isfinite(s_row)):
        raise ValueError("selector scores must be finite on the valid history")
    mx = s_row.max()
    return float(mx + math.log(np.exp(s_row - mx).sum()))


ACTIVATIONS = ("softmax", "sigmoid", "raw")


def gate_log(s_vals, lse: float, act: str = "softmax") -> np.ndarray:
    """log g_m of history blocks under the gate activation phi ([picx] Eq. 4):
    softmax: s_m - LSE(s) (Eq. 6); sigmoid: log sigmoid(s_m); raw: s_m."""
    s_vals = np.asarray(s_vals, dtype=np.float64)
    if act == "softmax":
        return s_vals - lse
    if act == "sigmoid":
        return -np.logaddexp(0.0, -s_vals)
    if act == "raw":
        return s_vals.copy()
    raise ValueError(f"unknown gate activation {act!r}")


def gate_values(s_vals, lse: float, act: str = "softmax") -> np.ndarray:
    """g_m = phi(s)_m for history blocks (exp of gate_log)."""
    return np.exp(gate_log(s_vals, lse, act))


def topk_history(s_row32: np.ndarray, K: int) -> np.ndarray:
    """Indices of the min(K, C) largest scores, ranked by (score descending,
    index ascending), returned in ascending index order.

    The comparison is on the fp32 values (equal fp32 values tie; -0.0 == +0.0)."""
    s_row = np.asarray(s_row32, dtype=np.float32).astype(np.float64)
    C = s_row.size
    if C == 0 or K <= 0:
        return np.zeros(0, dtype=np.int64)
    # lexsort: last key is primary.  -s ascending == s descending; ties -> index.
    order = np.lexsort((np.arange(C), -s_row))
    return np.sort(order[:min(K, C)])


def select_topk(s, K: int, row_offset: int = 0, C: Optional[int] = None, act: str = "softmax"):
    """Selection for every row of s [b,kv,T,>=C] (fp32 values).

    Returns idx int64 [b,kv,T,K] (ascending, -1 padded), logg float64
    [b,kv,T,K] (log g of the selected blocks under `act`, 0 on pads) and lse_s
    float64 [b,kv,T] (the LSE of the row's history scores, -inf when C_t = 0).
    phi is monotone for every activation, so the selection does not depend on it."""
    s = np.asarray(s.detach().cpu().numpy() if isinstance(s, torch.Tensor) else s,
                   dtype=np.float32)
    b, hkv, T = s.shape[:3]
    C = s.shape[3] if C is None else C
    idx = np.full((b, hkv, T, K), -1, dtype=np.int64)
    logg = np.zeros((b, hkv, T, K))
    lse_s = np.full((b, hkv, T), -math.inf)
    for bb in range(b):
        for kv in range(hkv):
            for t in range(T):
                ct = history_len(t, row_offset, C)
                if ct == 0:
                    continue
                row = s[bb, kv, t, :ct]
                lse = gate_normaliser(row)
                sel = topk_history(row, K)
                lse_s[bb, kv, t] = lse
                idx[bb, kv, t, :sel.size] = sel
                logg[bb, kv, t, :sel.size] = gate_log(row[sel].astype(np.float64), lse, act)
    return idx, logg, lse_s


# --------------------------------------------------------------------------- (4)+(5) forward

def key_set(t: int, idx_row, logg_row, bs: int, n: int, last_pos: Optional[int] = None):
    """Key positions, biases and causal limits seen by query block t.

    Returns (J, bias, slot, cur) where J are token positions (selected history
    blocks in ascending block order, then the current block B_t), bias is the
    log-gate of each key (0 on the current block, and 0 everywhere when
    logg_row is None), slot[j] is the Top-K slot of the key's block (-1 for the
    current block) and cur marks keys of the current block (to be causally
    masked against the query position)."""
    J, bias, slot, cur = [], [], [], []
    for sl, m in enumerate(np.asarray(idx_row).tolist()):
        if m < 0:
            continue
        if m >= t:
            raise ValueError(f"selected block {m} is not history of block {t}")
        lo, hi = block_span(m, bs, n)
        J.extend(range(lo, hi))
        bias.extend([0.0 if logg_row is None else float(logg_row[sl])] * (hi - lo))
        slot.extend([sl] * (hi - lo))
        cur.extend([False] * (hi - lo))
    lo, hi = block_span(t, bs, n)
    if last_pos is not None:
        hi = min(hi, last_pos + 1)
    J.extend(range(lo, hi))
    bias.extend([0.0] * (hi - lo))
    slot.extend([-1] * (hi - lo))
    cur.extend([True] * (hi - lo))
    return (np.asarray(J, dtype=np.int64), np.asarray(bias), np.asarray(slot, dtype=np.int64),
            np.asarray(cur, dtype=bool))


def _logits(qrows, pos, kj, J, bias, cur, scale):
    """z[i, j] = q_i . k_j * scale + bias_j, -inf where a current-block key lies
    after the query position."""
    z = (qrows @ kj.T) * scale + bias[None, :]
    future = cur[None, :] & (J[None, :] > pos[:, None])
    return np.where(future, -np.inf, z)


def _softmax_stats(z):
    mx = z.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(z - mx).sum(axis=1))
    p = np.exp(z - lse[:, None])
    return p, lse


def fwd_row_block(q, k, v, idx, logg, bs: int, scale: float, bb: int, kv: int, t: int,
                  outer: bool = False):
    """Forward of one row block: (o [G,rows,d], lse [G,rows], P list, J data).
    With outer gating the logits carry no bias and each key's value is scaled by
    its block's gate g = exp(log g) after the softmax; P and LSE are ungated."""
    hq, n = q.shape[1], q.shape[2]
    g = hq // k.shape[1]
    idx_row = _npint(idx[bb, kv, t])
    logg_row = None if logg is None else _np64(logg[bb, kv, t])
    J, bias, slot, cur = key_set(t, idx_row, logg_row, bs, n)
    kj = _rows(k[bb, kv], J)
    vj = _rows(v[bb, kv], J)
    lo, hi = block_span(t, bs, n)
    pos = np.arange(lo, hi)
    os_, lses, ps = [], [], []
    zbias = np.zeros_like(bias) if outer else bias
    vg = vj * np.exp(bias)[:, None] if outer else vj
    for h in range(kv * g, (kv + 1) * g):
        z = _logits(_np64(q[bb, h, lo:hi]), pos, kj, J, zbias, cur, scale)
        p, lse = _softmax_stats(z)
        os_.append(p @ vg)
        lses.append(lse)
        ps.append(p)
    return np.stack(os_), np.stack(lses), ps, (J, bias, slot, cur, kj, vj)


def attn_fwd(q, k, v, idx, logg, bs: int, scale: Optional[float] = None, outer: bool = False):
    """o [b,hq,N,d] and LSE [b,hq,N] (float64) of gated block-sparse attention
    (inner gating, Eq. 9; or outer gating)."""
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = default_scale(d) if scale is None else scale
    o = np.zeros((b, hq, n, d))
    lse = np.zeros((b, hq, n))
    for bb in range(b):
        for kv in range(hkv):
            for t in range(n_blocks(n, bs)):
                lo, hi = block_span(t, bs, n)
                ob, lb, _, _ = fwd_row_block(q, k, v, idx, logg, bs, scale, bb, kv, t, outer)
                o[bb, kv * g:(kv + 1) * g, lo:hi] = ob
                lse[bb, kv * g:(kv + 1) * g, lo:hi] = lb
    return o, lse


def attn_fwd_dense(q, k, v, idx, logg, bs: int, scale: Optional[float] = None):
    """Second formulation for small inputs: materialise the whole N x N logit
    matrix, put log g on selected history blocks, 0 on the causal part of the
    current block and -inf everywhere else, then take a row softmax
    ([picx] 'Kernel Design': masking non-selected blocks; [daiwk] 'Scope':
    a dense-materialised reference)."""
    q, k, v = _np64(q), _np64(k), _np64(v)
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = default_scale(d) if scale is None else scale
    idx = _npint(idx)
    logg = None if logg is None else _np64(logg)
    T = n_blocks(n, bs)
    o = np.zeros_like(q)
    lse = np.zeros((b, hq, n))
    for bb in range(b):
        for kv in range(hkv):
            bias = np.full((n, n), -np.inf)
            for t in range(T):
                lo, hi = block_span(t, bs, n)
                for sl in range(idx.shape[3]):
                    m = idx[bb, kv, t, sl]
                    if m < 0:
                        continue
                    mlo, mhi = block_span(m, bs, n)
                    bias[lo:hi, mlo:mhi] = 0.0 if logg is None else logg[bb, kv, t, sl]
                for i in range(lo, hi):
                    bias[i, lo:i + 1] = 0.0
            for h in range(kv * g, (kv + 1) * g):
                z = q[bb, h] @ k[bb, kv].T * scale + bias
                p, l = _softmax_stats(z)
                o[bb, h] = p @ v[bb, kv]
                lse[bb, h] = l
    return o, lse


# --------------------------------------------------------------------------- (6) backward

def bwd_row_block(q, k, v, dout, idx, logg, bs: int, scale: float, bb: int, kv: int, t: int,
                  outer: bool = False):
    """Backward of one row block for L = sum dO . o.

    Returns dq [G,rows,d], dlogg [K] (dL/d(log g_m): with inner gating the sum
    of dS over each selected block, all G heads and all rows of the block; with
    outer gating g_m times dL/dg_m = sum p dO . v over the block, Eq. 5 right),
    and the key-side contributions (J, dk_J, dv_J) to be summed over row blocks."""
    o, lse, ps, (J, bias, slot, cur, kj, vj) = fwd_row_block(q, k, v, idx, logg, bs, scale,
                                                             bb, kv, t, outer)
    mult = np.exp(bias) if outer else np.ones_like(bias)   # value scale per key
    hq, n = q.shape[1], q.shape[2]
    g = hq // k.shape[1]
    K = idx.shape[3]
    lo, hi = block_span(t, bs, n)
    dq = np.zeros((g, hi - lo, kj.shape[1]))
    dk_j = np.zeros_like(kj)
    dv_j = np.zeros_like(vj)
    dlogg = np.zeros(K)
    for gi, h in enumerate(range(kv * g, (kv + 1) * g)):
        p = ps[gi]
        do = _np64(dout[bb, h, lo:hi])
        qh = _np64(q[bb, h, lo:hi])
        D = (do * o[gi]).sum(axis=1)                  # D_i = dO_i . o_i
        dp = (do @ vj.T) * mult[None, :]              # dP_ij = dO_i . (g v_j)
        ds_ = p * (dp - D[:, None])                   # dS_ij = p_ij (dP_ij - D_i)
        dq[gi] = (ds_ @ kj) * scale
        dk_j += (ds_.T @ qh) * scale
        dv_j += (p.T @ do) * mult[:, None]
        col = (p * dp).sum(axis=0) if outer else ds_.sum(axis=0)
        for sl in range(K):
            dlogg[sl] += col[slot == sl].sum()
    return dq, dlogg, (J, dk_j, dv_j)


def ds_row(s_row, lse_s: float, idx_row, dlogg_row, act: str = "softmax",
           ste: bool = False) -> np.ndarray:
    """Selector gradient over the whole valid history of a row, from
    dlogg_m = dL/d(log g_m) at the selected blocks (Top-K carries none,
    [picx] 'Theoretical Foundation'):
      softmax (Eq. 6): ds_m = 1[m in I] dlogg_m - g_m * sum_{m' in I} dlogg_{m'},
                       g_m = exp(s_m - lse_s)
      sigmoid:         ds_m = 1[m in I] dlogg_m (1 - sigmoid(s_m))
      raw:             ds_m = 1[m in I] dlogg_m
    With ste the forward was hard (g = 1), so dlogg is dL/dg there; the soft
    gate's Jacobian then acts on it, which is the same formula applied to
    g_m dlogg_m."""
    s_row = np.asarray(s_row, dtype=np.float64)
    gates = gate_values(s_row, lse_s, act)
    own = np.zeros_like(s_row)
    for sl, m in enumerate(np.asarray(idx_row).tolist()):
        if m < 0:
            continue
        own[m] += dlogg_row[sl] * (gates[m] if ste else 1.0)
    if act == "softmax":
        return own - gates * own.sum()
    if act == "sigmoid":
        return own * (1.0 - gates)
    return own


def attn_bwd(q, k, v, dout, idx, logg, s, lse_s, bs: int, scale: Optional[float] = None,
             row_offset: int = 0, act: str = "softmax", outer: bool = False, ste: bool = False):
    """All gradients: dq [b,hq,N,d], dk/dv [b,hkv,N,d], dlogg [b,kv,T,K],
    ds [b,kv,T,C] (0 where m >= C_t).  With ste the attention is the hard
    (ungated) forward whatever logg holds."""
    if ste:
        logg = None
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = default_scale(d) if scale is None else scale
    T = n_blocks(n, bs)
    K = idx.shape[3]
    s32 = np.asarray(s.detach().cpu().numpy() if isinstance(s, torch.Tensor) else s,
                     dtype=np.float32)
    C = s32.shape[3]
    lse_s = _np64(lse_s)
    dq = np.zeros((b, hq, n, d))
    dk = np.zeros((b, hkv, n, d))
    dv = np.zeros((b, hkv, n, d))
    dlogg = np.zeros((b, hkv, T, K))
    ds = np.zeros((b, hkv, T, C))
    for bb in range(b):
        for kv in range(hkv):
            for t in range(T):
                lo, hi = block_span(t, bs, n)
                dqb, dl, (J, dkj, dvj) = bwd_row_block(q, k, v, dout, idx, logg, bs, scale,
                                                       bb, kv, t, outer)
                dq[bb, kv * g:(kv + 1) * g, lo:hi] = dqb
                dk[bb, kv, J] += dkj
                dv[bb, kv, J] += dvj
                dlogg[bb, kv, t] = dl
                ct = history_len(t, row_offset, C)
                if ct > 0:
                    ds[bb, kv, t, :ct] = ds_row(s32[bb, kv, t, :ct], lse_s[bb, kv, t],
                                                _npint(idx[bb, kv, t]), dl, act, ste)
    return {"dq": dq, "dk": dk, "dv": dv, "dlogg": dlogg, "ds": ds}


def bwd_key_block(q, k, v, dout, idx, logg, bs: int, scale: float, bb: int, kv: int, m: int,
                  outer: bool = False):
    """dk, dv on the tokens of key block B_m only: the sum over every row block
    whose key set contains B_m (the blocks that selected m, and m itself)."""
    n = q.shape[2]
    T = n_blocks(n, bs)
    lo, hi = block_span(m, bs, n)
    idx_np = _npint(idx[bb, kv])
    dk = np.zeros((hi - lo, q.shape[3]))
    dv = np.zeros_like(dk)
    for t in range(m, T):
        if t != m and m not in idx_np[t].tolist():
            continue
        _, _, (J, dkj, dvj) = bwd_row_block(q, k, v, dout, idx, logg, bs, scale, bb, kv, t,
                                            outer)
        sel = (J >= lo) & (J < hi)
        dk[J[sel] - lo] += dkj[sel]
        dv[J[sel] - lo] += dvj[sel]
    return dk, dv


# --------------------------------------------------------------------------- (7) decode

def decode(q, kcache, vcache, L: int, idx, logg, bs: int, scale: Optional[float] = None,
           outer: bool = False):
    """Single-token attention at position L - 1 over the selected history blocks
    and the current block's prefix.  logg None -> ungated ([picx] Eq. 2, the
    deployed form in [evolve] 'Summary'); outer: gates scale the values after
    the softmax.  q [b,hq,d] -> o [b,hq,d], lse [b,hq]."""
    b, hq, d = q.shape
    hkv = kcache.shape[1]
    g = hq // hkv
    scale = default_scale(d) if scale is None else scale
    c = (L - 1) // bs
    o = np.zeros((b, hq, d))
    lse = np.zeros((b, hq))
    for bb in range(b):
        for kv in range(hkv):
            idx_row = _npint(idx[bb, kv])
            logg_row = None if logg is None else _np64(logg[bb, kv])
            J, bias, _, _ = key_set(c, idx_row, logg_row, bs, L, last_pos=L - 1)
            kj = _rows(kcache[bb, kv], J)
            vj = _rows(vcache[bb, kv], J)
            if outer:
                vj = vj * np.exp(bias)[:, None]
                bias = np.zeros_like(bias)
            for h in range(kv * g, (kv + 1) * g):
                z = (_np64(q[bb, h]) @ kj.T) * scale + bias
                p, l = _softmax_stats(z[None, :])
                o[bb, h] = (p @ vj)[0]
                lse[bb, h] = l[0]
    return o, lse


def gather_pages(pages, table_row, L: int, bs: int) -> np.ndarray:
    """Dense cache [hkv, L, d] (float64) of one sequence whose logical block m
    sits in page table_row[m] of pages [num_pages, hkv, bs, d] (page = block)."""
    blocks = [_np64(pages[int(table_row[m])]) for m in range(n_blocks(L, bs))]
    return np.concatenate(blocks, axis=1)[:, :L]


def decode_paged(q, kpages, vpages, block_table, seq_lens, idx, logg, bs: int,
                 scale: Optional[float] = None, outer: bool = False):
    """Decode of a ragged batch over a paged cache ([picx] 'Decode Efficiency':
    the serving setting): sequence b has its own length L_b = seq_lens[b] (new
    token at L_b - 1, C_b = (L_b - 1) // bs history blocks) and its cache is
    read through its block table.  Each sequence is exactly `decode` of its
    gathered dense cache."""
    b, hq, d = q.shape
    o = np.zeros((b, hq, d))
    lse = np.zeros((b, hq))
    for bb in range(b):
        L = int(seq_lens[bb])
        kc = gather_pages(kpages, block_table[bb], L, bs)[None]
        vc = gather_pages(vpages, block_table[bb], L, bs)[None]
        ob, lb = decode(_np64(q[bb:bb + 1]), kc, vc, L, _npint(idx[bb:bb + 1]),
                        None if logg is None else _np64(logg[bb:bb + 1]), bs, scale, outer)
        o[bb], lse[bb] = ob[0], lb[0]
    return o, lse


def decode_qbar(q, hkv: int) -> np.ndarray:
    """Decode-mode pooled query: mean over the G query heads of each KV head,
    shaped [b,kv,1,d] (float64)."""
    q = _np64(q)
    b, hq, d = q.shape
    g = hq // hkv
    return q.reshape(b, hkv, g, d).mean(axis=2)[:, :, None, :]


# --------------------------------------------------------------------------- (8) selector backward

def selector_bwd(ds, qbar, kbar, scale: float, row_offset: int = 0):
    """Gradient of the stand-in scores s[t, m] = scale * qbar[t] . kbar[m] (m < C_t)
    with respect to the pooled summaries, given ds = dL/ds:
        dqbar[t] = scale * sum_{m < C_t} ds[t, m] kbar[m]
        dkbar[m] = scale * sum_{t : m < C_t} ds[t, m] qbar[t]
    Entries of ds with m >= C_t are not part of s and are not read.
    ds [b,kv,T,C], qbar [b,kv,T,d], kbar [b,kv,>=C,d] -> dqbar [b,kv,T,d],
    dkbar [b,kv,C,d] (float64).  The selector is trained through the gates, the
    hard Top-K carrying no gradient ([picx] 'Theoretical Foundation' and 'Key
    Idea'; [evolve] FAQ for the pooled block summaries)."""
    ds = _np64(ds)
    qb = _np64(qbar)
    b, hkv, T, C = ds.shape
    kb = _np64(kbar)[:, :, :C]
    mask = np.zeros((T, C))
    for t in range(T):
        mask[t, :history_len(t, row_offset, C)] = 1.0
    dsm = ds * mask
    dqbar = scale * (dsm @ kb)
    dkbar = scale * (np.swapaxes(dsm, 2, 3) @ qb)
    return dqbar, dkbar


def pool_queries_bwd(dqbar, hq: int, n: int, bs: int) -> np.ndarray:
    """Adjoint of pool_queries: every query row i of block t and head h of group
    kv receives dqbar[kv, t] / (G * n_t), n_t the block's valid token count."""
    dqbar = _np64(dqbar)
    b, hkv, T, d = dqbar.shape
    g = hq // hkv
    dq = np.zeros((b, hq, n, d))
    for t in range(T):
        lo, hi = block_span(t, bs, n)
        share = dqbar[:, :, t] / (g * (hi - lo))          # [b, kv, d]
        for h in range(hq):
            dq[:, h, lo:hi] = share[:, h // g, None, :]
    return dq


def pool_keys_bwd(dkbar, n: int, bs: int) -> np.ndarray:
    """Adjoint of pool_keys: every key row j of block m receives dkbar[m] / n_m."""
    dkbar = _np64(dkbar)
    b, hkv, C, d = dkbar.shape
    dk = np.zeros((b, hkv, n, d))
    for m in range(C):
        lo, hi = block_span(m, bs, n)
        dk[:, :, lo:hi] = dkbar[:, :, m, None, :] / (hi - lo)
    return dk


# --------------------------------------------------------------------------- (9) ragged batches

def ragged_train(q, k, v, dout, seq_lens, K: int, bs: int, s=None, act: str = "softmax",
                 outer: bool = False, ste: bool = False, standin: bool = False):
    """A ragged training batch in the padded layout [b, h, Nmax, d]: sequence b
    is its first n_b = seq_lens[b] tokens and is exactly the dense method run on
    those alone (selection, forward, backward, ds; with standin the scores are
    the pooled stand-in of its own tokens, else s[b, :, :T_b, :T_b]).
    Rows past a sequence's end carry no result: o = 0, lse = +inf (no mass),
    every gradient 0; selection rows t >= T_b = ceil(n_b / bs) hold idx -1,
    logg 0, lse_s -inf and ds 0."""
    b, hq, n, d = q.shape
    hkv = k.shape[1]
    T = n_blocks(n, bs)
    out = {"o": np.zeros((b, hq, n, d)), "lse": np.full((b, hq, n), np.inf),
           "idx": np.full((b, hkv, T, K), -1, dtype=np.int64), "logg": np.zeros((b, hkv, T, K)),
           "lse_s": np.full((b, hkv, T), -np.inf), "s": np.zeros((b, hkv, T, T), dtype=np.float32),
           "dq": np.zeros((b, hq, n, d)), "dk": np.zeros((b, hkv, n, d)),
           "dv": np.zeros((b, hkv, n, d)), "dlogg": np.zeros((b, hkv, T, K)),
           "ds": np.zeros((b, hkv, T, T)), "qbar": np.zeros((b, hkv, T, d)),
           "kbar": np.zeros((b, hkv, T, d))}
    for bb in range(b):
        nb = int(seq_lens[bb])
        if nb == 0:
            continue
        Tb = n_blocks(nb, bs)
        qs, ks, vs, ds_ = (x[bb:bb + 1, :, :nb] for x in (q, k, v, dout))
        if standin:
            qb = to_f32(pool_queries(qs, hkv, bs))
            kb = to_f32(pool_keys(ks, bs))
            out["qbar"][bb, :, :Tb], out["kbar"][bb, :, :Tb] = qb[0], kb[0]
            sb = standin_scores(qb, kb, default_scale(d), Tb)
        else:
            sb = np.asarray(s[bb:bb + 1, :, :Tb, :Tb], dtype=np.float32)
        idx, logg, lse_s = select_topk(sb, K, act=act)
        o, lse = attn_fwd(qs, ks, vs, idx, None if ste else logg, bs, outer=outer)
        gr = attn_bwd(qs, ks, vs, ds_, idx, logg, sb, lse_s, bs, act=act, outer=outer, ste=ste)
        out["o"][bb, :, :nb], out["lse"][bb, :, :nb] = o[0], lse[0]
        out["idx"][bb, :, :Tb], out["logg"][bb, :, :Tb] = idx[0], logg[0]
        out["lse_s"][bb, :, :Tb] = lse_s[0]
        out["s"][bb, :, :Tb, :Tb] = sb[0]
        for key in ("dq", "dk", "dv"):
            out[key][bb, :, :nb] = gr[key][0]
        out["dlogg"][bb, :, :Tb] = gr["dlogg"][0]
        out["ds"][bb, :, :Tb, :Tb] = gr["ds"][0]
    return out


# --------------------------------------------------------------------------- work counts

def selected_pairs(idx, n: int, bs: int, g: int) -> int:
    """Number of (query head, query row, key) pairs attended: selected history
    blocks count fully, the current block causally."""
    idx = _npint(idx)
    b, hkv, T, _ = idx.shape
    total = 0
    for t in range(T):
        lo, hi = block_span(t, bs, n)
        rows = hi - lo
        hist = 0
        for m in idx[:, :, t].reshape(-1).tolist():
            if m >= 0:
                mlo, mhi = block_span(m, bs, n)
                hist += mhi - mlo
        total += hist * rows + b * hkv * rows * (rows + 1) // 2
    return total * g
