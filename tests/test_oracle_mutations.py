"""Plant plausible mistakes in the oracle (CPU only) and check that a pin fails.

Each mutation is applied with monkeypatch to the oracle module, one at a time;
the pins of test_oracle_pins are then run and at least one must fail."""
import numpy as np
import pytest

from oracle import sas_oracle as O
import tests.test_oracle_pins as pins


def _ds_row_no_softmax_term(s_row, lse_s, idx_row, dlogg_row, act="softmax", ste=False):
    ds = np.zeros(len(s_row))
    for sl, m in enumerate(np.asarray(idx_row).tolist()):
        if m >= 0:
            ds[m] += dlogg_row[sl]
    return ds


def _topk_ties_high_index(s_row32, K):
    s = np.asarray(s_row32, dtype=np.float32).astype(np.float64)
    C = s.size
    if C == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((-np.arange(C), -s))
    return np.sort(order[:min(K, C)])


def _gate_normaliser_selected_only(s_row):
    # softmax over the top-K only would change lse; emulate with max only
    s_row = np.asarray(s_row, dtype=np.float64)
    return float(s_row.max()) if s_row.size else -np.inf


_orig_logits = O._logits


def _logits_no_causal(qrows, pos, kj, J, bias, cur, scale):
    return (qrows @ kj.T) * scale + bias[None, :]


def _logits_bias_sign(qrows, pos, kj, J, bias, cur, scale):
    return _orig_logits(qrows, pos, kj, J, -bias, cur, scale)


def _logits_no_scale(qrows, pos, kj, J, bias, cur, scale):
    return _orig_logits(qrows, pos, kj, J, bias, cur, 1.0)


_orig_bwd_row = O.bwd_row_block


def _bwd_row_dk_unscaled(*a, **k):
    dq, dl, (J, dkj, dvj) = _orig_bwd_row(*a, **k)
    return dq, dl, (J, dkj / a[7], dvj)


_orig_selector_bwd = O.selector_bwd
_orig_pool_q_bwd = O.pool_queries_bwd


def _selector_bwd_no_scale(ds, qbar, kbar, scale, row_offset=0):
    return _orig_selector_bwd(ds, qbar, kbar, 1.0, row_offset)


def _selector_bwd_no_mask(ds, qbar, kbar, scale, row_offset=0):
    ds = O._np64(ds)
    return _orig_selector_bwd(ds, qbar, kbar, scale, row_offset=ds.shape[3])


def _selector_bwd_untransposed(ds, qbar, kbar, scale, row_offset=0):
    dq, _ = _orig_selector_bwd(ds, qbar, kbar, scale, row_offset)
    ds = O._np64(ds)
    C = ds.shape[3]
    mask = np.array([[1.0 if m < O.history_len(t, row_offset, C) else 0.0 for m in range(C)]
                     for t in range(ds.shape[2])])
    return dq, scale * ((ds * mask) @ O._np64(qbar)[:, :, :C])


def _pool_q_bwd_no_group(dqbar, hq, n, bs):
    hkv = O._np64(dqbar).shape[1]
    return _orig_pool_q_bwd(dqbar, hq, n, bs) * (hq // hkv)


_orig_ds_row = O.ds_row
_orig_fwd_row = O.fwd_row_block
_orig_gate_log = O.gate_log


def _ds_row_sigmoid_without_slope(s_row, lse_s, idx_row, dlogg_row, act="softmax", ste=False):
    return _orig_ds_row(s_row, lse_s, idx_row, dlogg_row, "raw" if act == "sigmoid" else act, ste)


def _ds_row_ste_without_gate(s_row, lse_s, idx_row, dlogg_row, act="softmax", ste=False):
    return _orig_ds_row(s_row, lse_s, idx_row, dlogg_row, act, False)


def _fwd_row_outer_ignored(*a, **k):
    if len(a) > 10:
        a = a[:10] + (False,)
    k.pop("outer", None)
    return _orig_fwd_row(*a, **k)


def _gate_log_sigmoid_as_softmax(s_vals, lse, act="softmax"):
    return _orig_gate_log(s_vals, lse, "softmax" if act == "sigmoid" else act)


_orig_decode = O.decode
_orig_key_block = O.bwd_key_block


def _decode_qbar_transposed_groups(q, hkv):
    q = O._np64(q)
    b, hq, d = q.shape
    return q.reshape(b, hq // hkv, hkv, d).mean(axis=1)[:, :, None, :]


def _decode_outer_ignored(q, kcache, vcache, L, idx, logg, bs, scale=None, outer=False):
    return _orig_decode(q, kcache, vcache, L, idx, logg, bs, scale, False)


def _key_block_without_diagonal(q, k, v, dout, idx, logg, bs, scale, bb, kv, m, outer=False):
    n = q.shape[2]
    lo, hi = O.block_span(m, bs, n)
    dk = np.zeros((hi - lo, q.shape[3]))
    dv = np.zeros_like(dk)
    idx_np = O._npint(idx[bb, kv])
    for t in range(m + 1, O.n_blocks(n, bs)):
        if m not in idx_np[t].tolist():
            continue
        _, _, (J, dkj, dvj) = O.bwd_row_block(q, k, v, dout, idx, logg, bs, scale, bb, kv, t,
                                              outer)
        sel = (J >= lo) & (J < hi)
        dk[J[sel] - lo] += dkj[sel]
        dv[J[sel] - lo] += dvj[sel]
    return dk, dv


MUTATIONS = [
    ("ds_row", _ds_row_no_softmax_term),
    ("topk_history", _topk_ties_high_index),
    ("gate_normaliser", _gate_normaliser_selected_only),
    ("_logits", _logits_no_causal),
    ("_logits", _logits_bias_sign),
    ("_logits", _logits_no_scale),
    ("bwd_row_block", _bwd_row_dk_unscaled),
    ("selector_bwd", _selector_bwd_no_scale),
    ("selector_bwd", _selector_bwd_no_mask),
    ("selector_bwd", _selector_bwd_untransposed),
    ("pool_queries_bwd", _pool_q_bwd_no_group),
    ("ds_row", _ds_row_sigmoid_without_slope),
    ("ds_row", _ds_row_ste_without_gate),
    ("fwd_row_block", _fwd_row_outer_ignored),
    ("gate_log", _gate_log_sigmoid_as_softmax),
    ("decode_qbar", _decode_qbar_transposed_groups),
    ("decode", _decode_outer_ignored),
    ("bwd_key_block", _key_block_without_diagonal),
]

PINS = [
    pins.test_p2_score_shift_invariance,
    pins.test_p3_ds_sums_to_zero,
    pins.test_p5_topk_bruteforce_with_ties,
    pins.test_p7_inner_gate_gradient_closed_form,
    pins.test_p9_dominant_gate_limit,
    pins.test_p10_gather_equals_dense_and_rows_normalise,
    lambda: pins.test_p1_single_history_block_is_dense_causal(2, 1),
    pins.test_p4_dense_scope_matches_library_softmax_and_autograd,
    pins.test_p6_finite_differences,
    pins.test_p11_standin_chain_finite_differences,
    pins.test_p12_pool_adjoints,
    pins.test_p13_selector_bwd_matches_autograd,
    pins.test_p14_gate_activations_closed_forms,
    pins.test_p15_outer_gating_forward_and_eq5,
    lambda: pins.test_p16_variant_finite_differences("sigmoid", False),
    lambda: pins.test_p16_variant_finite_differences("softmax", True),
    lambda: pins.test_p17_straight_through("softmax"),
    pins.test_p20_decode_qbar_groups_the_heads_of_each_kv_head,
    lambda: pins.test_p21_outer_decode_equals_last_outer_forward_row(61),
    pins.test_p22_key_block_gradients_equal_the_full_backward,
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            failures += 1
    assert failures > 0, f"no pin caught mutation {fn.__name__}"
