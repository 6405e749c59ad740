"""GPU parity of block scoring, gate normalisation and Top-K (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import GATE_ATOL, gpu_select_given, max_abs, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def check_select(s_cpu, K, row_offset=0, C=None):
    say(f"select s{tuple(s_cpu.shape)} K={K} row_offset={row_offset} C={C}")
    idx, logg, lse_s = gpu_select_given(s_cpu.to(DEV), K, row_offset, C)
    torch.cuda.synchronize()
    oi, ol, os_ = O.select_topk(s_cpu, K, row_offset=row_offset, C=C)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    assert max_abs(logg.cpu().numpy(), ol) <= GATE_ATOL
    lg = lse_s.cpu().numpy().astype(np.float64)
    fin = np.isfinite(os_)
    assert np.array_equal(np.isfinite(lg), fin)
    assert max_abs(lg[fin], os_[fin]) <= GATE_ATOL


def test_select_tiny_fp32_workload():
    w = synth.workload(1)
    check_select(synth.train_inputs(w)["s"], w.topk)


@pytest.mark.parametrize("T,K", [(1, 4), (5, 4), (16, 16), (33, 7), (130, 31), (200, 64),
                                 (512, 15), (300, 200), (255, 254), (700, 31), (1100, 64)])
def test_select_shapes(T, K):
    s = synth.random_scores((2, 3, T, T), seed=T * 100 + K)
    s[..., torch.ones(T, T, dtype=torch.bool).triu()] = float("nan")
    check_select(s, K)


def test_select_ties_lowest_index_and_signed_zero():
    """Quantised scores make many exact ties; the kept blocks must be the lower
    indices (picx Eq. 3 with ties to the lower block index).  -0.0 == +0.0."""
    T, K = 96, 9
    s = torch.round(synth.random_scores((1, 4, T, T), seed=5) * 2) / 2
    s[0, 1] = 0.0
    s[0, 2, :, ::2] = -0.0
    s[..., torch.ones(T, T, dtype=torch.bool).triu()] = float("nan")
    check_select(s, K)


def test_select_ties_with_several_keys_per_lane():
    """Rows of up to 399 history blocks (up to seven keys per lane of the
    one-wave selection), scores quantised so that the K-th largest value is
    shared by many blocks: the lower indices among them are kept."""
    T, K = 400, 50
    s = torch.round(synth.random_scores((1, 2, T, T), seed=11) * 4) / 4
    s[..., torch.ones(T, T, dtype=torch.bool).triu()] = float("nan")
    check_select(s, K)


def test_select_decode_mode_long_history():
    """Decode rows: T = 1, C = history blocks, row_offset = C (all visible)."""
    for C in (1, 63, 513, 1023, 8191, 16384):
        s = synth.random_scores((1, 8, 1, C), seed=C)
        check_select(s, 31, row_offset=C, C=C)
    # many exact ties across chunk boundaries
    s = torch.round(synth.random_scores((2, 4, 1, 3000), seed=7))
    check_select(s, 64, row_offset=3000, C=3000)


def test_decode_selection_fp32_pooled_keys_long():
    """Stand-in scores over an fp32 pooled-key cache with 2000 history blocks
    (chunked path), d = 64 and d = 128."""
    from gated_block_sparse_scores_amd import ops
    for d in (64, 128):
        gen = torch.Generator().manual_seed(d)
        kb = torch.randn(2, 3, 2001, d, generator=gen) * 0.1
        qb = torch.randn(2, 3, 1, d, generator=gen)
        C = 2000
        idx, logg, lse_s, s = ops.select_topk(2, 3, 1, C, 17, row_offset=C, qbar=qb.to(DEV),
                                              kbar=kb.to(DEV))
        torch.cuda.synchronize()
        so = O.standin_scores(qb.numpy(), kb.numpy(), O.default_scale(d), C, row_offset=C)
        s_gpu = s.cpu().numpy()
        assert np.sum(s_gpu != so) <= 2
        oi, ol, ols = O.select_topk(so, 17, row_offset=C, C=C)
        np.testing.assert_array_equal(idx.cpu().numpy(), oi)
        assert max_abs(logg.cpu().numpy(), ol) <= GATE_ATOL
        assert max_abs(lse_s.cpu().numpy(), ols) <= GATE_ATOL


def test_select_large_training_rows():
    w = synth.workload(3)
    gen = torch.Generator().manual_seed(3)
    T = w.nblocks
    s = torch.randn(1, 8, T, T, generator=gen) * math.sqrt(2)
    s[..., torch.ones(T, T, dtype=torch.bool).triu()] = float("nan")
    check_select(s, w.topk)


# ------------------------------------------------------------------ stand-in scorer

def pool_gpu(x, block, group, out_dtype=torch.float32):
    from gated_block_sparse_scores_amd import ops
    return ops.block_pool(x.to(DEV), block, group, out_dtype)


def test_pool_matches_oracle_bits():
    for (b, h, n, d, bs, g, dt) in [(1, 8, 200, 64, 16, 4, torch.float32),
                                    (2, 4, 130, 128, 64, 2, torch.bfloat16),
                                    (1, 32, 8192, 128, 64, 4, torch.bfloat16)]:
        say(f"pool b={b} h={h} n={n} d={d} bs={bs} g={g} {dt}")
        gen = torch.Generator().manual_seed(n)
        x = torch.randn(b, h, n, d, generator=gen).to(dt)
        out = pool_gpu(x, bs, g).cpu().numpy()
        hkv = h // g
        ref = O.to_f32(O.pool_queries(x, hkv, bs) if g > 1 else O.pool_keys(x, bs))
        diff = out.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64)
        assert np.abs(diff).max() <= 1            # at most one ulp, from fp64 summation order
        assert (diff != 0).mean() < 1e-4
        outb = pool_gpu(x, bs, g, torch.bfloat16).cpu()
        refb = O.f32_to_bf16_bits(out)  # bf16 rounding of the same fp32 values
        assert torch.equal(outb.view(torch.int16), refb.view(torch.int16))


def test_standin_training_selection_qwen3_4b_shape():
    """8K tokens, 32/8 heads, d 128, block 64, K 31: pooled q and k, fp64 dot,
    fp32 scores; Top-K decided on those fp32 scores on both sides."""
    from gated_block_sparse_scores_amd import ops
    w = synth.workload(2)
    x = synth.train_inputs(w, device=DEV)
    qb = ops.block_pool(x["q"], w.block, w.group)
    kb = ops.block_pool(x["k"], w.block, 1)
    T = w.nblocks
    idx, logg, lse_s, s = ops.select_topk(1, 8, T, T, w.topk, qbar=qb, kbar=kb)
    torch.cuda.synchronize()
    qo = O.to_f32(O.pool_queries(x["q"].cpu(), 8, w.block))
    ko = O.to_f32(O.pool_keys(x["k"].cpu(), w.block))
    so = O.standin_scores(qo, ko, O.default_scale(w.head_dim), T)
    s_gpu = s.cpu().numpy()
    say(f"stand-in scores: {np.sum(s_gpu != so)} of {so.size} differ")
    assert np.sum(s_gpu != so) <= 2
    oi, ol, ols = O.select_topk(so, w.topk)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    assert max_abs(logg.cpu().numpy(), ol) <= GATE_ATOL


@pytest.mark.parametrize("wl", [4, 5])
def test_decode_selection_pooled_keys(wl):
    """Decode selection over the pooled-key cache (bf16, rounded from fp32):
    the query is pooled over the G heads of each KV head."""
    from gated_block_sparse_scores_amd import ops
    w = synth.workload(wl)
    x = synth.decode_inputs(w, device=DEV)
    L = w.seqlen
    C = (L - 1) // w.block
    kb32 = ops.block_pool(x["kcache"], w.block, 1)
    kb16 = ops.block_pool(x["kcache"], w.block, 1, torch.bfloat16)
    qb = ops.block_pool(x["q"].unsqueeze(2), w.block, w.group)
    idx, logg, lse_s, s = ops.select_topk(w.batch, w.hkv, 1, C, w.topk, row_offset=C,
                                          qbar=qb, kbar=kb16)
    torch.cuda.synchronize()
    say(f"decode selection workload {wl}: C={C}")
    ko = O.to_f32(O.pool_keys(x["kcache"].cpu(), w.block))
    assert np.abs(kb32.cpu().numpy().view(np.int32).astype(np.int64)
                  - ko.view(np.int32).astype(np.int64)).max() <= 1
    ko16 = O.f32_to_bf16_bits(ko).to(torch.float64).numpy()
    qo = O.to_f32(O.decode_qbar(x["q"].cpu(), w.hkv))
    so = O.standin_scores(qo, ko16, O.default_scale(w.head_dim), C, row_offset=C)
    s_gpu = s.cpu().numpy()
    ndiff = np.sum(s_gpu != so)
    say(f"  scores differing: {ndiff} of {so.size}")
    assert ndiff <= 2
    oi, ol, ols = O.select_topk(so, w.topk, row_offset=C, C=C)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    assert max_abs(logg.cpu().numpy(), ol) <= GATE_ATOL
