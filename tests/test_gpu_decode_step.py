"""GPU parity of the fused decode step (stand-in selection + split-K decode in
one call, C ABI sas_decode_step) against the oracle, and against the same step
taken through the separate calls (sas_block_pool, sas_select_topk, sas_decode).

Every oracle input is synthetic or made by the oracle: the pooled-key cache is
the oracle's block mean of the key cache, rounded to the kbar dtype on the CPU.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import GATE_ATOL, max_abs, say, tols

pytestmark = pytest.mark.gpu
DEV = "cuda"


def oracle_kbar(kcache, L, bs, kbar_dtype):
    """Block means of the first L cache rows (oracle), rounded to kbar_dtype."""
    C = (L - 1) // bs
    kb = O.pool_keys(kcache[:, :, :C * bs], bs) if C > 0 else \
        np.zeros(kcache.shape[:2] + (0, kcache.shape[3]))
    return torch.from_numpy(O.to_f32(kb)).to(kbar_dtype)


def oracle_step(x, kbar, L, bs, K, gated):
    """Oracle selection from the pooled query and kbar, then the oracle decode."""
    b, hq, d = x["q"].shape
    hkv = x["kcache"].shape[1]
    C = (L - 1) // bs
    qbar32 = O.to_f32(O.decode_qbar(x["q"], hkv))
    kbar32 = kbar.float().numpy()
    s = O.standin_scores(qbar32, kbar32, O.default_scale(d), C, row_offset=C) if C > 0 else \
        np.zeros((b, hkv, 1, 0), dtype=np.float32)
    idx, logg, lse_s = O.select_topk(s, K, row_offset=C, C=C)
    o, lse = O.decode(x["q"], x["kcache"], x["vcache"], L, idx[:, :, 0],
                      logg[:, :, 0] if gated else None, bs)
    return idx[:, :, 0], logg[:, :, 0], lse_s[:, :, 0], o, lse


def step_case(seed, b, hq, hkv, L, d, bs, K, dtype, kbar_dtype=torch.bfloat16, cache_len=None):
    w = synth.workload(4, batch=b, hq=hq, hkv=hkv, seqlen=L, head_dim=d, block=bs, topk=K,
                       dtype="f32" if dtype == torch.float32 else "bf16")
    x = synth.decode_inputs(w, seed=seed, cache_len=cache_len)
    return x, oracle_kbar(x["kcache"], L, bs, kbar_dtype)


def run_step(x, kbar, L, bs, K, gated, kbar_ld=None, workspace=None):
    from gated_block_sparse_scores_amd import ops
    kb = kbar.to(DEV)
    if kbar_ld is not None and kbar_ld > kb.shape[2]:   # padded kbar rows (never read)
        pad = torch.full(kb.shape[:2] + (kbar_ld - kb.shape[2], kb.shape[3]), float("nan"),
                         dtype=kb.dtype, device=DEV)
        kb = torch.cat([kb, pad], dim=2)
    if kb.shape[2] == 0:
        kb = torch.zeros(kb.shape[:2] + (1, kb.shape[3]), dtype=kb.dtype, device=DEV)
    out = ops.decode_step(x["q"].to(DEV), kb, x["kcache"].to(DEV), x["vcache"].to(DEV), L, K,
                          bs, gated=gated, workspace=workspace)
    torch.cuda.synchronize()
    return [t.cpu() for t in out]


def check_against_oracle(out, ref, dtype, C, K):
    o, lse, idx, logg, lse_s = out
    ridx, rlogg, rlse_s, ro, rlse = ref
    assert np.array_equal(idx.numpy().astype(np.int64), ridx), "Top-K indices differ"
    assert max_abs(logg, rlogg) <= GATE_ATOL
    if C > 0:
        assert max_abs(lse_s, rlse_s) <= GATE_ATOL
    else:
        assert torch.all(torch.isneginf(lse_s))
    atol, _ = tols(dtype)
    eo, el = max_abs(o, ro), max_abs(lse, rlse)
    say(f"  o {eo:.2e} lse {el:.2e}")
    assert eo <= atol and el <= atol


STEP_CASES = [
    # b, hq, hkv, L,      d,  bs, K,  dtype
    (2, 8, 2, 1000, 128, 64, 5, torch.bfloat16),        # fused, one chunk
    (1, 8, 8, 64, 128, 64, 4, torch.bfloat16),          # C = 0: current block only
    (8, 16, 8, 1500, 128, 64, 63, torch.bfloat16),      # C = 23 < K
    (8, 16, 8, 1520, 128, 64, 63, torch.bfloat16),      # 32 keys per wave, current block of 48
    (3, 5, 1, 4097, 128, 64, 64, torch.bfloat16),       # C = K = 64
    (2, 16, 2, 64 * 700 + 5, 128, 64, 31, torch.bfloat16),   # 3 chunks (odd), ragged tail
    (1, 40, 8, 64 * 2300 + 1, 128, 64, 31, torch.bfloat16),  # 9 chunks, G = 5
    (2, 8, 2, 64 * 1300 + 7, 128, 64, 64, torch.bfloat16),   # 6 chunks, K = 64: full-width folds
    (1, 4, 4, 17, 64, 16, 2, torch.float32),            # separate-call path, short history
    (2, 8, 2, 3000, 64, 16, 8, torch.float32),          # separate-call path, two-stage select
    (1, 16, 2, 3000, 128, 32, 64, torch.bfloat16),      # separate-call path (block 32)
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[str(c[:7]) for c in STEP_CASES])
def test_decode_step_vs_oracle(case):
    b, hq, hkv, L, d, bs, K, dtype = case
    C = (L - 1) // bs
    say(f"decode_step {case}")
    x, kbar = step_case(sum(case[:7]), b, hq, hkv, L, d, bs, K, dtype)
    for gated in (True, False):
        out = run_step(x, kbar, L, bs, K, gated)
        ref = oracle_step(x, kbar, L, bs, K, gated)
        say(f" gated={gated}")
        check_against_oracle(out, ref, dtype, C, K)


def test_decode_step_f32_kbar_and_padded_rows():
    """An fp32 pooled-key cache whose rows past C hold NaN (never read)."""
    b, hq, hkv, L, d, bs, K = 2, 16, 4, 64 * 300 + 9, 128, 64, 16
    x, kbar = step_case(77, b, hq, hkv, L, d, bs, K, torch.bfloat16, kbar_dtype=torch.float32)
    out = run_step(x, kbar, L, bs, K, True, kbar_ld=(L - 1) // bs + 40)
    check_against_oracle(out, oracle_step(x, kbar, L, bs, K, True), torch.bfloat16,
                         (L - 1) // bs, K)


def test_decode_step_equals_separate_calls():
    """The fused step and pool + select + decode give the same selection and
    (up to the last bits of the gate LSE) the same output."""
    from gated_block_sparse_scores_amd import ops
    for (b, hq, hkv, L, K) in [(4, 32, 8, 64 * 1023 + 1, 63), (2, 16, 2, 64 * 300 + 1, 31)]:
        say(f"fused vs separate {(b, hq, hkv, L, K)}")
        x, kbar = step_case(L, b, hq, hkv, L, 128, 64, K, torch.bfloat16)
        xd = {k_: v_.to(DEV) for k_, v_ in x.items()}
        kb = kbar.to(DEV)
        C = (L - 1) // 64
        qb = ops.block_pool(xd["q"].unsqueeze(2), 64, hq // hkv)
        idx, logg, lse_s, _ = ops.select_topk(b, hkv, 1, C, K, row_offset=C, qbar=qb, kbar=kb)
        o, lse = ops.decode(xd["q"], xd["kcache"], xd["vcache"], L, idx[:, :, 0].contiguous(),
                            logg[:, :, 0].contiguous(), 64)
        fo, flse, fidx, flogg, flse_s = ops.decode_step(xd["q"], kb, xd["kcache"], xd["vcache"],
                                                        L, K, 64)
        torch.cuda.synchronize()
        assert torch.equal(fidx.cpu(), idx[:, :, 0].cpu())
        assert max_abs(flogg.cpu(), logg[:, :, 0].cpu()) <= 2e-6
        assert max_abs(flse_s.cpu(), lse_s[:, :, 0].cpu()) <= 2e-6
        assert max_abs(fo.cpu(), o.cpu()) <= 1e-2 and max_abs(flse.cpu(), lse.cpu()) <= 1e-5


def test_decode_step_without_selection_outputs_and_workspace_reuse():
    """idx/logg/lse_s omitted; one garbage-filled workspace reused across shapes
    (the second call smaller)."""
    from gated_block_sparse_scores_amd import _lib as L_
    from gated_block_sparse_scores_amd import ops
    shapes = [(4, 32, 8, 64 * 500 + 3, 63), (1, 8, 2, 64 * 40 + 1, 7)]
    need = max(L_.sas_decode_step_workspace_size(
        ops.Shape(b, hq, hkv, Lq, 128, 64, L_.SAS_DTYPE_BF16), K) for b, hq, hkv, Lq, K in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    for i, (b, hq, hkv, Lq, K) in enumerate(shapes):
        say(f"no selection outputs, shared workspace {(b, hq, hkv, Lq, K)}")
        x, kbar = step_case(300 + i, b, hq, hkv, Lq, 128, 64, K, torch.bfloat16)
        o, lse = ops.decode_step(x["q"].to(DEV), kbar.to(DEV), x["kcache"].to(DEV),
                                 x["vcache"].to(DEV), Lq, K, 64, with_selection=False,
                                 workspace=ws)
        torch.cuda.synchronize()
        ref = oracle_step(x, kbar, Lq, 64, K, True)
        assert max_abs(o.cpu(), ref[3]) <= 2e-2 and max_abs(lse.cpu(), ref[4]) <= 2e-2


@pytest.mark.parametrize("wl", [4, 5])
def test_decode_step_workload_full(wl):
    """8 x 64K (32/8 heads, K 63) and 1 x 512K (40/8 heads, K 31): the fused step
    at full size, selection bit-exact and outputs within the bf16 bound."""
    w = synth.workload(wl)
    say(f"decode_step workload {wl}")
    x = synth.decode_inputs(w)
    L = w.seqlen
    kbar = oracle_kbar(x["kcache"], L, w.block, torch.bfloat16)
    C = (L - 1) // w.block
    for gated in (True, False):
        out = run_step(x, kbar, L, w.block, w.topk, gated)
        ref = oracle_step(x, kbar, L, w.block, w.topk, gated)
        say(f" gated={gated}")
        check_against_oracle(out, ref, torch.bfloat16, C, w.topk)
