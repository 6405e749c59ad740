"""GPU parity of the paged-cache, ragged-batch decode (sas_decode_paged,
sas_decode_step_paged) against the oracle (its per-sequence gather + decode)."""
import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import GATE_ATOL, max_abs, say, tols

pytestmark = pytest.mark.gpu
DEV = "cuda"


def paged_case(seed, lens, hq, hkv, d, bs, dtype, extra_pages=5):
    """Dense per-sequence caches (synthetic), scattered into randomly permuted
    pages; rows past each sequence's end hold NaN (never read); unused table
    entries are -1."""
    b = len(lens)
    maxlen = max(lens)
    w = synth.workload(4, batch=b, hq=hq, hkv=hkv, seqlen=maxlen, head_dim=d, block=bs,
                       dtype="f32" if dtype == torch.float32 else "bf16")
    x = synth.decode_inputs(w, seed=seed, cache_len=O.n_blocks(maxlen, bs) * bs)
    bt_ld = O.n_blocks(maxlen, bs) + 2
    nblk = [O.n_blocks(L, bs) for L in lens]
    npages = sum(nblk) + extra_pages
    rng = np.random.default_rng(seed)
    perm = rng.permutation(npages)
    table = np.full((b, bt_ld), -1, dtype=np.int32)
    kp = torch.full((npages, hkv, bs, d), float("nan"), dtype=dtype)
    vp = torch.full((npages, hkv, bs, d), float("nan"), dtype=dtype)
    pos = 0
    for bb, L in enumerate(lens):
        for m in range(nblk[bb]):
            p = int(perm[pos])
            pos += 1
            table[bb, m] = p
            rows = min(bs, L - m * bs)
            kp[p, :, :rows] = x["kcache"][bb, :, m * bs:m * bs + rows]
            vp[p, :, :rows] = x["vcache"][bb, :, m * bs:m * bs + rows]
    return x, kp, vp, table


def oracle_selection(x, lens, kbar, bs, K, act="softmax"):
    """Per-sequence stand-in selection (oracle): idx [b,hkv,K], logg, lse_s."""
    b, hkv = kbar.shape[:2]
    d = x["q"].shape[-1]
    idx = np.full((b, hkv, K), -1, dtype=np.int64)
    logg = np.zeros((b, hkv, K))
    lse_s = np.full((b, hkv), -np.inf)
    qbar32 = O.to_f32(O.decode_qbar(x["q"], hkv))
    for bb, L in enumerate(lens):
        C = (L - 1) // bs
        if C == 0:
            continue
        s = O.standin_scores(qbar32[bb:bb + 1], kbar[bb:bb + 1].float().numpy(),
                             O.default_scale(d), C, row_offset=C)
        i, lg, ls = O.select_topk(s, K, row_offset=C, C=C, act=act)
        idx[bb], logg[bb], lse_s[bb] = i[0, :, 0], lg[0, :, 0], ls[0, :, 0]
    return idx, logg, lse_s


PAGED = [
    # lens,                      hq, hkv, d,   bs, K, dtype
    ([1000, 64, 3000, 4097], 8, 2, 128, 64, 8, torch.bfloat16),
    ([300, 17, 129], 4, 4, 64, 16, 4, torch.float32),
    ([4096 * 4 + 7, 130, 65], 40, 8, 128, 64, 31, torch.bfloat16),
    # batch 8 x 8 KV heads, K 63: the grid that takes four waves of two blocks
    ([4500, 8000, 6100, 4200, 5000, 7777, 4160, 4500], 32, 8, 128, 64, 63, torch.bfloat16),
]


@pytest.mark.parametrize("case", PAGED, ids=[str(c[0]) for c in PAGED])
def test_decode_paged_vs_oracle(case):
    from gated_block_sparse_scores_amd import ops
    lens, hq, hkv, d, bs, K, dtype = case
    say(f"paged decode {case[:6]}")
    x, kp, vp, table = paged_case(len(lens) + K, lens, hq, hkv, d, bs, dtype)
    rng = np.random.default_rng(7)
    b = len(lens)
    idx = np.full((b, hkv, K), -1, dtype=np.int64)
    for bb, L in enumerate(lens):
        C = (L - 1) // bs
        for kv in range(hkv):
            sel = np.sort(rng.choice(C, size=min(K, C), replace=False)) if C else []
            idx[bb, kv, :len(sel)] = sel
    logg = rng.standard_normal((b, hkv, K)) - 2.0
    atol, _ = tols(dtype)
    xd = {k_: v_.to(DEV) for k_, v_ in x.items()}
    args = (kp.to(DEV), vp.to(DEV), torch.from_numpy(table).to(DEV),
            torch.tensor(lens, dtype=torch.int32, device=DEV))
    for gated in (True, False):
        o, lse = ops.decode_paged(xd["q"], *args, torch.from_numpy(idx.astype(np.int32)).to(DEV),
                                  torch.from_numpy(logg.astype(np.float32)).to(DEV) if gated
                                  else None, bs, max_len=max(lens))
        torch.cuda.synchronize()
        oo, ol = O.decode_paged(x["q"], kp, vp, table, lens, idx,
                                logg.astype(np.float32) if gated else None, bs)
        eo, el = max_abs(o.cpu(), oo), max_abs(lse.cpu(), ol)
        say(f"  gated={gated}: o {eo:.2e} lse {el:.2e}")
        assert eo <= atol and el <= atol


def test_decode_paged_empty_page_entry():
    """A selected block whose page number is out of range reads nothing: the
    result equals the decode without that block."""
    from gated_block_sparse_scores_amd import ops
    lens, hq, hkv, d, bs, K = [2000, 1500], 8, 2, 128, 64, 6
    x, kp, vp, table = paged_case(11, lens, hq, hkv, d, bs, torch.bfloat16)
    idx = np.array([[[1, 5, 9, 20, 25, 30]] * hkv, [[0, 2, 4, 6, 8, 10]] * hkv])
    logg = np.full((2, hkv, K), -1.5)
    bad = table.copy()
    bad[0, 9] = 10 ** 6          # out of range
    bad[1, 4] = -7
    o, lse = ops.decode_paged(x["q"].to(DEV), kp.to(DEV), vp.to(DEV),
                              torch.from_numpy(bad).to(DEV),
                              torch.tensor(lens, dtype=torch.int32, device=DEV),
                              torch.from_numpy(idx.astype(np.int32)).to(DEV),
                              torch.from_numpy(logg.astype(np.float32)).to(DEV), bs,
                              max_len=max(lens))
    torch.cuda.synchronize()
    idx_o = idx.copy()
    idx_o[0, :, 2] = -1
    idx_o[1, :, 2] = -1
    oo, ol = O.decode_paged(x["q"], kp, vp, table, lens, idx_o, logg, bs)
    assert max_abs(o.cpu(), oo) <= 2e-2 and max_abs(lse.cpu(), ol) <= 2e-2


STEP = [
    # lens,                                  hq, hkv, K
    ([1000, 64, 3000, 4097], 8, 2, 8),
    ([64 * 700 + 5, 64 * 40 + 1, 65, 64 * 1023 + 1], 32, 8, 63),
    # batch 8 x 8 KV heads, K 63: four waves of two blocks per workgroup
    ([4500, 8000, 6100, 4200, 5000, 7777, 4160, 64 * 63 + 1], 32, 8, 63),
]


@pytest.mark.parametrize("case", STEP, ids=[str(c[0]) for c in STEP])
def test_decode_step_paged_vs_oracle(case):
    """The fused step over a paged cache: every sequence ranks its own
    history; selection bit-exact, gates and outputs against the oracle."""
    from gated_block_sparse_scores_amd import ops
    lens, hq, hkv, K = case
    d, bs = 128, 64
    say(f"paged step {case}")
    x, kp, vp, table = paged_case(sum(lens) % 1000, lens, hq, hkv, d, bs, torch.bfloat16)
    b = len(lens)
    maxC = (max(lens) - 1) // bs
    kbar = torch.full((b, hkv, maxC + 3, d), float("nan"), dtype=torch.bfloat16)
    for bb, L in enumerate(lens):
        C = (L - 1) // bs
        if C:
            kbar[bb, :, :C] = torch.from_numpy(
                O.to_f32(O.pool_keys(x["kcache"][bb:bb + 1, :, :C * bs], bs)))[0].to(torch.bfloat16)
    ridx, rlogg, rlse_s = oracle_selection(x, lens, kbar, bs, K)
    atol, _ = tols(torch.bfloat16)
    for gated in (True, False):
        fo, flse, fidx, flogg, flse_s = ops.decode_step_paged(
            x["q"].to(DEV), kbar.to(DEV), kp.to(DEV), vp.to(DEV), torch.from_numpy(table).to(DEV),
            torch.tensor(lens, dtype=torch.int32, device=DEV), K, bs, max_len=max(lens),
            gated=gated)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(fidx.cpu().numpy().astype(np.int64), ridx)
        assert max_abs(flogg.cpu(), rlogg) <= GATE_ATOL
        np.testing.assert_allclose(flse_s.cpu().numpy(), rlse_s, rtol=0, atol=GATE_ATOL)
        oo, ol = O.decode_paged(x["q"], kp, vp, table, lens, ridx, rlogg if gated else None, bs)
        eo, el = max_abs(fo.cpu(), oo), max_abs(flse.cpu(), ol)
        say(f"  gated={gated}: o {eo:.2e} lse {el:.2e}")
        assert eo <= atol and el <= atol
