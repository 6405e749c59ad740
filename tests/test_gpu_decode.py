"""GPU parity of the split-K single-token decode (C ABI)."""
import numpy as np
import pytest
import torch

import synth
from oracle import sas_oracle as O
from tests._gpu_helpers import max_abs, say, tols

pytestmark = pytest.mark.gpu
DEV = "cuda"


def decode_case(seed, b, hq, hkv, L, d, bs, K, dtype, cache_len=None, gated=True):
    w = synth.workload(4, batch=b, hq=hq, hkv=hkv, seqlen=L, head_dim=d, block=bs, topk=K,
                       dtype="f32" if dtype == torch.float32 else "bf16")
    x = synth.decode_inputs(w, seed=seed, cache_len=cache_len)
    C = (L - 1) // bs
    s = synth.random_scores((b, hkv, 1, max(C, 1)), seed=seed + 3)[..., :C]
    idx, logg, _ = O.select_topk(s, K, row_offset=C, C=C)
    return x, idx, (logg if gated else None)


def run_decode(x, idx, logg, L, bs):
    from gated_block_sparse_scores_amd import ops
    idx_g = torch.from_numpy(idx[:, :, 0].astype(np.int32)).to(DEV)
    lg = None if logg is None else torch.from_numpy(logg[:, :, 0].astype(np.float32)).to(DEV)
    o, lse = ops.decode(x["q"].to(DEV), x["kcache"].to(DEV), x["vcache"].to(DEV), L, idx_g, lg,
                        bs)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


CASES = [
    # b, hq, hkv, L,    d,  bs, K
    (1, 1, 1, 256, 64, 16, 4),
    (2, 8, 2, 1000, 128, 64, 5),
    (3, 5, 1, 4097, 128, 64, 63),
    (1, 4, 4, 17, 64, 16, 2),
    (2, 8, 1, 64, 128, 64, 3),      # no history: current block only
    (1, 16, 2, 3000, 128, 32, 64),
    (4, 32, 8, 2049, 128, 64, 8),
    (8, 16, 8, 1500, 128, 64, 63),  # two blocks per workgroup; C = 23 < K: empty waves;
                                    # current block of 28 keys: its second wave is empty
    (8, 16, 8, 1520, 128, 64, 63),  # current block of 48 keys: its second wave has 16
    (1, 8, 2, 660, 128, 64, 7),     # one block per workgroup, current block of 20 keys:
                                    # the second wave has 4, the last two none
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_small(case, dtype):
    b, hq, hkv, L, d, bs, K = case
    say(f"decode {case} {dtype}")
    for gated in (True, False):
        x, idx, logg = decode_case(sum(case), b, hq, hkv, L, d, bs, K, dtype, gated=gated)
        o, lse = run_decode(x, idx, logg, L, bs)
        oo, ol = O.decode(x["q"], x["kcache"], x["vcache"], L, idx[:, :, 0],
                          None if logg is None else logg[:, :, 0], bs)
        atol, _ = tols(dtype)
        eo, el = max_abs(o, oo), max_abs(lse, ol)
        say(f"  gated={gated}: o {eo:.2e} lse {el:.2e}")
        assert eo <= atol and el <= atol


def test_decode_cache_longer_than_L():
    """Positions at or past L in the cache hold data that must not be read."""
    b, hq, hkv, L, d, bs, K = 2, 8, 2, 700, 128, 64, 4
    x, idx, logg = decode_case(5, b, hq, hkv, L, d, bs, K, torch.bfloat16, cache_len=1024)
    o, lse = run_decode(x, idx, logg, L, bs)
    x2 = dict(x)
    x2["kcache"] = x["kcache"].clone()
    x2["vcache"] = x["vcache"].clone()
    x2["kcache"][:, :, L:] = 1000.0
    x2["vcache"][:, :, L:] = float("nan")
    o2, lse2 = run_decode(x2, idx, logg, L, bs)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    oo, ol = O.decode(x["q"], x["kcache"], x["vcache"], L, idx[:, :, 0], logg[:, :, 0], bs)
    assert max_abs(o, oo) <= 2e-2


def test_decode_equals_forward_last_row():
    """The device decode at position N-1 equals the device forward's row N-1
    under the same selection (same keys and biases)."""
    from gated_block_sparse_scores_amd import ops
    b, hq, hkv, n, d, bs, K = 1, 8, 2, 640, 128, 64, 4
    w = synth.workload(1, batch=b, hq=hq, hkv=hkv, seqlen=n, head_dim=d, block=bs, topk=K,
                       dtype="f32")
    x = {k_: v_.to(DEV) for k_, v_ in synth.train_inputs(w, seed=9).items() if v_ is not None}
    T = n // bs
    s = synth.random_scores((b, hkv, T, T), seed=10).to(DEV)
    idx, logg, lse_s, _ = ops.select_topk(b, hkv, T, T, K, s=s)
    o, lse = ops.attn_fwd(x["q"], x["k"], x["v"], idx, logg, bs)
    od, lsed = ops.decode(x["q"][:, :, n - 1].contiguous(), x["k"], x["v"], n,
                          idx[:, :, T - 1].contiguous(), logg[:, :, T - 1].contiguous(), bs)
    torch.cuda.synchronize()
    assert max_abs(od.cpu(), o[:, :, n - 1].cpu()) <= 2e-6
    assert max_abs(lsed.cpu(), lse[:, :, n - 1].cpu()) <= 2e-6


@pytest.mark.parametrize("wl", [4, 5])
def test_decode_workload_full(wl):
    """8 x 64K (32/8 heads, K 63) and 1 x 512K (40/8 heads, K 31), bf16 caches.
    The selection is the oracle's (stand-in scores from the oracle's pooled query
    and pooled keys); the device selection from the same pooled keys must match
    it bit for bit, and the device decode under it must match the oracle's, with
    and without gates."""
    from gated_block_sparse_scores_amd import ops
    w = synth.workload(wl)
    say(f"decode workload {wl}")
    x = synth.decode_inputs(w)
    L = w.seqlen
    C = (L - 1) // w.block
    kbar = torch.from_numpy(O.to_f32(O.pool_keys(x["kcache"][:, :, :C * w.block], w.block)))
    kbar = kbar.to(torch.bfloat16)
    qbar32 = O.to_f32(O.decode_qbar(x["q"], w.hkv))
    s = O.standin_scores(qbar32, kbar.float().numpy(), O.default_scale(w.head_dim), C,
                         row_offset=C)
    ridx, rlogg, _ = O.select_topk(s, w.topk, row_offset=C, C=C)
    xd = {k_: v_.to(DEV) for k_, v_ in x.items()}
    qb = ops.block_pool(xd["q"].unsqueeze(2), w.block, w.group)
    idx, _, _, _ = ops.select_topk(w.batch, w.hkv, 1, C, w.topk, row_offset=C, qbar=qb,
                                   kbar=kbar.to(DEV))
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), ridx)
    idx_g = torch.from_numpy(ridx[:, :, 0].astype(np.int32)).to(DEV)
    logg_g = torch.from_numpy(rlogg[:, :, 0].astype(np.float32)).to(DEV)
    for gated in (True, False):
        o, lse = ops.decode(xd["q"], xd["kcache"], xd["vcache"], L, idx_g,
                            logg_g if gated else None, w.block)
        torch.cuda.synchronize()
        oo, ol = O.decode(x["q"], x["kcache"], x["vcache"], L, ridx[:, :, 0],
                          rlogg[:, :, 0] if gated else None, w.block)
        eo, el = max_abs(o.cpu(), oo), max_abs(lse.cpu(), ol)
        say(f"  gated={gated}: o {eo:.2e} lse {el:.2e}")
        assert eo <= 2e-2 and el <= 2e-2


def test_decode_workspace_reuse():
    """One workspace (filled with garbage first) serves consecutive calls of
    different shapes, every call matching the oracle.  Includes rows whose
    selection has -1 pads and entries that are not history (empty splits)."""
    from gated_block_sparse_scores_amd import _lib as L
    from gated_block_sparse_scores_amd import ops
    shapes = [(4, 32, 8, 4097, 128, 64, 31), (16, 16, 4, 5000, 128, 64, 63),
              (1, 8, 8, 130, 128, 64, 9)]
    ws_n = max(L.sas_decode_workspace_size(
        ops.Shape(b, hq, hkv, Lq, d, bs, L.SAS_DTYPE_BF16), K) for b, hq, hkv, Lq, d, bs, K in shapes)
    ws = torch.full((ws_n,), 0x7F, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        for i, (b, hq, hkv, Lq, d, bs, K) in enumerate(shapes):
            say(f"workspace reuse rep {rep} shape {(b, hq, hkv, Lq, d, bs, K)}")
            x, idx, logg = decode_case(100 + i, b, hq, hkv, Lq, d, bs, K, torch.bfloat16)
            if i == 1:
                idx = idx.copy()
                idx[0, 0, 0, -3:] = -1            # pads in the middle of the slot list
                idx[1, 1, 0, 0] = (Lq - 1) // bs  # an entry that is not history: ignored
            idx_g = torch.from_numpy(idx[:, :, 0].astype(np.int32)).to(DEV)
            lg = torch.from_numpy(logg[:, :, 0].astype(np.float32)).to(DEV)
            o, lse = ops.decode(x["q"].to(DEV), x["kcache"].to(DEV), x["vcache"].to(DEV), Lq,
                                idx_g, lg, bs, workspace=ws)
            torch.cuda.synchronize()
            idx_o = np.where(idx[:, :, 0] >= (Lq - 1) // bs, -1, idx[:, :, 0])  # ignored entries
            oo, ol = O.decode(x["q"], x["kcache"], x["vcache"], Lq, idx_o, logg[:, :, 0], bs)
            assert max_abs(o.cpu(), oo) <= 2e-2 and max_abs(lse.cpu(), ol) <= 2e-2
