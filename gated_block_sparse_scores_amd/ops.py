"""Allocating wrappers over the C ABI (torch supplies device memory and streams).

Each function allocates its outputs (and workspace) with torch on the inputs'
device and calls the matching libsas entry point; nothing is computed here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L
from ._lib import Shape


def _i32(shape, dev):
    return torch.empty(shape, dtype=torch.int32, device=dev)


def _f32(shape, dev):
    return torch.empty(shape, dtype=torch.float32, device=dev)


def _lens_ptr(seq_lens) -> int:
    if seq_lens is None:
        return 0
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous()
    return seq_lens.data_ptr()


def shape_of(q: torch.Tensor, k: torch.Tensor, block: int, scale: float = 0.0,
             seqlen: Optional[int] = None, gate: int = 0, seq_lens=None) -> Shape:
    """Shape of a training call (q [b,hq,N,d], k [b,hkv,N,d]) or, with q of
    rank 3, of a decode call (seqlen = valid cache length); gate = sas_gate
    bits (_lib.gate_code)."""
    if q.dim() == 4:
        b, hq, n, d = q.shape
    else:
        b, hq, d = q.shape
        n = seqlen
    return Shape(b, hq, k.shape[1], n if seqlen is None else seqlen, d, block,
                 L.dtype_code(q.dtype), scale, gate, _lens_ptr(seq_lens))


def block_pool(x: torch.Tensor, block: int, group: int = 1,
               out_dtype: torch.dtype = torch.float32, stream=None, seq_lens=None) -> torch.Tensor:
    """Mean of x [b,H,N,d] over each block's tokens and over groups of `group`
    heads -> [b, H/group, ceil(N/block), d]."""
    b, H, n, d = x.shape
    T = -(-n // block)
    out = torch.empty((b, H // group, T, d), dtype=out_dtype, device=x.device)
    sh = Shape(b, H, H, n, d, block, L.dtype_code(x.dtype), seq_lens=_lens_ptr(seq_lens))
    L.sas_block_pool(sh, x, H, group, L.dtype_code(out_dtype), out, stream)
    return out


def select_topk(batch: int, hkv: int, T: int, C: int, K: int, *, row_offset: int = 0,
                s: Optional[torch.Tensor] = None, qbar: Optional[torch.Tensor] = None,
                kbar: Optional[torch.Tensor] = None, head_dim: int = 0, scale: float = 0.0,
                stream=None, device=None, workspace: Optional[torch.Tensor] = None,
                gate: int = 0, seq_lens=None, seqlen: int = 1, block: int = 1):
    """Returns (idx, logg, lse_s, s_used).  With s None the stand-in score from
    qbar/kbar is formed on the device and returned as s_used."""
    dev = device or (s.device if s is not None else qbar.device)
    idx = _i32((batch, hkv, T, K), dev)
    logg = _f32((batch, hkv, T, K), dev)
    lse_s = _f32((batch, hkv, T), dev)
    s_out = None
    kdt, kld = L.SAS_DTYPE_F32, 0
    if s is None:
        s_out = _f32((batch, hkv, T, C), dev)
        kdt = L.dtype_code(kbar.dtype)
        kld = kbar.shape[2]
        head_dim = qbar.shape[-1]
    # a ragged batch (seq_lens) needs the token count seqlen and the block size
    sh = Shape(batch, hkv, hkv, seqlen, head_dim or 1, block, L.SAS_DTYPE_F32, scale, gate,
               _lens_ptr(seq_lens))
    ws_n = L.sas_select_topk_workspace_size(sh, T, C, K)
    if ws_n and (workspace is None or workspace.numel() < ws_n):
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    L.sas_select_topk(sh, T, C, row_offset, K, s, qbar, kbar, kdt, kld, s_out, idx, logg, lse_s,
                      workspace if ws_n else None, ws_n, stream)
    return idx, logg, lse_s, (s if s is not None else s_out)


def attn_fwd(q, k, v, idx, logg, block: int, scale: float = 0.0, stream=None, gate: int = 0,
             seq_lens=None):
    sh = shape_of(q, k, block, scale, gate=gate, seq_lens=seq_lens)
    K = idx.shape[-1]
    o = torch.empty_like(q)
    lse = _f32(q.shape[:3], q.device)
    ws_n = L.sas_attn_fwd_workspace_size(sh, K)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    L.sas_attn_fwd(sh, K, q, k, v, idx, logg, o, lse, ws, ws_n, stream)
    return o, lse


def attn_bwd(q, k, v, o, dout, lse, idx, logg, s, lse_s, block: int, scale: float = 0.0,
             want_ds: bool = True, stream=None, workspace: Optional[torch.Tensor] = None,
             gate: int = 0, seq_lens=None):
    sh = shape_of(q, k, block, scale, gate=gate, seq_lens=seq_lens)
    K = idx.shape[-1]
    T = idx.shape[2]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    selector = logg is not None or bool(gate & L.SAS_GATE_STE)
    dlogg = _f32(idx.shape, q.device) if selector else None
    ds = _f32((q.shape[0], k.shape[1], T, T), q.device) if (want_ds and selector) else None
    ws_n = L.sas_attn_bwd_workspace_size(sh, K)
    if workspace is None or workspace.numel() < ws_n:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    L.sas_attn_bwd(sh, K, q, k, v, o, dout, lse, idx, logg, s if ds is not None else None,
                   lse_s if ds is not None else None, dq, dk, dv, dlogg, ds, workspace, ws_n,
                   stream)
    return {"dq": dq, "dk": dk, "dv": dv, "dlogg": dlogg, "ds": ds}


def decode(q, kcache, vcache, L_: int, idx, logg, block: int, scale: float = 0.0,
           stream=None, workspace: Optional[torch.Tensor] = None, gate: int = 0,
           seq_lens=None):
    """q [b,hq,d]; caches [b,hkv,cache_len,d]; idx/logg [b,hkv,K]; seq_lens
    (ragged batch) the valid length of each sequence, L_ the longest."""
    sh = shape_of(q, kcache, block, scale, seqlen=L_, gate=gate, seq_lens=seq_lens)
    K = idx.shape[-1]
    o = torch.empty_like(q)
    lse = _f32(q.shape[:2], q.device)
    ws_n = L.sas_decode_workspace_size(sh, K)
    if workspace is None or workspace.numel() < ws_n:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    L.sas_decode(sh, kcache.shape[2], K, q, kcache, vcache, idx, logg, o, lse, workspace, ws_n,
                 stream)
    return o, lse


def decode_step(q, kbar, kcache, vcache, L_: int, K: int, block: int, gated: bool = True,
                scale: float = 0.0, with_selection: bool = True, stream=None,
                workspace: Optional[torch.Tensor] = None, gate: int = 0, seq_lens=None):
    """One fused decode step with the stand-in selector: q [b,hq,d]; kbar the
    pooled-key cache [b,hkv,>=C,d]; caches [b,hkv,cache_len,d].  Returns
    (o, lse) or, with with_selection, (o, lse, idx, logg, lse_s)."""
    sh = shape_of(q, kcache, block, scale, seqlen=L_, gate=gate, seq_lens=seq_lens)
    b, hkv = kcache.shape[0], kcache.shape[1]
    o = torch.empty_like(q)
    lse = _f32(q.shape[:2], q.device)
    idx = logg = lse_s = None
    if with_selection:
        idx = _i32((b, hkv, K), q.device)
        logg = _f32((b, hkv, K), q.device)
        lse_s = _f32((b, hkv), q.device)
    ws_n = L.sas_decode_step_workspace_size(sh, K)
    if workspace is None or workspace.numel() < ws_n:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    L.sas_decode_step(sh, kcache.shape[2], K, q, kbar, L.dtype_code(kbar.dtype), kbar.shape[2],
                      kcache, vcache, gated, o, lse, idx, logg, lse_s, workspace, ws_n, stream)
    return (o, lse, idx, logg, lse_s) if with_selection else (o, lse)


def selector_bwd(ds, qbar, kbar, block: int, seqlen: int, hq: int, dq=None, dk=None,
                 scale: float = 0.0, stream=None, seq_lens=None):
    """Stand-in selector backward of training rows: ds [b,hkv,T,T], qbar/kbar
    fp32 [b,hkv,T,d] -> (dqbar, dkbar) fp32 [b,hkv,T,d]; dq [b,hq,N,d] and
    dk [b,hkv,N,d], when given, receive the mean pools' adjoints in place."""
    b, hkv, T, d = qbar.shape
    dt = dq.dtype if dq is not None else (dk.dtype if dk is not None else torch.float32)
    sh = Shape(b, hq, hkv, seqlen, d, block, L.dtype_code(dt), scale,
               seq_lens=_lens_ptr(seq_lens))
    dqbar = torch.empty_like(qbar)
    dkbar = torch.empty_like(kbar)
    L.sas_selector_bwd(sh, ds, qbar, kbar, dqbar, dkbar, dq, dk, stream)
    return dqbar, dkbar


def decode_paged(q, kpages, vpages, block_table, seq_lens, idx, logg, block: int,
                 max_len: Optional[int] = None, scale: float = 0.0, stream=None,
                 workspace: Optional[torch.Tensor] = None, gate: int = 0):
    """Ragged decode over a paged cache: q [b,hq,d]; pages [num_pages,hkv,block,d];
    block_table int32 [b,bt_ld]; seq_lens int32 [b] (device); idx/logg [b,hkv,K].
    max_len (the longest sequence) defaults to bt_ld * block."""
    b, hq, d = q.shape
    hkv = kpages.shape[1]
    K = idx.shape[-1]
    L_ = max_len if max_len is not None else block_table.shape[1] * block
    sh = Shape(b, hq, hkv, L_, d, block, L.dtype_code(q.dtype), scale, gate)
    o = torch.empty_like(q)
    lse = _f32((b, hq), q.device)
    ws_n = L.sas_decode_workspace_size(sh, K)
    if workspace is None or workspace.numel() < ws_n:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    L.sas_decode_paged(sh, K, q, kpages, vpages, kpages.shape[0], block_table,
                       block_table.shape[1], seq_lens, idx, logg, o, lse, workspace, ws_n, stream)
    return o, lse


def decode_step_paged(q, kbar, kpages, vpages, block_table, seq_lens, K: int, block: int,
                      max_len: Optional[int] = None, gated: bool = True, scale: float = 0.0,
                      with_selection: bool = True, stream=None,
                      workspace: Optional[torch.Tensor] = None, gate: int = 0):
    """Fused decode step of a ragged batch over a paged cache (kbar dense
    [b,hkv,>=C,d]).  Returns (o, lse) or (o, lse, idx, logg, lse_s)."""
    b, hq, d = q.shape
    hkv = kpages.shape[1]
    L_ = max_len if max_len is not None else block_table.shape[1] * block
    sh = Shape(b, hq, hkv, L_, d, block, L.dtype_code(q.dtype), scale, gate)
    o = torch.empty_like(q)
    lse = _f32((b, hq), q.device)
    idx = logg = lse_s = None
    if with_selection:
        idx = _i32((b, hkv, K), q.device)
        logg = _f32((b, hkv, K), q.device)
        lse_s = _f32((b, hkv), q.device)
    ws_n = L.sas_decode_step_workspace_size(sh, K)
    if workspace is None or workspace.numel() < ws_n:
        workspace = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=q.device)
    L.sas_decode_step_paged(sh, K, q, kbar, L.dtype_code(kbar.dtype), kbar.shape[2], kpages,
                            vpages, kpages.shape[0], block_table, block_table.shape[1], seq_lens,
                            gated, o, lse, idx, logg, lse_s, workspace, ws_n, stream)
    return (o, lse, idx, logg, lse_s) if with_selection else (o, lse)
