"""ctypes binding of libsas.so: the C ABI declared in include/sas.h, same names.

Only argument marshalling happens here (tensor -> device pointer, stream ->
hipStream_t, status -> exception); every step of the computation runs in the
library's kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsas.so")

SAS_OK, SAS_ERR_INVALID_ARG, SAS_ERR_UNSUPPORTED, SAS_ERR_WORKSPACE, SAS_ERR_LAUNCH = range(5)
SAS_DTYPE_F32, SAS_DTYPE_BF16 = 0, 1
SAS_GATE_SOFTMAX, SAS_GATE_SIGMOID, SAS_GATE_RAW = 0, 1, 2
SAS_GATE_OUTER, SAS_GATE_STE = 4, 8
GATE_ACTIVATIONS = {"softmax": SAS_GATE_SOFTMAX, "sigmoid": SAS_GATE_SIGMOID,
                    "raw": SAS_GATE_RAW}


def gate_code(act: str = "softmax", outer: bool = False, ste: bool = False) -> int:
    """sas_gate bits of a variant (activation name, outer gating, straight-through)."""
    return GATE_ACTIVATIONS[act] | (SAS_GATE_OUTER if outer else 0) | (SAS_GATE_STE if ste else 0)

EXPORTED = [
    "sas_status_string", "sas_version", "sas_block_pool", "sas_select_topk_workspace_size",
    "sas_select_topk",
    "sas_attn_fwd_workspace_size", "sas_attn_fwd", "sas_attn_bwd_workspace_size",
    "sas_attn_bwd", "sas_decode_workspace_size", "sas_decode", "sas_decode_step_workspace_size",
    "sas_decode_step", "sas_decode_step_noalloc", "sas_decode_paged", "sas_decode_step_paged",
    "sas_selector_bwd",
    "sas_profiler_enable",
    "sas_profiler_reset", "sas_profiler_read",
]


class SasError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class sas_shape(C.Structure):
    _fields_ = [("batch", C.c_int), ("hq", C.c_int), ("hkv", C.c_int), ("seqlen", C.c_int),
                ("head_dim", C.c_int), ("block", C.c_int), ("dtype", C.c_int),
                ("scale", C.c_float), ("gate", C.c_int), ("seq_lens", C.c_void_p)]


class sas_kernel_time(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_longlong), ("total_ms", C.c_double)]


@dataclass(frozen=True)
class Shape:
    batch: int
    hq: int
    hkv: int
    seqlen: int
    head_dim: int
    block: int
    dtype: int = SAS_DTYPE_BF16
    scale: float = 0.0
    gate: int = 0
    seq_lens: int = 0        # device address of int32 [batch] lengths, 0 = uniform

    def c(self) -> sas_shape:
        return sas_shape(self.batch, self.hq, self.hkv, self.seqlen, self.head_dim, self.block,
                         self.dtype, self.scale, self.gate, self.seq_lens or None)


_lib = None
P = C.c_void_p


def lib():
    """Loads libsas.so (once).  Raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gated_block_sparse_scores_amd.build`")
    L = C.CDLL(LIB_PATH)
    sp = C.POINTER(sas_shape)
    L.sas_status_string.argtypes = [C.c_int]
    L.sas_status_string.restype = C.c_char_p
    L.sas_version.restype = C.c_int
    L.sas_block_pool.argtypes = [sp, P, C.c_int, C.c_int, C.c_int, P, P]
    L.sas_select_topk_workspace_size.argtypes = [sp, C.c_int, C.c_int, C.c_int]
    L.sas_select_topk_workspace_size.restype = C.c_size_t
    L.sas_select_topk.argtypes = [sp, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, C.c_int,
                                  C.c_int, P, P, P, P, P, C.c_size_t, P]
    L.sas_attn_fwd_workspace_size.argtypes = [sp, C.c_int]
    L.sas_attn_fwd_workspace_size.restype = C.c_size_t
    L.sas_attn_fwd.argtypes = [sp, C.c_int, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.sas_attn_bwd_workspace_size.argtypes = [sp, C.c_int]
    L.sas_attn_bwd_workspace_size.restype = C.c_size_t
    L.sas_attn_bwd.argtypes = [sp, C.c_int] + [P] * 16 + [C.c_size_t, P]
    L.sas_decode_workspace_size.argtypes = [sp, C.c_int]
    L.sas_decode_workspace_size.restype = C.c_size_t
    L.sas_decode.argtypes = [sp, C.c_int, C.c_int, P, P, P, P, P, P, P, P, C.c_size_t, P]
    L.sas_selector_bwd.argtypes = [sp, P, P, P, P, P, P, P, P]
    L.sas_decode_paged.argtypes = [sp, C.c_int, P, P, P, C.c_int, P, C.c_int, P, P, P, P, P, P,
                                   C.c_size_t, P]
    L.sas_decode_step_paged.argtypes = [sp, C.c_int, P, P, C.c_int, C.c_int, P, P, C.c_int, P,
                                        C.c_int, P, C.c_int, P, P, P, P, P, P, C.c_size_t, P]
    L.sas_decode_step_workspace_size.argtypes = [sp, C.c_int]
    L.sas_decode_step_workspace_size.restype = C.c_size_t
    L.sas_decode_step.argtypes = [sp, C.c_int, C.c_int, P, P, C.c_int, C.c_int, P, P, C.c_int,
                                  P, P, P, P, P, P, C.c_size_t, P]
    L.sas_decode_step_noalloc.argtypes = [sp, C.c_int, C.c_int, P, P, C.c_int, C.c_int, P, P,
                                          C.c_int, P, P, P, P, P, P]
    L.sas_profiler_enable.argtypes = [C.c_int]
    L.sas_profiler_reset.argtypes = []
    L.sas_profiler_read.argtypes = [C.POINTER(sas_kernel_time), C.c_int]
    L.sas_profiler_read.restype = C.c_int
    for name in ("sas_block_pool", "sas_select_topk", "sas_attn_fwd", "sas_attn_bwd",
                 "sas_decode", "sas_decode_step", "sas_decode_step_noalloc", "sas_decode_paged",
                 "sas_decode_step_paged",
                 "sas_selector_bwd"):
        getattr(L, name).restype = C.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().sas_status_string(status).decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libsas takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libsas takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != SAS_OK:
        raise SasError(fn, status)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return SAS_DTYPE_F32
    if dt == torch.bfloat16:
        return SAS_DTYPE_BF16
    raise ValueError(f"unsupported dtype {dt}")


# ---------------------------------------------------------------- the C ABI, same names

def sas_version() -> int:
    return lib().sas_version()


def sas_block_pool(shape: Shape, x, heads: int, group: int, out_dtype: int, out, stream=None):
    _check("sas_block_pool", lib().sas_block_pool(C.byref(shape.c()), _ptr(x), heads, group,
                                                   out_dtype, _ptr(out), _stream(stream)))


def sas_select_topk_workspace_size(shape: Shape, T: int, C_: int, K: int) -> int:
    return lib().sas_select_topk_workspace_size(C.byref(shape.c()), T, C_, K)


def sas_select_topk(shape: Shape, T: int, C_: int, row_offset: int, K: int, s, qbar, kbar,
                    kbar_dtype: int, kbar_ld: int, s_out, idx, logg, lse_s, workspace=None,
                    ws_bytes: int = 0, stream=None):
    _check("sas_select_topk", lib().sas_select_topk(
        C.byref(shape.c()), T, C_, row_offset, K, _ptr(s), _ptr(qbar), _ptr(kbar), kbar_dtype,
        kbar_ld, _ptr(s_out), _ptr(idx), _ptr(logg), _ptr(lse_s), _ptr(workspace), ws_bytes,
        _stream(stream)))


def sas_attn_fwd_workspace_size(shape: Shape, K: int) -> int:
    return lib().sas_attn_fwd_workspace_size(C.byref(shape.c()), K)


def sas_attn_fwd(shape: Shape, K: int, q, k, v, idx, logg, o, lse, workspace=None,
                 ws_bytes: int = 0, stream=None):
    _check("sas_attn_fwd", lib().sas_attn_fwd(
        C.byref(shape.c()), K, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(logg), _ptr(o),
        _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def sas_attn_bwd_workspace_size(shape: Shape, K: int) -> int:
    return lib().sas_attn_bwd_workspace_size(C.byref(shape.c()), K)


def sas_attn_bwd(shape: Shape, K: int, q, k, v, o, dout, lse, idx, logg, s, lse_s, dq, dk, dv,
                 dlogg, ds, workspace, ws_bytes: int, stream=None):
    _check("sas_attn_bwd", lib().sas_attn_bwd(
        C.byref(shape.c()), K, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
        _ptr(idx), _ptr(logg), _ptr(s), _ptr(lse_s), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlogg),
        _ptr(ds), _ptr(workspace), ws_bytes, _stream(stream)))


def sas_decode_workspace_size(shape: Shape, K: int) -> int:
    return lib().sas_decode_workspace_size(C.byref(shape.c()), K)


def sas_decode(shape: Shape, cache_len: int, K: int, q, kcache, vcache, idx, logg, o, lse,
               workspace, ws_bytes: int, stream=None):
    _check("sas_decode", lib().sas_decode(
        C.byref(shape.c()), cache_len, K, _ptr(q), _ptr(kcache), _ptr(vcache), _ptr(idx),
        _ptr(logg), _ptr(o), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def sas_decode_step_workspace_size(shape: Shape, K: int) -> int:
    return lib().sas_decode_step_workspace_size(C.byref(shape.c()), K)


def sas_decode_step(shape: Shape, cache_len: int, K: int, q, kbar, kbar_dtype: int, kbar_ld: int,
                    kcache, vcache, gated: bool, o, lse, idx, logg, lse_s, workspace,
                    ws_bytes: int, stream=None):
    _check("sas_decode_step", lib().sas_decode_step(
        C.byref(shape.c()), cache_len, K, _ptr(q), _ptr(kbar), kbar_dtype, kbar_ld, _ptr(kcache),
        _ptr(vcache), 1 if gated else 0, _ptr(o), _ptr(lse), _ptr(idx), _ptr(logg), _ptr(lse_s),
        _ptr(workspace), ws_bytes, _stream(stream)))


# Size of the static device scratch of sas_decode_step_noalloc (include/sas.h).
SAS_STATIC_SCRATCH_BYTES = 16 << 20


def sas_decode_step_noalloc(shape: Shape, cache_len: int, K: int, q, kbar, kbar_dtype: int,
                            kbar_ld: int, kcache, vcache, gated: bool, o, lse, idx, logg, lse_s,
                            stream=None):
    _check("sas_decode_step_noalloc", lib().sas_decode_step_noalloc(
        C.byref(shape.c()), cache_len, K, _ptr(q), _ptr(kbar), kbar_dtype, kbar_ld, _ptr(kcache),
        _ptr(vcache), 1 if gated else 0, _ptr(o), _ptr(lse), _ptr(idx), _ptr(logg), _ptr(lse_s),
        _stream(stream)))


def sas_decode_paged(shape: Shape, K: int, q, kpages, vpages, num_pages: int, block_table,
                     bt_ld: int, seq_lens, idx, logg, o, lse, workspace, ws_bytes: int,
                     stream=None):
    _check("sas_decode_paged", lib().sas_decode_paged(
        C.byref(shape.c()), K, _ptr(q), _ptr(kpages), _ptr(vpages), num_pages, _ptr(block_table),
        bt_ld, _ptr(seq_lens), _ptr(idx), _ptr(logg), _ptr(o), _ptr(lse), _ptr(workspace),
        ws_bytes, _stream(stream)))


def sas_decode_step_paged(shape: Shape, K: int, q, kbar, kbar_dtype: int, kbar_ld: int, kpages,
                          vpages, num_pages: int, block_table, bt_ld: int, seq_lens,
                          gated: bool, o, lse, idx, logg, lse_s, workspace, ws_bytes: int,
                          stream=None):
    _check("sas_decode_step_paged", lib().sas_decode_step_paged(
        C.byref(shape.c()), K, _ptr(q), _ptr(kbar), kbar_dtype, kbar_ld, _ptr(kpages),
        _ptr(vpages), num_pages, _ptr(block_table), bt_ld, _ptr(seq_lens), 1 if gated else 0,
        _ptr(o), _ptr(lse), _ptr(idx), _ptr(logg), _ptr(lse_s), _ptr(workspace), ws_bytes,
        _stream(stream)))


def sas_selector_bwd(shape: Shape, ds, qbar, kbar, dqbar, dkbar, dq=None, dk=None, stream=None):
    _check("sas_selector_bwd", lib().sas_selector_bwd(
        C.byref(shape.c()), _ptr(ds), _ptr(qbar), _ptr(kbar), _ptr(dqbar), _ptr(dkbar), _ptr(dq),
        _ptr(dk), _stream(stream)))


def sas_profiler_enable(on: bool = True):
    lib().sas_profiler_enable(1 if on else 0)


def sas_profiler_reset():
    lib().sas_profiler_reset()


def sas_profiler_read() -> dict:
    n = lib().sas_profiler_read(None, 0)
    arr = (sas_kernel_time * max(n, 1))()
    n = lib().sas_profiler_read(arr, n)
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}
