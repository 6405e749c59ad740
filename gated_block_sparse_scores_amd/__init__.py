"""MI355X (gfx950) library for SAS gated block-sparse attention.

The computation lives in libsas.so (HIP kernels behind the C ABI of
include/sas.h); this package is its Python binding (`_lib`, same names as the
C calls) plus allocating helpers (`ops`).
"""
from . import _lib
from ._lib import (SAS_DTYPE_BF16, SAS_DTYPE_F32, SasError, Shape, sas_attn_bwd,  # noqa: F401
                   sas_attn_bwd_workspace_size, sas_attn_fwd, sas_attn_fwd_workspace_size,
                   sas_block_pool, sas_decode, sas_decode_step, sas_decode_step_workspace_size, sas_selector_bwd,
                   sas_decode_paged, sas_decode_step_paged,
                   sas_decode_workspace_size, sas_profiler_enable,
                   sas_profiler_read, sas_profiler_reset, sas_select_topk,
                   sas_select_topk_workspace_size, sas_version)
from . import ops  # noqa: F401
