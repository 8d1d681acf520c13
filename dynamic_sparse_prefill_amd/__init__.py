"""CRISP sparse-prefill attention for AMD Instinct MI355X (gfx950).

The computation lives in libcrisp.so (hand-written HIP kernels behind the C
ABI in include/crisp.h); this package only marshals PyTorch tensors into it.
"""
from .api import (BLOCK, FLAG_ROUTE_JSD, FLAG_VS_COVERAGE, FLAG_VS_MEDIAN, CrispError, CrispParams, Selection,
                  attn_workspace_bytes, col_capacity, crisp_dense_attn, crisp_prefill, crisp_prefill_noalloc,
                  crisp_select, noalloc_scratch_bytes,
                  crisp_prefill_varlen, crisp_sparse_attn, lib, make_shape, new_selection, new_varlen_selection,
                  select_workspace_bytes, varlen_col_capacity, varlen_workspace_bytes, workspace_bytes)

__all__ = ["BLOCK", "FLAG_ROUTE_JSD", "FLAG_VS_COVERAGE", "FLAG_VS_MEDIAN", "CrispError", "CrispParams",
           "Selection", "attn_workspace_bytes", "col_capacity", "crisp_dense_attn", "crisp_prefill",
           "crisp_prefill_noalloc", "crisp_select", "noalloc_scratch_bytes",
           "crisp_prefill_varlen", "crisp_sparse_attn", "lib", "make_shape", "new_selection", "new_varlen_selection",
           "select_workspace_bytes", "varlen_col_capacity", "varlen_workspace_bytes", "workspace_bytes"]
