"""Stitched memory-intensive subgraphs and cross-tile GEMM epilogues on MI355X (gfx950).

The computation lives in ``libcf.so`` (hand-written HIP kernels behind the
C-ABI in ``include/cf.h``); this package is its Python binding.  Import does
not load the library; the first call does, and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    CF_EALIGN,
    CF_EHIP,
    CF_EINVAL,
    CF_EOCCUPANCY,
    CF_EUNSUPPORTED,
    CF_EWORKSPACE,
    CF_OK,
    CF_OP_GEMM_LN,
    CF_OP_GEMM_SOFTMAX,
    CF_OP_GEMM_SOFTMAX_GEMM,
    CF_OP_STITCH_LAYERNORM,
    CF_OP_STITCH_POW_BCAST_ADD,
    CF_OP_STITCH_SOFTMAX,
    CFError,
    LIB_PATH,
    Workspace,
    cf_gemm_ln,
    cf_gemm_softmax,
    cf_gemm_softmax_gemm,
    cf_graph_begin,
    cf_graph_destroy,
    cf_graph_end,
    cf_graph_launch,
    cf_stitch_layernorm,
    cf_stitch_pow_bcast_add,
    cf_stitch_softmax,
    cf_unfused_workspace_bytes,
    cf_util_copy_f32,
    cf_util_fill_f32,
    cf_workspace_bytes,
    header_functions,
    last_plan,
    lib,
    status_str,
)
