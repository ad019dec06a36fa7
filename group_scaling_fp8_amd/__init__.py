"""MI355X (gfx950) per-group fp8 scaling: Python binding of libmgs.so.

The functions below carry the names of the C entry points in include/mgs.h
and only marshal arguments: they check torch tensors, allocate outputs the
caller did not pass, and call the library on the current HIP stream. Every
step of the computation runs in the library's HIP kernels. There is no CPU
fallback: if libmgs.so is missing, the first call raises.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    MGS_ERR_HIP, MGS_ERR_INVALID_ARG, MGS_ERR_UNSUPPORTED, MGS_FLAG_POW2_SCALE, MGS_FLAG_VALIDATE,
    MGS_MAX_GROUPS,
    MGS_MX_FLOOR, MGS_MX_RCEIL, MGS_OK, MgsError, lib, library_path,
)
from .api import (  # noqa: F401
    dim0_workspace, mgs_cast_e4m3, mgs_copy, mgs_dim0_workspace_bytes, mgs_mx_dequant_dim0,
    mgs_mx_quant_dim0, mgs_mx_quant_dim1, mgs_quant_experts_dim1, mgs_quant_groups_dim0,
    mgs_quant_groups_dim0_noalloc, mgs_quant_groups_dim0_t, mgs_quant_groups_dim1,
)
