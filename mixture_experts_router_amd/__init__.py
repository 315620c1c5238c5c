"""MI355X (gfx950) Mixture-of-Experts FFN layer: router -> top-k softmax ->
expert-grouped dispatch -> grouped GEGLU expert GEMMs -> weighted combine.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe.so in this directory).  This package only marshals arguments; every
call raises if the library is missing.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, MOE_FORWARD_STAGES, MOE_W_BF16, MOE_W_MXFP4, MOE_W_MXFP4_A4, MOE_W_NVFP4, MOE_W_NVFP4_A4,
    MoeError,
    MoeShape, NOALLOC_SCRATCH_BYTES, combine, forward, forward_noalloc, forward_shared, gemm_down, gemm_gateup, load, nvfp4_header_bytes,
    nvfp4_scale_buffer, permute, permute_workspace_bytes, route, quantize_mx, quantize_nv, route_workspace_bytes, shape,
    workspace_bytes, workspace_shared_bytes,
)
