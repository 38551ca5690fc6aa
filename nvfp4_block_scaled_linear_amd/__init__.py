"""NVFP4 block-scaled linear layer for AMD MI355X (gfx950).

The compute lives in libnvfp4.so (hand-written HIP kernels behind the C ABI of
include/nvfp4.h); this package is its thin Python binding over torch tensors.
"""
from ._binding import (  # noqa: F401
    ACT_BF16,
    ACT_BF16_QUANTIZE,
    ACT_NVFP4,
    EXPORTS,
    F_CHECK,
    FAULT_BAD_ROUTE,
    FAULT_NAN_SCALE,
    FAULT_NONFINITE,
    LIB_PATH,
    NVFP4Error,
    OUT_COMBINE,
    OUT_REUSE_GROUPING,
    OUT_ROUTES,
    OUT_SWIGLU_BF16,
    NOALLOC_SCRATCH_BYTES,
    grouped_linear,
    grouped_linear_noalloc,
    grouped_workspace_size,
    linear,
    prefetch,
    load_library,
    quantize_act,
    read_probe,
    status_string,
)
