"""Zero-copy MoE dispatch -> expert -> combine over a symmetric heap, on one
MI355X (gfx950).

The path runs in hand-written HIP kernels behind a C ABI (include/cco_moe.h,
built into libcco_moe.so next to this file); this package is the Python
binding.  Importing it without the built library raises ImportError.
"""
from ._capi import (  # noqa: F401
    CCO_ERR_BAD_EXPERT,
    CCO_ERR_CAPACITY,
    CCO_ERR_DISABLED,
    CCO_ERR_HEAP_FULL,
    CCO_ERR_HIP,
    CCO_ERR_INVALID_ARG,
    CCO_ERR_OUT_OF_MEMORY,
    CCO_ERR_TIMEOUT,
    CCO_ERR_TOO_LARGE,
    CCO_INFO_COPIED,
    CCO_OK,
    KERNEL_KINDS,
    LIB_PATH,
    CcoError,
    lib,
    status_string,
)
from .moe import MoE, SymHeap, device_to_host, host_to_device, required_slot_bytes  # noqa: F401
