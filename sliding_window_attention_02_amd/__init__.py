"""MI355X-native SWA(w,s) attention: prefill and ring-buffer decode (HIP kernels for gfx950).

The compute lives in libswa.so (C ABI in include/swa.h); this package is its ctypes
binding (``binding``), the seeded synthetic workloads (``inputs``), FLOP/byte accounting
(``accounting``) and the build script (``build``).
"""
from .binding import (  # noqa: F401
    ADDITIVE,
    TOTAL,
    SwaError,
    alloc_cache,
    alloc_workspace,
    cache_slots,
    append_decode_step,
    debug_decode_slots,
    debug_prefill_mask,
    decode_describe,
    decode_step,
    decode_step_noalloc,
    decode_workspace_bytes,
    kv_append,
    last_error,
    layer_decode_step,
    layer_workspace_bytes,
    linear,
    local_window,
    prefill,
    prefill_chunk,
    prefill_describe,
    rmsnorm,
    stack_decode_step,
    stack_workspace_bytes,
)
