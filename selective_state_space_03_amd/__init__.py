"""MI355X (gfx950) selective-scan hot path: fused prefill scan, in-place decode
step, multi-head chunked scan and its in-place decode step, as hand-written HIP
kernels behind the C ABI of include/ssm_mi355x.h.  This package is the thin
Python binding."""
from .binding import (  # noqa: F401
    EXPORTED,
    Call,
    LIB_PATH,
    SCAN_BLOCKED,
    SsmError,
    chunk_decode_step,
    chunk_scan_fwd,
    decode_step,
    layer_fwd,
    lib,
    linear_fwd,
    scan_bwd,
    scan_fwd,
    scan_fwd_noalloc,
    set_timing_events,
)
