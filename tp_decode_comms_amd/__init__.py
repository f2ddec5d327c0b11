"""tp_decode_comms_amd -- barrier-free fixed-order bf16 AllReduce for
tensor-parallel decode on MI355X (gfx950).

The compute path is the HIP library libtpdc_ar.so (C ABI, include/ar.h);
this package only marshals arguments to it.  There is no CPU fallback:
loading fails loudly when the library is missing.
"""
from .ar import (  # noqa: F401
    AR_ALGO_AUTO, AR_ALGO_ONESHOT, AR_ALGO_TWOSHOT,
    AR_PROTO_AUTO, AR_PROTO_LL, AR_PROTO_LL128, AR_PROTO_SENTINEL, AR_PROTO_DIRECT,
    AR_PROTO_BARRIER, AR_PROTO_ATOMIC,
    AR_SCOPE_AUTO, AR_SCOPE_DEVICE, AR_SCOPE_CROSS_XCD,
    ArError, lib, lib_path, init, destroy, allreduce, allreduce_noalloc, allreduce_f32_debug,
    allreduce_add_rmsnorm,
    add_rmsnorm, gemv, copy, flag_ping, set_options,
    set_launch, set_scope, set_staging, set_watchdog, step_end, set_sequence, set_delays, set_timestamps,
    get_status, reset,
    query, strerror, EXPORTED_SYMBOLS,
)
