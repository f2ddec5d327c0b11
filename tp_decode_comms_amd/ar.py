"""ctypes binding of libtpdc_ar.so (names follow include/ar.h).

Argument marshalling only: torch tensors give device pointers and streams;
every step of the AllReduce runs in the library's HIP kernels.
"""
import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libtpdc_ar.so"

AR_OK = 0
AR_ERR_INVALID = -1
AR_ERR_NOT_INIT = -2
AR_ERR_STATE = -3
AR_ERR_OOM = -4
AR_ERR_HIP = -5
AR_ERR_TIMEOUT = -6
AR_SCOPE_AUTO, AR_SCOPE_DEVICE, AR_SCOPE_CROSS_XCD = 0, 1, 2

AR_ALGO_AUTO, AR_ALGO_ONESHOT, AR_ALGO_TWOSHOT = 0, 1, 2
AR_PROTO_AUTO, AR_PROTO_LL, AR_PROTO_LL128, AR_PROTO_SENTINEL, AR_PROTO_DIRECT = 0, 1, 2, 3, 4
AR_PROTO_BARRIER = 5
AR_PROTO_ATOMIC = 6
MAX_RANKS = 16

_c_int, _c_u32, _c_size, _c_vp = ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes), as declared in include/ar.h
_SIGS = {
    "ar_init": (_c_int, [_c_int, _c_size]),
    "ar_allreduce": (_c_int, [ctypes.POINTER(_c_vp), _c_vp, _c_size, _c_u32, _c_vp]),
    "ar_allreduce_f32_debug": (_c_int, [ctypes.POINTER(_c_vp), _c_vp, _c_size, _c_u32, _c_vp]),
    "ar_allreduce_add_rmsnorm": (_c_int, [ctypes.POINTER(_c_vp), ctypes.POINTER(_c_vp), _c_vp,
                                          ctypes.c_float, _c_vp, _c_vp, _c_size, _c_size, _c_u32,
                                          _c_vp]),
    "ar_add_rmsnorm": (_c_int, [_c_vp, ctypes.POINTER(_c_vp), _c_vp, ctypes.c_float, _c_vp, _c_vp,
                                _c_size, _c_size, _c_vp]),
    "ar_allreduce_noalloc": (_c_int, [ctypes.POINTER(_c_vp), _c_vp, _c_size, _c_int, _c_vp]),
    "ar_destroy": (_c_int, []),
    "ar_set_options": (_c_int, [_c_int, _c_int]),
    "ar_set_launch": (_c_int, [_c_int, _c_int]),
    "ar_set_scope": (_c_int, [_c_int]),
    "ar_set_staging": (_c_int, [_c_size]),
    "ar_set_watchdog": (_c_int, [_c_u32]),
    "ar_step_end": (_c_int, [_c_vp]),
    "ar_set_delays": (_c_int, [_c_vp, _c_size]),
    "ar_set_timestamps": (_c_int, [_c_vp, _c_size, _c_size, _c_int]),
    "ar_set_sequence": (_c_int, [_c_u32, _c_vp]),
    "ar_get_status": (_c_int, [ctypes.POINTER(_c_u32)]),
    "ar_reset": (_c_int, [_c_vp]),
    "ar_strerror": (ctypes.c_char_p, [_c_int]),
    "ar_last_hip_error": (_c_int, []),
    "ar_query": (ctypes.c_longlong, [_c_int, _c_size]),
    # include/ar_gemv.h (compute step of the overlap harness)
    "ar_gemv_bf16": (_c_int, [ctypes.POINTER(_c_vp), ctypes.POINTER(_c_vp), ctypes.POINTER(_c_vp),
                              _c_size, _c_size, _c_int, _c_int, _c_vp]),
    # include/ar_copy.h (the bandwidth reference)
    "ar_copy": (_c_int, [_c_vp, _c_vp, _c_size, _c_vp]),
    # include/ar_ping.h (the flag hop, the latency floor beside a graph node)
    "ar_flag_ping": (_c_int, [_c_u32, _c_int, _c_vp, _c_vp]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lock = threading.Lock()
_lib = None


class ArError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = "%s failed: %d (%s)" % (fn, code, strerror(code))
        if code == AR_ERR_HIP and _lib is not None:
            msg += " hipError=%d" % _lib.ar_last_hip_error()
        super().__init__(msg)


def lib_path():
    return os.environ.get("TPDC_AR_LIB", os.path.join(HERE, _LIB_NAME))


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    "HIP library %s is missing: build it with "
                    "`python -m tp_decode_comms_amd.build`" % path)
            # The process must run one HIP runtime: load torch's first so that
            # the library's libamdhip64 dependency binds to that same copy.
            import torch  # noqa: F401
            L = ctypes.CDLL(path)
            for name, (res, args) in _SIGS.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
        return _lib


def strerror(code):
    if _lib is None:
        return str(code)
    return _lib.ar_strerror(int(code)).decode()


def _check(fn, rc):
    if rc != AR_OK:
        raise ArError(fn, rc)
    return rc


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return t if isinstance(t, int) else t.data_ptr()


def init(n_ranks, max_elems):
    return _check("ar_init", lib().ar_init(int(n_ranks), int(max_elems)))


def destroy():
    return _check("ar_destroy", lib().ar_destroy())


def _rank_array(rank_bufs):
    ptrs = [_ptr(b) for b in rank_bufs]
    return (_c_vp * len(ptrs))(*ptrs)


def allreduce(rank_bufs, out, n, epoch, stream=None, check=True):
    """rank_bufs: N bf16 device tensors (or pointers) of >= n elements;
    out: bf16 device tensor [N, n].  Enqueued on `stream` (default: torch's
    current stream).  Returns the status code (raises unless check=False)."""
    rc = lib().ar_allreduce(_rank_array(rank_bufs), _ptr(out), int(n), int(epoch),
                            _stream_handle(stream))
    return _check("ar_allreduce", rc) if check else rc


def allreduce_noalloc(rank_bufs, out, n, stream=None, check=True):
    """The allocation-free AllReduce (no ar_init needed): rank_bufs N bf16
    device tensors, out bf16 [N, n]; n == 0 re-arms the device's inboxes."""
    rc = lib().ar_allreduce_noalloc(_rank_array(rank_bufs), _ptr(out) if out is not None else None,
                                    int(n), len(rank_bufs), _stream_handle(stream))
    return _check("ar_allreduce_noalloc", rc) if check else rc


def allreduce_add_rmsnorm(rank_bufs, residuals, gamma, eps, out_h, out_y, rows, hidden, epoch,
                          stream=None, check=True):
    """AllReduce with the residual add and RMS norm fused behind it:
    residuals N bf16 device tensors [rows*hidden], gamma bf16 [hidden],
    out_h / out_y bf16 [N, rows*hidden].  Takes the next epoch like allreduce."""
    rc = lib().ar_allreduce_add_rmsnorm(_rank_array(rank_bufs), _rank_array(residuals),
                                        _ptr(gamma), float(eps), _ptr(out_h), _ptr(out_y),
                                        int(rows), int(hidden), int(epoch), _stream_handle(stream))
    return _check("ar_allreduce_add_rmsnorm", rc) if check else rc


def add_rmsnorm(a, residuals, gamma, eps, out_h, out_y, rows, hidden, stream=None, check=True):
    """The same residual add and RMS norm as a kernel of its own, on an
    AllReduce result a [N, rows*hidden] already in memory."""
    rc = lib().ar_add_rmsnorm(_ptr(a), _rank_array(residuals), _ptr(gamma), float(eps),
                              _ptr(out_h), _ptr(out_y), int(rows), int(hidden),
                              _stream_handle(stream))
    return _check("ar_add_rmsnorm", rc) if check else rc


def gemv(weights, xs, ys, M, K, stream=None, max_workgroups=0, check=True):
    """y_r = W_r x_r for every rank: weights N bf16 device tensors [M, K],
    xs N bf16 [K], ys N bf16 [M] (include/ar_gemv.h)."""
    rc = lib().ar_gemv_bf16(_rank_array(weights), _rank_array(xs), _rank_array(ys), int(M), int(K),
                            len(weights), int(max_workgroups), _stream_handle(stream))
    return _check("ar_gemv_bf16", rc) if check else rc


def copy(src, dst, nbytes, stream=None, check=True):
    """dst[0:nbytes) = src[0:nbytes) on the device (include/ar_copy.h): the
    bandwidth reference of the large AllReduce calls."""
    rc = lib().ar_copy(_ptr(src), _ptr(dst), int(nbytes), _stream_handle(stream))
    return _check("ar_copy", rc) if check else rc


def flag_ping(rounds, cross_xcd, out, stream=None, check=True):
    """`rounds` round trips of a flag between two workgroups (include/ar_ping.h);
    `out` is a device buffer of 5 int64 words that receives the clock ticks,
    the two statuses and the two workgroups' XCDs."""
    rc = lib().ar_flag_ping(int(rounds), int(cross_xcd), _ptr(out), _stream_handle(stream))
    return _check("ar_flag_ping", rc) if check else rc


def allreduce_f32_debug(rank_bufs, out_f32, n, epoch, stream=None, check=True):
    rc = lib().ar_allreduce_f32_debug(_rank_array(rank_bufs), _ptr(out_f32), int(n), int(epoch),
                                      _stream_handle(stream))
    return _check("ar_allreduce_f32_debug", rc) if check else rc


def set_options(algo=AR_ALGO_AUTO, proto=AR_PROTO_AUTO):
    return _check("ar_set_options", lib().ar_set_options(int(algo), int(proto)))


def set_launch(wgs_per_rank=0, threads=0):
    return _check("ar_set_launch", lib().ar_set_launch(int(wgs_per_rank), int(threads)))


def set_scope(scope=AR_SCOPE_AUTO):
    return _check("ar_set_scope", lib().ar_set_scope(int(scope)))


def set_staging(window_bytes=0):
    """Staging window (bytes per rank or inbox pair and buffer; 0 = all)."""
    return _check("ar_set_staging", lib().ar_set_staging(int(window_bytes)))


def set_watchdog(budget_us=0):
    return _check("ar_set_watchdog", lib().ar_set_watchdog(int(budget_us)))


def step_end(stream=None):
    return _check("ar_step_end", lib().ar_step_end(_stream_handle(stream)))


def set_delays(dev_ns=None, calls=0):
    p = 0 if dev_ns is None else _ptr(dev_ns)
    return _check("ar_set_delays", lib().ar_set_delays(p or None, int(calls)))


def set_timestamps(dev_ts=None, slots=0, records_per_slot=0, phases=False):
    """dev_ts: uint64/int64 device tensor [slots, records_per_slot, 4]."""
    p = 0 if dev_ts is None else _ptr(dev_ts)
    return _check("ar_set_timestamps",
                  lib().ar_set_timestamps(p or None, int(slots), int(records_per_slot),
                                          1 if phases else 0))


def set_sequence(seq, stream=None):
    """Test hook: sets the device round sequence (between steps)."""
    return _check("ar_set_sequence", lib().ar_set_sequence(int(seq), _stream_handle(stream)))


def get_status():
    """Returns (code, rank, source, flag) of the device status record."""
    buf = (_c_u32 * 4)()
    rc = lib().ar_get_status(buf)
    if rc not in (AR_OK, AR_ERR_TIMEOUT):
        raise ArError("ar_get_status", rc)
    return tuple(int(x) for x in buf)


def reset(stream=None):
    return _check("ar_reset", lib().ar_reset(_stream_handle(stream)))


def query(key, n=0):
    v = lib().ar_query(int(key), int(n))
    if v < 0:
        raise ArError("ar_query", int(v))
    return int(v)
