"""The C-ABI library loads and exports every entry point include/*.h
declares, and its host-side validation works without a GPU (no compute
calls are made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(ar_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    import tp_decode_comms_amd as ar
    path = ar.lib_path()
    if not os.path.exists(path):
        from tp_decode_comms_amd import build
        build.build()
    return ar.lib()


def test_header_declares_entry_points():
    names = _declared()
    for must in ("ar_init", "ar_allreduce", "ar_destroy"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    import tp_decode_comms_amd as ar
    for name in _declared():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)
    assert set(_declared()) == set(ar.EXPORTED_SYMBOLS)


def test_host_validation_without_device(lib):
    import tp_decode_comms_amd.ar as a
    assert lib.ar_init(0, 16) == a.AR_ERR_INVALID
    assert lib.ar_init(17, 16) == a.AR_ERR_INVALID
    assert lib.ar_init(4, 0) == a.AR_ERR_INVALID
    assert lib.ar_init(4, (1 << 28) + 1) == a.AR_ERR_INVALID
    # nothing is initialised in this process
    assert lib.ar_destroy() == a.AR_ERR_NOT_INIT
    assert lib.ar_set_options(0, 0) == a.AR_ERR_NOT_INIT
    assert lib.ar_step_end(None) == a.AR_ERR_NOT_INIT
    assert lib.ar_reset(None) == a.AR_ERR_NOT_INIT
    assert lib.ar_query(0, 0) == a.AR_ERR_NOT_INIT
    ptrs = (ctypes.c_void_p * 1)(0)
    assert lib.ar_allreduce(ptrs, None, 8, 1, None) == a.AR_ERR_NOT_INIT
    assert lib.ar_allreduce_add_rmsnorm(ptrs, ptrs, 16, 1e-5, 16, 16, 1, 256, 1,
                                        None) == a.AR_ERR_NOT_INIT
    assert lib.ar_add_rmsnorm(16, ptrs, 16, 1e-5, 16, 16, 1, 256, None) == a.AR_ERR_NOT_INIT
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.ar_strerror(code)
    assert lib.ar_strerror(-99) == b"unknown status"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import tp_decode_comms_amd.ar as a
    monkeypatch.setenv("TPDC_AR_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(a, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        a.lib()


def test_gemv_validation_without_device(lib):
    import tp_decode_comms_amd.ar as a
    P = ctypes.c_void_p * 1
    good = P(16)
    assert lib.ar_gemv_bf16(None, good, good, 8, 8, 1, 0, None) == a.AR_ERR_INVALID
    assert lib.ar_gemv_bf16(good, good, good, 0, 8, 1, 0, None) == a.AR_ERR_INVALID   # M = 0
    assert lib.ar_gemv_bf16(good, good, good, 8, 12, 1, 0, None) == a.AR_ERR_INVALID  # K % 8
    assert lib.ar_gemv_bf16(good, good, good, 8, 8, 0, 0, None) == a.AR_ERR_INVALID   # n_ranks
    assert lib.ar_gemv_bf16(good, good, good, 8, 8, 17, 0, None) == a.AR_ERR_INVALID
    assert lib.ar_gemv_bf16(P(8), good, P(4096), 8, 8, 1, 0, None) == a.AR_ERR_INVALID  # unaligned W
    assert lib.ar_gemv_bf16(good, good, P(16), 8, 8, 1, 0, None) == a.AR_ERR_INVALID  # y aliases W
    assert lib.ar_gemv_bf16(good, good, P(4096), 8, 8, 1, -1, None) == a.AR_ERR_INVALID
    assert lib.ar_gemv_bf16(good, good, P(1 << 33), 1, (1 << 28) + 8, 1, 0, None) == a.AR_ERR_INVALID  # K
    # the copy reference: alignment, size and overlap checks launch nothing
    assert lib.ar_copy(None, 4096, 16, None) == a.AR_ERR_INVALID
    assert lib.ar_copy(4096, 8192, 0, None) == a.AR_ERR_INVALID
    assert lib.ar_copy(4096, 8192, 24, None) == a.AR_ERR_INVALID          # not whole vectors
    assert lib.ar_copy(4104, 8192, 16, None) == a.AR_ERR_INVALID          # unaligned source
    assert lib.ar_copy(4096, 4096 + 16, 32, None) == a.AR_ERR_INVALID     # overlap
    assert lib.ar_copy(1 << 40, 1 << 41, 1 << 31, None) == a.AR_ERR_INVALID   # too large
    # the flag hop: round count, output pointer and placement are checked first
    assert lib.ar_flag_ping(0, 0, 4096, None) == a.AR_ERR_INVALID                # no rounds
    assert lib.ar_flag_ping((1 << 20) + 1, 0, 4096, None) == a.AR_ERR_INVALID    # too many
    assert lib.ar_flag_ping(10, 0, None, None) == a.AR_ERR_INVALID               # no output
    assert lib.ar_flag_ping(10, 1, 4100, None) == a.AR_ERR_INVALID               # unaligned
    assert lib.ar_flag_ping(10, 2, 4096, None) == a.AR_ERR_INVALID               # placement
