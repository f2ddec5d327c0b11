"""The C-ABI library loads and exports every entry point include/ar.h
declares, and its host-side validation works without a GPU (no compute
calls are made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ar.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z0-9_]+)\s*\(", text)))


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
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.ar_strerror(code)
    assert lib.ar_strerror(-99) == b"unknown status"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import tp_decode_comms_amd.ar as a
    monkeypatch.setenv("TPDC_AR_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(a, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        a.lib()
