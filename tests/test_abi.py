"""The C ABI without a GPU: libhg.so loads, exports every function that
include/hg.h declares, and its host-side argument checks return the documented
codes before touching a device."""

import ctypes
import os
import re

import pytest

from tp_vocab_logits_amd import _lib
from oracle import gather as oracle_gather

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"#[^\n]*", " ", text)
    return sorted(set(re.findall(r"\b(hg_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for required in ["hg_create", "hg_arm", "hg_gather", "hg_destroy", "hg_push", "hg_collect",
                     "hg_parity", "hg_mailbox", "hg_strerror"]:
        assert required in names
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with hg.h"


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_create_validation_matches_the_oracle_rules():
    lib = _lib.lib()
    h = ctypes.c_void_p(1)
    for tp in range(0, 5):
        for shard in range(0, 41):
            for cap in (0, 1, 3):
                if oracle_gather.create_ok(tp, shard, cap):
                    continue  # a valid create needs a device; not run here
                rc = lib.hg_create(tp, shard, cap, ctypes.byref(h))
                assert rc == _lib.HG_EINVAL, (tp, shard, cap)
                assert not h.value
    assert lib.hg_create(65, 8, 1, ctypes.byref(h)) == _lib.HG_EINVAL  # above HG_MAX_TP
    assert lib.hg_create(2, 8, 1, None) == _lib.HG_EINVAL
    # a mailbox of 2^31 vectors per parity or more is refused
    assert lib.hg_create(8, 8 * 2 ** 20, 2 ** 8, ctypes.byref(h)) == _lib.HG_EINVAL


def test_null_context_paths():
    lib = _lib.lib()
    null = ctypes.c_void_p()
    ptrs = _lib.pointer_array([16, 32])
    assert lib.hg_destroy(null) == _lib.HG_OK
    assert lib.hg_arm(null, None) == _lib.HG_EINVAL
    assert lib.hg_gather(null, ptrs, 1, ctypes.c_void_p(64), None) == _lib.HG_EINVAL
    assert lib.hg_push(null, ptrs, 1, None) == _lib.HG_EINVAL
    assert lib.hg_push_ranks(null, ptrs, 1, 1, None) == _lib.HG_EINVAL
    assert lib.hg_collect(null, 1, ctypes.c_void_p(64), None) == _lib.HG_EINVAL
    assert lib.hg_parity(null) == _lib.HG_EINVAL
    dev, nbytes = ctypes.c_void_p(), ctypes.c_size_t()
    assert lib.hg_mailbox(null, 0, ctypes.byref(dev), ctypes.byref(nbytes)) == _lib.HG_EINVAL
    assert lib.hg_copy_mailbox(null, 0, ctypes.c_void_p(64), None) == _lib.HG_EINVAL
    assert lib.hg_set_poll_limit(null, 5) == _lib.HG_EINVAL
    assert lib.hg_poll_status(null, None) == _lib.HG_EINVAL
    assert lib.hg_fused_grid_limit(null, 1) == _lib.HG_EINVAL
    assert lib.hg_set_device_parity(null, 1, None) == _lib.HG_EINVAL
    assert lib.hg_set_vocab(null, 5) == _lib.HG_EINVAL
    assert lib.hg_vocab(null) == _lib.HG_EINVAL


def test_stock_gather_argument_checks():
    lib = _lib.lib()
    ptrs = _lib.pointer_array([16, 32])
    out = ctypes.c_void_p(4096)
    assert lib.hg_stock_gather(0, 8, ptrs, 1, out, 8, None) == _lib.HG_EINVAL
    assert lib.hg_stock_gather(2, 0, ptrs, 1, out, 1, None) == _lib.HG_EINVAL   # empty rows
    assert lib.hg_stock_gather(2, 8, ptrs, -1, out, 16, None) == _lib.HG_EINVAL
    assert lib.hg_stock_gather(2, 8, ptrs, 1, out, 0, None) == _lib.HG_EINVAL    # vocab < 1
    assert lib.hg_stock_gather(2, 8, ptrs, 1, out, 17, None) == _lib.HG_EINVAL   # vocab > tp*shard
    assert lib.hg_stock_gather(2, 8, ptrs, 0, out, 16, None) == _lib.HG_OK  # nothing to do
    assert lib.hg_stock_gather(2, 8, ptrs, 1, ctypes.c_void_p(4100), 16, None) == _lib.HG_EINVAL
    bad = _lib.pointer_array([16, 40])  # rank-1 pointer not 16-byte aligned (vector rows)
    assert lib.hg_stock_gather(2, 8, bad, 1, out, 16, None) == _lib.HG_EINVAL
    odd = _lib.pointer_array([16, 41])  # not even 2-byte aligned (element rows)
    assert lib.hg_stock_gather(2, 12, odd, 1, out, 24, None) == _lib.HG_EINVAL
    overlap = _lib.pointer_array([16, 4096])  # rank 1 overlaps the output
    assert lib.hg_stock_gather(2, 8, overlap, 1, out, 16, None) == _lib.HG_EINVAL


def test_static_gather_host_checks():
    # sizes are refused before any device call (hg_gather_static's limit is
    # HG_STATIC_PARITY_BYTES per parity: 25 rows of V = 163840)
    lib = _lib.lib()
    ptrs = _lib.pointer_array([16] * 8)
    out = ctypes.c_void_p(1 << 30)
    assert lib.hg_gather_static(8, 20480, ptrs, 26, out, None) == _lib.HG_ESIZE
    assert b"static" in lib.hg_last_error_detail()
    assert lib.hg_gather_static(8, 20480, ptrs, 1 << 30, out, None) == _lib.HG_ESIZE
    assert lib.hg_gather_static(1, 20480, ptrs, 1, out, None) == _lib.HG_EINVAL
    assert lib.hg_gather_static(8, 12, ptrs, 1, out, None) == _lib.HG_EINVAL
    assert lib.hg_gather_static(8, 20480, ptrs, -1, out, None) == _lib.HG_EINVAL
    assert lib.hg_gather_static(8, 20480, ptrs, 0, out, None) == _lib.HG_EDECLINE
    assert lib.hg_gather_static(8, 20480, None, 1, out, None) == _lib.HG_EINVAL
    assert lib.hg_strerror(_lib.HG_ESIZE) == b"request exceeds the static scratch buffer"


def test_status_strings():
    lib = _lib.lib()
    for code in (_lib.HG_OK, _lib.HG_EDECLINE, _lib.HG_EINVAL, _lib.HG_ENOMEM, _lib.HG_EHIP,
                 _lib.HG_ETIMEOUT, _lib.HG_ESTATE, _lib.HG_ESIZE, 1234):
        assert lib.hg_strerror(code)
    assert lib.hg_last_error_detail() is not None


def test_fastcall_binding():
    """The fast-call wrappers reach the same entry points as ctypes: null
    handles give HG_EINVAL, malformed calls raise before reaching C."""
    f = _lib.fast()
    assert f.gather(0, 0, 1, 0, 0) == _lib.HG_EINVAL
    assert f.push(0, 0, 1, 0) == _lib.HG_EINVAL
    assert f.collect(0, 1, 0, 0) == _lib.HG_EINVAL
    assert f.stock(0, 8, 0, 1, 4096, 8, 0) == _lib.HG_EINVAL  # tp 0
    assert f.stock(2, 8, 0, 1, 4096, 16, 0) == _lib.HG_EINVAL  # no shard array
    assert f.stock(2, 8, 0, 0, 4096, 16, 0) == _lib.HG_OK  # no rows: nothing to do
    with pytest.raises(TypeError):
        f.gather(0, 0, 1, 0)
    with pytest.raises(OverflowError):
        f.collect(0, 1 << 40, 0, 0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no fallback implementation: without libhg.so the loader raises (every
    # entry point of the binding goes through it)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libhg.so"))
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "_FAST", None)
    with pytest.raises(ImportError):
        _lib.lib()
    with pytest.raises(ImportError):
        _lib.fast()
