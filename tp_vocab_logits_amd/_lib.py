"""ctypes binding of libhg.so (declared in include/hg.h): argument marshalling
only. Every step of the gather runs in the library's HIP kernels.

torch is imported before the library is loaded so that libhg.so binds to the
HIP runtime torch already loaded (both carry the soname ``libamdhip64.so.7``);
device pointers and streams are then shared between the two.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads torch's HIP runtime first; see the module docstring)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhg.so")

HG_OK = 0
HG_EDECLINE = 1
HG_EINVAL = -1
HG_ENOMEM = -2
HG_EHIP = -3
HG_ETIMEOUT = -4
HG_ESTATE = -5
HG_ESIZE = -6
HG_STATIC_PARITY_BYTES = 8 << 20
HG_MAX_TP = 64

_vp = ctypes.c_void_p
_i = ctypes.c_int
_ull = ctypes.c_ulonglong
_size = ctypes.c_size_t
_ctxp = ctypes.c_void_p

# name -> (restype, argtypes); the C declarations are in include/hg.h
SIGNATURES = {
    "hg_create": (_i, [_i, _i, _i, ctypes.POINTER(_ctxp)]),
    "hg_destroy": (_i, [_ctxp]),
    "hg_arm": (_i, [_ctxp, _vp]),
    "hg_gather": (_i, [_ctxp, ctypes.POINTER(_vp), _i, _vp, _vp]),
    "hg_push": (_i, [_ctxp, ctypes.POINTER(_vp), _i, _vp]),
    "hg_push_ranks": (_i, [_ctxp, ctypes.POINTER(_vp), _i, _ull, _vp]),
    "hg_collect": (_i, [_ctxp, _i, _vp, _vp]),
    "hg_stock_gather": (_i, [_i, _i, ctypes.POINTER(_vp), _i, _vp, _i, _vp]),
    "hg_lmhead": (_i, [_i, _i, _vp, ctypes.POINTER(_vp), _i, _i, ctypes.POINTER(_vp), _vp]),
    "hg_gemm_gather": (_i, [_ctxp, _vp, ctypes.POINTER(_vp), _i, _i, _vp, ctypes.POINTER(_vp), _vp]),
    "hg_parity": (_i, [_ctxp]),
    "hg_set_device_parity": (_i, [_ctxp, _i, _vp]),
    "hg_set_vocab": (_i, [_ctxp, _i]),
    "hg_vocab": (_i, [_ctxp]),
    "hg_mailbox": (_i, [_ctxp, _i, ctypes.POINTER(_vp), ctypes.POINTER(_size)]),
    "hg_copy_mailbox": (_i, [_ctxp, _i, _vp, _vp]),
    "hg_set_poll_limit": (_i, [_ctxp, _ull]),
    "hg_poll_status": (_i, [_ctxp, _vp]),
    "hg_fused_grid_limit": (_i, [_ctxp, _i]),
    "hg_gather_static": (_i, [_i, _i, ctypes.POINTER(_vp), _i, _vp, _vp]),
    "hg_strerror": (ctypes.c_char_p, [_i]),
    "hg_last_error_detail": (ctypes.c_char_p, []),
}


class HgError(RuntimeError):
    """A negative status from libhg.so."""

    def __init__(self, code: int, where: str):
        self.code = code
        detail = ""
        if code == HG_EHIP:
            detail = " [" + (lib().hg_last_error_detail() or b"").decode(errors="replace") + "]"
        msg = (lib().hg_strerror(code) or b"?").decode()
        super().__init__(f"{where}: {msg} ({code}){detail}")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if libhg.so was not built:
    there is no fallback implementation."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m tp_vocab_logits_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


_REF = None


def ref() -> ctypes.CDLL:
    """libhgref.so: the reference streaming kernel the benchmark times beside
    the gather (``hgref_stream``). Raises if it was not built."""
    global _REF
    if _REF is None:
        path = os.path.join(os.path.dirname(LIB_PATH), "libhgref.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m tp_vocab_logits_amd.build`")
        handle = ctypes.CDLL(path)
        handle.hgref_stream.restype = ctypes.c_int
        handle.hgref_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                        ctypes.c_void_p]
        _REF = handle
    return _REF


_FAST = None


def fast():
    """The ``_hgcall`` extension, bound to the loaded library: ``gather``,
    ``push``, ``collect`` and ``stock`` taking plain integers (handle, sizes,
    host-array address, rows, device address, stream) in the C argument order
    and returning the status code -- the same calls as through ctypes, with
    less per-call conversion."""
    global _FAST
    if _FAST is None:
        from . import _hgcall

        handle = lib()
        _hgcall.bind(*[ctypes.cast(getattr(handle, n), ctypes.c_void_p).value
                       for n in ("hg_gather", "hg_push", "hg_collect", "hg_stock_gather")])
        _FAST = _hgcall
    return _FAST


def check(code: int, where: str) -> int:
    """Raise :class:`HgError` on a negative status; return it otherwise."""
    if code < 0:
        raise HgError(code, where)
    return code


def pointer_array(ptrs) -> ctypes.Array:
    """A C array of device pointers (``const void *const *``)."""
    return (_vp * len(ptrs))(*[_vp(int(p)) for p in ptrs])
