"""roctx ranges around the driver's units of work (members, blocks, forward and backward), so
that a profile taken with `rocprofv3 --marker-trace` shows where each member and block starts
and ends.  The ranges go through ROCm's roctx library if it can be loaded, and cost nothing
otherwise; they never touch the GPU."""
from __future__ import annotations

import contextlib
import ctypes as C
import os

_LIB_NAMES = ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so")
_lib = None
_tried = False


def _roctx():
    global _lib, _tried
    if not _tried:
        _tried = True
        rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
        for name in _LIB_NAMES:
            for path in (name, os.path.join(rocm, "lib", name)):
                try:
                    h = C.CDLL(path)
                    h.roctxRangePushA.argtypes = [C.c_char_p]
                    h.roctxRangePushA.restype = C.c_int
                    h.roctxRangePop.argtypes = []
                    h.roctxRangePop.restype = C.c_int
                    _lib = h
                    return _lib
                except (OSError, AttributeError):
                    continue
    return _lib


def available() -> bool:
    return _roctx() is not None


@contextlib.contextmanager
def trace_range(name: str):
    """A roctx range named `name` around the body (nested ranges nest)."""
    lib = _roctx()
    if lib is not None:
        lib.roctxRangePushA(name.encode())
    try:
        yield
    finally:
        if lib is not None:
            lib.roctxRangePop()
