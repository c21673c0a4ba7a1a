"""Optional roctx ranges around the phases of the round loop, for
`rocprofv3 --marker-trace`: prefill, round, draft, verify, accept, calibrate.

Enabled by SPEC_ROCTX=1 (the ranges cost a host call each); the ROCm marker
library is loaded with ctypes.  Disabled, `rng(name)` is a no-op context."""
from __future__ import annotations

import contextlib
import ctypes
import os

_lib = None
_tried = False


def _load():
    global _lib, _tried
    if _tried:
        return _lib
    _tried = True
    if os.environ.get("SPEC_ROCTX", "0") != "1":
        return None
    for name in ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4", "librocprofiler-sdk-roctx.so", "libroctx64.so"):
        try:
            lib = ctypes.CDLL(name)
        except OSError:
            try:
                lib = ctypes.CDLL(os.path.join("/opt/rocm/lib", name))
            except OSError:
                continue
        lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
        lib.roctxRangePushA.restype = ctypes.c_int
        lib.roctxRangePop.argtypes = []
        lib.roctxRangePop.restype = ctypes.c_int
        _lib = lib
        break
    return _lib


@contextlib.contextmanager
def rng(name: str):
    lib = _load()
    if lib is None:
        yield
        return
    lib.roctxRangePushA(name.encode())
    try:
        yield
    finally:
        lib.roctxRangePop()


def enabled() -> bool:
    return _load() is not None
