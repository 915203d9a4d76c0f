"""roctx ranges around the step's phases, for rocprofv3's marker trace
(`rocprofv3 --marker-trace ...`).

Off unless enable() is called; then every `with span("name"):` pushes a
named host range (librocprofiler-sdk-roctx) that the trace shows beside the
kernels the range enqueued.  A range times the host-side enqueue, not the
kernels; the kernel trace gives their device time.
"""
import contextlib
import ctypes as C
import os

_lib = None


def enable(path=None):
    """Load the roctx library (ROCM_PATH or /opt/rocm by default); raises
    OSError if it is not there."""
    global _lib
    if path is None:
        root = os.environ.get("ROCM_PATH", "/opt/rocm")
        path = os.path.join(root, "lib", "librocprofiler-sdk-roctx.so")
    lib = C.CDLL(path)
    lib.roctxRangePushA.argtypes = [C.c_char_p]
    lib.roctxRangePushA.restype = C.c_int
    lib.roctxRangePop.argtypes = []
    lib.roctxRangePop.restype = C.c_int
    _lib = lib


def enabled():
    return _lib is not None


@contextlib.contextmanager
def span(name):
    if _lib is None:
        yield
        return
    _lib.roctxRangePushA(name.encode())
    try:
        yield
    finally:
        _lib.roctxRangePop()
