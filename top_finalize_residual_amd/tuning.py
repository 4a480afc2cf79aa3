"""Launch override of the HIP library, for tests, sweeps and tuning.

This wraps the library's tuning interface (csrc/mfr_tuning.h), which is not
part of the op's C ABI: every entry point picks its launch shape by itself.
The override belongs to the calling thread.
"""
import ctypes

from . import binding

STORE_AUTO = 0
STORE_WRITE_BACK = 1
STORE_WRITE_THROUGH = 2

_lib = binding.lib()
_lib.mfr_tuning_force_launch.restype = ctypes.c_int
_lib.mfr_tuning_force_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]


def force_launch(path=0, vectors_per_thread=0, store_policy=0):
    """Force the launch path, vectors per thread and store policy of this
    thread's later calls (0 = automatic for each)."""
    rc = _lib.mfr_tuning_force_launch(int(path), int(vectors_per_thread), int(store_policy))
    if rc != binding.MFR_OK:
        raise binding.MFRError(rc)


class forced:
    """Context manager: force a launch configuration on this thread, back to
    automatic on exit."""

    def __init__(self, path=0, vpt=0, store=0):
        self.args = (path, vpt, store)

    def __enter__(self):
        force_launch(*self.args)
        return self

    def __exit__(self, *exc):
        force_launch(0, 0, 0)
        return False
