"""Launch override of the HIP library, for tests, sweeps and tuning.

This wraps the library's tuning interface (csrc/mfr_tuning.h), which is not
part of the op's C ABI: every entry point picks its launch shape by itself.
The override belongs to the calling thread.
"""
import ctypes
import threading

from . import binding

STORE_AUTO = 0
STORE_WRITE_BACK = 1
STORE_WRITE_THROUGH = 2

_lib = binding.lib()
_lib.mfr_tuning_force_launch.restype = ctypes.c_int
_lib.mfr_tuning_force_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.mfr_tuning_force_residency.restype = ctypes.c_int
_lib.mfr_tuning_force_residency.argtypes = [ctypes.c_int]


# this thread's current override, mirrored here so that forced() can restore it
_state = threading.local()


def _current():
    return getattr(_state, "launch", (0, 0, 0)), getattr(_state, "residency", 0)


def force_launch(path=0, vectors_per_thread=0, store_policy=0):
    """Force the launch path, vectors per thread and store policy of this
    thread's later calls (0 = automatic for each)."""
    args = (int(path), int(vectors_per_thread), int(store_policy))
    rc = _lib.mfr_tuning_force_launch(*args)
    if rc != binding.MFR_OK:
        raise binding.MFRError(rc)
    _state.launch = args


def force_residency(workgroups_per_cu=0):
    """Cap the persistent path's workgroups per CU on this thread (0 = as many
    as fit)."""
    rc = _lib.mfr_tuning_force_residency(int(workgroups_per_cu))
    if rc != binding.MFR_OK:
        raise binding.MFRError(rc)
    _state.residency = int(workgroups_per_cu)


class forced:
    """Context manager: force a launch configuration on this thread (and, for
    the persistent path, its workgroups per CU); the thread's previous
    override is back on exit. With every argument 0 (automatic) the
    enclosing override is kept, so a helper that forces nothing does not
    undo its caller's choice."""

    def __init__(self, path=0, vpt=0, store=0, residency=0):
        self.args = (path, vpt, store)
        self.residency = residency

    def __enter__(self):
        self.saved = _current()
        if self.args != (0, 0, 0) or self.residency:
            force_launch(*self.args)
            force_residency(self.residency)
        return self

    def __exit__(self, *exc):
        force_launch(*self.saved[0])
        force_residency(self.saved[1])
        return False
