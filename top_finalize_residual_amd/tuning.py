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
# non-temporal output stores: the top-8 bf16 kernels of the grid paths only
STORE_NONTEMPORAL = 3
STORE_NONTEMPORAL_WRITE_THROUGH = 4

ORDER_DEFAULT = 0
ORDER_XCD_RANGES = 1  # each XCD takes one contiguous range of tokens

_lib = binding.lib()
_lib.mfr_tuning_force_launch.restype = ctypes.c_int
_lib.mfr_tuning_force_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.mfr_tuning_force_residency.restype = ctypes.c_int
_lib.mfr_tuning_force_residency.argtypes = [ctypes.c_int]
_lib.mfr_tuning_force_token_order.restype = ctypes.c_int
_lib.mfr_tuning_force_token_order.argtypes = [ctypes.c_int]


# this thread's current override, mirrored here so that forced() can restore it
_state = threading.local()


def _current():
    return (getattr(_state, "launch", (0, 0, 0)), getattr(_state, "residency", 0),
            getattr(_state, "order", 0))


def force_launch(path=0, vectors_per_thread=0, store_policy=0):
    """Force the launch path, vectors per thread and store policy of this
    thread's later calls (0 = automatic for each)."""
    args = (int(path), int(vectors_per_thread), int(store_policy))
    rc = _lib.mfr_tuning_force_launch(*args)
    if rc != binding.MFR_OK:
        raise binding.MFRError(rc)
    _state.launch = args


def force_residency(workgroups_per_cu=0):
    """Cap the workgroups per CU on this thread: the persistent path's grid,
    or, on the grid paths, through LDS reserved at launch. 0 = automatic (the
    library's own rule); a value at or above what the kernel's registers
    allow means no cap."""
    rc = _lib.mfr_tuning_force_residency(int(workgroups_per_cu))
    if rc != binding.MFR_OK:
        raise binding.MFRError(rc)
    _state.residency = int(workgroups_per_cu)


def force_token_order(order=ORDER_DEFAULT):
    """Token order of the grid paths on this thread (ORDER_DEFAULT or
    ORDER_XCD_RANGES)."""
    rc = _lib.mfr_tuning_force_token_order(int(order))
    if rc != binding.MFR_OK:
        raise binding.MFRError(rc)
    _state.order = int(order)


class forced:
    """Context manager: force a launch configuration on this thread (path,
    vectors per thread, store policy, workgroups per CU, token order); the
    thread's previous override is back on exit. With every argument 0
    (automatic) the enclosing override is kept, so a helper that forces
    nothing does not undo its caller's choice."""

    def __init__(self, path=0, vpt=0, store=0, residency=0, order=0):
        self.args = (path, vpt, store)
        self.residency = residency
        self.order = order

    def __enter__(self):
        self.saved = _current()
        if self.args != (0, 0, 0) or self.residency or self.order:
            force_launch(*self.args)
            force_residency(self.residency)
            force_token_order(self.order)
        return self

    def __exit__(self, *exc):
        force_launch(*self.saved[0])
        force_residency(self.saved[1])
        force_token_order(self.saved[2])
        return False
