"""Python binding of libmoe_finalize_rmsnorm.so (ctypes; argument marshalling only).

Every step of the op runs in the HIP library. torch supplies device memory and
the current stream. There is no CPU fallback: if the library is missing,
importing this module raises.
"""
import contextlib
import ctypes
import os

import torch

from . import build as _build

MFR_OK = 0
MFR_ERR_NULL = 1
MFR_ERR_SHAPE = 2
MFR_ERR_ALIGN = 3
MFR_ERR_ALIAS = 4
MFR_ERR_SCALAR = 5
MFR_ERR_HIP = 6
MFR_ERR_ARG = 7

PATH_UNSUPPORTED = 0
PATH_TOKEN = 1
PATH_STREAM = 2

STORE_AUTO = 0
STORE_WRITE_BACK = 1
STORE_WRITE_THROUGH = 2

LIB_PATH = _build.LIB
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run top_finalize_residual_amd/build.py (hipcc, gfx950) first")
_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib.moe_finalize_rmsnorm.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_float, ctypes.c_float,
                                      _p, _p, _i64, _i64, _i64, _p]
_lib.moe_finalize_rmsnorm_path.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_path.argtypes = [_i64, _i64, _i64]
_lib.moe_finalize_rmsnorm_strerror.restype = ctypes.c_char_p
_lib.moe_finalize_rmsnorm_strerror.argtypes = [ctypes.c_int]
_lib.moe_finalize_rmsnorm_fp8.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_fp8.argtypes = [_p, _p, _p, _p, _p, _p, ctypes.c_float, ctypes.c_float,
                                          _p, _p, _p, _p, _i64, _i64, _i64, _p]
_lib.residual_add_rmsnorm.restype = ctypes.c_int
_lib.residual_add_rmsnorm.argtypes = [_p, _p, _p, ctypes.c_float, _p, _p, _i64, _i64, _p]
_lib.residual_add_rmsnorm_fp8.restype = ctypes.c_int
_lib.residual_add_rmsnorm_fp8.argtypes = [_p, _p, _p, ctypes.c_float, _p, _p, _p, _p, _i64, _i64,
                                          _p]
_lib.moe_finalize_rmsnorm_checked.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_checked.argtypes = [_p, _i64, _p, _p, _p, _p, _p, ctypes.c_float,
                                              ctypes.c_float, _p, _p, _p, _i64, _i64, _i64, _p]
_lib.moe_finalize_rmsnorm_fp8_checked.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_fp8_checked.argtypes = [_p, _i64, _p, _p, _p, _p, _p, ctypes.c_float,
                                                  ctypes.c_float, _p, _p, _p, _p, _p, _i64, _i64,
                                                  _i64, _p]
_lib.moe_finalize_rmsnorm_force.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_force.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]


class MFRError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"moe_finalize_rmsnorm: {strerror(status)} (status {status})")


def lib():
    """The loaded ctypes library (for raw-pointer calls)."""
    return _lib


def strerror(status):
    return _lib.moe_finalize_rmsnorm_strerror(int(status)).decode()


def moe_finalize_rmsnorm_path(T, H, K):
    return _lib.moe_finalize_rmsnorm_path(int(T), int(H), int(K))


def moe_finalize_rmsnorm_force(path=0, vectors_per_thread=0, store_policy=0):
    """Process-wide launch override (0 = automatic for each); see the C header."""
    rc = _lib.moe_finalize_rmsnorm_force(int(path), int(vectors_per_thread), int(store_policy))
    if rc != MFR_OK:
        raise MFRError(rc)


def moe_finalize_rmsnorm_raw(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                             scale, residual_out, normed_out, T, H, K, stream):
    """Direct C call with integer addresses; returns the status code."""
    return _lib.moe_finalize_rmsnorm(expert_out, perm_idx, topk_w, shared_out, residual, gamma,
                                     float(eps), float(scale), residual_out, normed_out,
                                     int(T), int(H), int(K), stream)


def _check(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one GPU, got {sorted(str(d) for d in devs)}")


def _launch_context(dev, stream):
    """The stream to launch on (the device's current stream by default) and a
    context that makes the tensors' GPU current for the call: the library
    launches on the calling thread's current device."""
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    if dev.index is None or dev.index == torch.cuda.current_device():
        return stream, contextlib.nullcontext()
    return stream, torch.cuda.device(dev)


def moe_finalize_rmsnorm(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale,
                         residual_out=None, normed_out=None, stream=None):
    """Fused MoE finalize + residual add + RMSNorm on the current (or given) stream.

    expert_out [R, H] bf16, perm_idx [T, K] int32 (-1 = masked), topk_w [T, K] fp32,
    shared_out / residual [T, H] bf16, gamma [H] bf16; eps, scale are floats.
    residual_out / normed_out ([T, H] bf16) are allocated when not given;
    residual_out may be `residual` itself. Returns (residual_out, normed_out).
    """
    _check(expert_out, "expert_out", torch.bfloat16, 2)
    _check(perm_idx, "perm_idx", torch.int32, 2)
    _check(topk_w, "topk_w", torch.float32, 2)
    _check(shared_out, "shared_out", torch.bfloat16, 2)
    _check(residual, "residual", torch.bfloat16, 2)
    _check(gamma, "gamma", torch.bfloat16, 1)
    T, K = perm_idx.shape
    H = gamma.shape[0]
    if expert_out.shape[1] != H:
        raise ValueError("expert_out width differs from gamma length")
    for name, t in (("shared_out", shared_out), ("residual", residual)):
        if tuple(t.shape) != (T, H):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(T, H)}")
    if tuple(topk_w.shape) != (T, K):
        raise ValueError("topk_w shape differs from perm_idx shape")
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=residual.device)
    if normed_out is None:
        normed_out = torch.empty((T, H), dtype=torch.bfloat16, device=residual.device)
    _check(residual_out, "residual_out", torch.bfloat16, 2)
    _check(normed_out, "normed_out", torch.bfloat16, 2)
    if tuple(residual_out.shape) != (T, H) or tuple(normed_out.shape) != (T, H):
        raise ValueError("outputs must be [T, H]")
    _same_device(expert_out, perm_idx, topk_w, shared_out, residual, gamma, residual_out, normed_out)
    stream, ctx = _launch_context(residual.device, stream)
    with ctx:
        rc = _lib.moe_finalize_rmsnorm(
            expert_out.data_ptr(), perm_idx.data_ptr(), topk_w.data_ptr(), shared_out.data_ptr(),
            residual.data_ptr(), gamma.data_ptr(), float(eps), float(scale),
            residual_out.data_ptr(), normed_out.data_ptr(), T, H, K, stream.cuda_stream)
    if rc != MFR_OK:
        raise MFRError(rc)
    return residual_out, normed_out


def moe_finalize_rmsnorm_checked(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                                 scale, residual_out=None, normed_out=None, bad_index=None,
                                 stream=None):
    """moe_finalize_rmsnorm told R = expert_out.shape[0]: a slot whose index
    is at or past R is treated as masked instead of reading outside
    expert_out, and bad_index (a one-element int32 GPU tensor, allocated
    zeroed when not given) is set to 1 if any token holds such an index.
    Returns (residual_out, normed_out, bad_index)."""
    _check(expert_out, "expert_out", torch.bfloat16, 2)
    _check(perm_idx, "perm_idx", torch.int32, 2)
    _check(topk_w, "topk_w", torch.float32, 2)
    _check(shared_out, "shared_out", torch.bfloat16, 2)
    _check(residual, "residual", torch.bfloat16, 2)
    _check(gamma, "gamma", torch.bfloat16, 1)
    T, K = perm_idx.shape
    H = gamma.shape[0]
    R = expert_out.shape[0]
    if expert_out.shape[1] != H or tuple(shared_out.shape) != (T, H) or \
            tuple(residual.shape) != (T, H) or tuple(topk_w.shape) != (T, K):
        raise ValueError("inconsistent shapes")
    dev = residual.device
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if normed_out is None:
        normed_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if bad_index is None:
        bad_index = torch.zeros((1,), dtype=torch.int32, device=dev)
    _check(residual_out, "residual_out", torch.bfloat16, 2)
    _check(normed_out, "normed_out", torch.bfloat16, 2)
    _check(bad_index, "bad_index", torch.int32, 1)
    if tuple(residual_out.shape) != (T, H) or tuple(normed_out.shape) != (T, H):
        raise ValueError("outputs must be [T, H]")
    if bad_index.numel() < 1:
        raise ValueError("bad_index must hold one int32")
    _same_device(expert_out, perm_idx, topk_w, shared_out, residual, gamma, residual_out,
                 normed_out, bad_index)
    stream, ctx = _launch_context(dev, stream)
    with ctx:
        rc = _lib.moe_finalize_rmsnorm_checked(
            expert_out.data_ptr(), R, perm_idx.data_ptr(), topk_w.data_ptr(),
            shared_out.data_ptr(), residual.data_ptr(), gamma.data_ptr(), float(eps),
            float(scale), residual_out.data_ptr(), normed_out.data_ptr(), bad_index.data_ptr(),
            T, H, K, stream.cuda_stream)
    if rc != MFR_OK:
        raise MFRError(rc)
    return residual_out, normed_out, bad_index


def moe_finalize_rmsnorm_fp8_checked_raw(expert_out, R, perm_idx, topk_w, shared_out, residual,
                                         gamma, eps, scale, residual_out, normed_out, normed_fp8,
                                         fp8_scale, bad_index, T, H, K, stream):
    """Direct C call with integer addresses (normed_out and bad_index may be
    0/None); returns the status."""
    return _lib.moe_finalize_rmsnorm_fp8_checked(
        expert_out, int(R), perm_idx, topk_w, shared_out, residual, gamma, float(eps),
        float(scale), residual_out, normed_out or None, normed_fp8, fp8_scale, bad_index or None,
        int(T), int(H), int(K), stream)


def moe_finalize_rmsnorm_fp8_checked(expert_out, perm_idx, topk_w, shared_out, residual, gamma,
                                     eps, scale, residual_out=None, normed_fp8=None,
                                     fp8_scale=None, bf16_normed=False, normed_out=None,
                                     bad_index=None, stream=None):
    """moe_finalize_rmsnorm_fp8 told R = expert_out.shape[0]: a slot whose
    index is at or past R is treated as masked, and bad_index (a one-element
    int32 GPU tensor, allocated zeroed when not given) is set to 1 if any
    token holds such an index. Returns (residual_out, normed_fp8, fp8_scale,
    normed_out or None, bad_index)."""
    _check(expert_out, "expert_out", torch.bfloat16, 2)
    _check(perm_idx, "perm_idx", torch.int32, 2)
    _check(topk_w, "topk_w", torch.float32, 2)
    _check(shared_out, "shared_out", torch.bfloat16, 2)
    _check(residual, "residual", torch.bfloat16, 2)
    _check(gamma, "gamma", torch.bfloat16, 1)
    T, K = perm_idx.shape
    H = gamma.shape[0]
    R = expert_out.shape[0]
    if expert_out.shape[1] != H or tuple(shared_out.shape) != (T, H) or \
            tuple(residual.shape) != (T, H) or tuple(topk_w.shape) != (T, K):
        raise ValueError("inconsistent shapes")
    dev = residual.device
    residual_out, normed_fp8, fp8_scale, normed_out = _fp8_outputs(
        T, H, dev, residual_out, normed_fp8, fp8_scale, normed_out, bf16_normed)
    if bad_index is None:
        bad_index = torch.zeros((1,), dtype=torch.int32, device=dev)
    _check(bad_index, "bad_index", torch.int32, 1)
    if bad_index.numel() < 1:
        raise ValueError("bad_index must hold one int32")
    _same_device(expert_out, perm_idx, topk_w, shared_out, residual, gamma, residual_out,
                 normed_fp8, fp8_scale, normed_out, bad_index)
    stream, ctx = _launch_context(dev, stream)
    with ctx:
        rc = _lib.moe_finalize_rmsnorm_fp8_checked(
            expert_out.data_ptr(), R, perm_idx.data_ptr(), topk_w.data_ptr(),
            shared_out.data_ptr(), residual.data_ptr(), gamma.data_ptr(), float(eps),
            float(scale), residual_out.data_ptr(),
            normed_out.data_ptr() if normed_out is not None else None, normed_fp8.data_ptr(),
            fp8_scale.data_ptr(), bad_index.data_ptr(), T, H, K, stream.cuda_stream)
    if rc != MFR_OK:
        raise MFRError(rc)
    return residual_out, normed_fp8, fp8_scale, normed_out, bad_index


def residual_add_rmsnorm_raw(x, residual, gamma, eps, residual_out, normed_out, T, H, stream):
    """Direct C call with integer addresses; returns the status code."""
    return _lib.residual_add_rmsnorm(x, residual, gamma, float(eps), residual_out, normed_out,
                                     int(T), int(H), stream)


def residual_add_rmsnorm(x, residual, gamma, eps, residual_out=None, normed_out=None, stream=None):
    """Dense residual add + RMSNorm (no routed part) on the current (or given) stream.

    x / residual [T, H] bf16, gamma [H] bf16. Outputs are allocated when not
    given; residual_out may be `residual` itself. Returns (residual_out, normed_out).
    """
    _check(x, "x", torch.bfloat16, 2)
    _check(residual, "residual", torch.bfloat16, 2)
    _check(gamma, "gamma", torch.bfloat16, 1)
    T, H = x.shape
    if tuple(residual.shape) != (T, H) or gamma.shape[0] != H:
        raise ValueError("x and residual must be [T, H] and gamma [H]")
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if normed_out is None:
        normed_out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _check(residual_out, "residual_out", torch.bfloat16, 2)
    _check(normed_out, "normed_out", torch.bfloat16, 2)
    if tuple(residual_out.shape) != (T, H) or tuple(normed_out.shape) != (T, H):
        raise ValueError("outputs must be [T, H]")
    _same_device(x, residual, gamma, residual_out, normed_out)
    stream, ctx = _launch_context(x.device, stream)
    with ctx:
        rc = _lib.residual_add_rmsnorm(x.data_ptr(), residual.data_ptr(), gamma.data_ptr(),
                                       float(eps), residual_out.data_ptr(), normed_out.data_ptr(),
                                       T, H, stream.cuda_stream)
    if rc != MFR_OK:
        raise MFRError(rc)
    return residual_out, normed_out


def _fp8_outputs(T, H, dev, residual_out, normed_fp8, fp8_scale, normed_out, bf16_normed):
    """Allocates the outputs of an FP8-output call that were not given and
    checks all of them: residual_out [T, H] bf16, normed_fp8 [T, H] E4M3 (or
    uint8), fp8_scale [T] fp32, and normed_out [T, H] bf16 when it is written
    (given, or asked for with bf16_normed)."""
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if normed_fp8 is None:
        normed_fp8 = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=dev)
    if fp8_scale is None:
        fp8_scale = torch.empty((T,), dtype=torch.float32, device=dev)
    if normed_out is None and bf16_normed:
        normed_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(residual_out, "residual_out", torch.bfloat16, 2)
    if normed_fp8.dtype not in (torch.float8_e4m3fn, torch.uint8) or not normed_fp8.is_cuda or \
            not normed_fp8.is_contiguous() or tuple(normed_fp8.shape) != (T, H):
        raise ValueError("normed_fp8 must be a contiguous [T, H] float8_e4m3fn (or uint8) GPU tensor")
    if tuple(residual_out.shape) != (T, H):
        raise ValueError("residual_out must be [T, H]")
    _check(fp8_scale, "fp8_scale", torch.float32, 1)
    if tuple(fp8_scale.shape) != (T,):
        raise ValueError(f"fp8_scale has shape {tuple(fp8_scale.shape)}, expected {(T,)}")
    if normed_out is not None:
        _check(normed_out, "normed_out", torch.bfloat16, 2)
        if tuple(normed_out.shape) != (T, H):
            raise ValueError("normed_out must be [T, H]")
    return residual_out, normed_fp8, fp8_scale, normed_out


def moe_finalize_rmsnorm_fp8_raw(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                                 scale, residual_out, normed_out, normed_fp8, fp8_scale, T, H, K,
                                 stream):
    """Direct C call with integer addresses (normed_out may be 0/None); returns the status."""
    return _lib.moe_finalize_rmsnorm_fp8(expert_out, perm_idx, topk_w, shared_out, residual, gamma,
                                         float(eps), float(scale), residual_out, normed_out or None,
                                         normed_fp8, fp8_scale, int(T), int(H), int(K), stream)


def moe_finalize_rmsnorm_fp8(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale,
                             residual_out=None, normed_fp8=None, fp8_scale=None, bf16_normed=False,
                             normed_out=None, stream=None):
    """The fused op with the normalised output as dynamic per-token FP8 (E4M3).

    Returns (residual_out, normed_fp8 [T, H] torch.float8_e4m3fn, fp8_scale [T]
    float32, normed_out or None). The bf16 normed output is written only when
    bf16_normed is true or normed_out is given.
    """
    _check(expert_out, "expert_out", torch.bfloat16, 2)
    _check(perm_idx, "perm_idx", torch.int32, 2)
    _check(topk_w, "topk_w", torch.float32, 2)
    _check(shared_out, "shared_out", torch.bfloat16, 2)
    _check(residual, "residual", torch.bfloat16, 2)
    _check(gamma, "gamma", torch.bfloat16, 1)
    T, K = perm_idx.shape
    H = gamma.shape[0]
    if expert_out.shape[1] != H or tuple(shared_out.shape) != (T, H) or \
            tuple(residual.shape) != (T, H) or tuple(topk_w.shape) != (T, K):
        raise ValueError("inconsistent shapes")
    dev = residual.device
    residual_out, normed_fp8, fp8_scale, normed_out = _fp8_outputs(
        T, H, dev, residual_out, normed_fp8, fp8_scale, normed_out, bf16_normed)
    _same_device(expert_out, perm_idx, topk_w, shared_out, residual, gamma, residual_out,
                 normed_fp8, fp8_scale, normed_out)
    stream, ctx = _launch_context(dev, stream)
    with ctx:
        rc = _lib.moe_finalize_rmsnorm_fp8(
            expert_out.data_ptr(), perm_idx.data_ptr(), topk_w.data_ptr(), shared_out.data_ptr(),
            residual.data_ptr(), gamma.data_ptr(), float(eps), float(scale),
            residual_out.data_ptr(), normed_out.data_ptr() if normed_out is not None else None,
            normed_fp8.data_ptr(), fp8_scale.data_ptr(), T, H, K, stream.cuda_stream)
    if rc != MFR_OK:
        raise MFRError(rc)
    return residual_out, normed_fp8, fp8_scale, normed_out


def residual_add_rmsnorm_fp8_raw(x, residual, gamma, eps, residual_out, normed_out, normed_fp8,
                                 fp8_scale, T, H, stream):
    """Direct C call with integer addresses (normed_out may be 0/None); returns the status."""
    return _lib.residual_add_rmsnorm_fp8(x, residual, gamma, float(eps), residual_out,
                                         normed_out or None, normed_fp8, fp8_scale, int(T), int(H),
                                         stream)


def residual_add_rmsnorm_fp8(x, residual, gamma, eps, residual_out=None, normed_fp8=None,
                             fp8_scale=None, bf16_normed=False, normed_out=None, stream=None):
    """Dense residual add + RMSNorm with the normalised output as dynamic
    per-token FP8 (E4M3).

    x / residual [T, H] bf16, gamma [H] bf16. Returns (residual_out, normed_fp8
    [T, H] torch.float8_e4m3fn, fp8_scale [T] float32, normed_out or None); the
    bf16 normed output is written only when bf16_normed is true or normed_out
    is given. residual_out may be `residual` itself.
    """
    _check(x, "x", torch.bfloat16, 2)
    _check(residual, "residual", torch.bfloat16, 2)
    _check(gamma, "gamma", torch.bfloat16, 1)
    T, H = x.shape
    if tuple(residual.shape) != (T, H) or gamma.shape[0] != H:
        raise ValueError("inconsistent shapes")
    dev = residual.device
    residual_out, normed_fp8, fp8_scale, normed_out = _fp8_outputs(
        T, H, dev, residual_out, normed_fp8, fp8_scale, normed_out, bf16_normed)
    _same_device(x, residual, gamma, residual_out, normed_fp8, fp8_scale, normed_out)
    stream, ctx = _launch_context(dev, stream)
    with ctx:
        rc = _lib.residual_add_rmsnorm_fp8(
            x.data_ptr(), residual.data_ptr(), gamma.data_ptr(), float(eps),
            residual_out.data_ptr(), normed_out.data_ptr() if normed_out is not None else None,
            normed_fp8.data_ptr(), fp8_scale.data_ptr(), T, H, stream.cuda_stream)
    if rc != MFR_OK:
        raise MFRError(rc)
    return residual_out, normed_fp8, fp8_scale, normed_out
