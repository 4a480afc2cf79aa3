"""Python binding of libmoe_finalize_rmsnorm.so (ctypes; argument marshalling only).

Every step of the op runs in the HIP library. torch supplies device memory and
the current stream. There is no CPU fallback: if the library is missing,
importing this module raises.

The tensor-level calls of the fused op (moe_finalize_rmsnorm and
moe_finalize_rmsnorm_fp8) go through the library's checked entry points, told
R = expert_out.shape[0]: an index that a faulty producer left at or past R is
then treated as masked (and reported when a flag tensor is passed) instead of
being read outside expert_out. The *_raw functions are the plain C calls on
integer addresses, for C-level callers and the benchmark.

The checks here are the ones the library cannot make from raw pointers:
dtype (it sets the element size the kernels address with), shape (T, H, K and
R come from the tensors), device and contiguity. Alignment, overlap, scalar
values and the shape limits are checked by the library, which refuses a call
with a status code before anything is enqueued.
"""
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
PATH_PERSIST = 3

LIB_PATH = _build.LIB
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run top_finalize_residual_amd/build.py (hipcc, gfx950) first")
_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_f = ctypes.c_float
_lib.moe_finalize_rmsnorm.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm.argtypes = [_p, _p, _p, _p, _p, _p, _f, _f, _p, _p, _i64, _i64, _i64, _p]
_lib.moe_finalize_rmsnorm_path.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_path.argtypes = [_i64, _i64, _i64]
_lib.moe_finalize_rmsnorm_strerror.restype = ctypes.c_char_p
_lib.moe_finalize_rmsnorm_strerror.argtypes = [ctypes.c_int]
_lib.moe_finalize_rmsnorm_fp8.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_fp8.argtypes = [_p, _p, _p, _p, _p, _p, _f, _f, _p, _p, _p, _p, _i64,
                                          _i64, _i64, _p]
_lib.residual_add_rmsnorm.restype = ctypes.c_int
_lib.residual_add_rmsnorm.argtypes = [_p, _p, _p, _f, _p, _p, _i64, _i64, _p]
_lib.residual_add_rmsnorm_fp8.restype = ctypes.c_int
_lib.residual_add_rmsnorm_fp8.argtypes = [_p, _p, _p, _f, _p, _p, _p, _p, _i64, _i64, _p]
_lib.moe_finalize_rmsnorm_checked.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_checked.argtypes = [_p, _i64, _p, _p, _p, _p, _p, _f, _f, _p, _p, _p,
                                              _i64, _i64, _i64, _p]
_lib.moe_finalize_rmsnorm_fp8_checked.restype = ctypes.c_int
_lib.moe_finalize_rmsnorm_fp8_checked.argtypes = [_p, _i64, _p, _p, _p, _p, _p, _f, _f, _p, _p,
                                                  _p, _p, _p, _i64, _i64, _i64, _p]

_BF16, _I32, _F32 = torch.bfloat16, torch.int32, torch.float32
_FP8_CODES = (torch.float8_e4m3fn, torch.uint8)
# dtypes of (expert_out, perm_idx, topk_w, shared_out, residual, gamma)
_MOE_IN = (_BF16, _I32, _F32, _BF16, _BF16, _BF16)
_MOE_NAMES = ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma")
_current_stream = torch._C._cuda_getCurrentRawStream
_current_device = torch._C._cuda_getDevice


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


# ---------------------------------------------------------------------------
# argument checks
# ---------------------------------------------------------------------------

def _fail_dtype(names, tensors, dtypes):
    for name, t, want in zip(names, tensors, dtypes):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in (want if isinstance(want, tuple) else (want,)):
            raise TypeError(f"{name} must be {want}, got {t.dtype}")
    raise TypeError("unexpected dtype")


def _check_dtypes(names, tensors, dtypes):
    try:
        got = tuple(t.dtype for t in tensors)
    except AttributeError:
        _fail_dtype(names, tensors, dtypes)
    if got != dtypes:
        _fail_dtype(names, tensors, dtypes)


def _device_of(names, tensors):
    """The GPU index all tensors live on; every tensor contiguous."""
    dev = tensors[0].get_device()
    for name, t in zip(names, tensors):
        if t.get_device() != dev or dev < 0:
            if dev < 0 or t.get_device() < 0:
                raise ValueError(f"{name} must be on the GPU, got {t.device}")
            raise ValueError(f"all tensors must be on one GPU, {name} is on {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return dev


def _shape(name, t, want):
    if t.shape != want:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")


def _moe_shapes(expert_out, perm_idx, topk_w, shared_out, residual, gamma):
    """(T, H, K, R) of the fused op's inputs, checked against each other."""
    if perm_idx.dim() != 2 or gamma.dim() != 1 or expert_out.dim() != 2:
        raise ValueError("perm_idx must be [T, K], gamma [H] and expert_out [R, H]")
    T, K = perm_idx.shape
    H = gamma.shape[0]
    R = expert_out.shape[0]
    if expert_out.shape[1] != H:
        raise ValueError("expert_out width differs from gamma length")
    _shape("topk_w", topk_w, (T, K))
    _shape("shared_out", shared_out, (T, H))
    _shape("residual", residual, (T, H))
    return T, H, K, R


def _launch(dev, stream, fn, *args):
    """Call the library on the tensors' GPU and its current (or the given)
    stream; the library launches on the calling thread's current device."""
    if stream is not None:
        if stream.device_index != dev:
            raise ValueError(f"stream is on cuda:{stream.device_index}, the tensors on cuda:{dev}")
        s = stream.cuda_stream
    else:
        s = _current_stream(dev)
    if dev == _current_device():
        rc = fn(*args, s)
    else:
        with torch.cuda.device(dev):
            rc = fn(*args, s)
    if rc != MFR_OK:
        raise MFRError(rc)


def _ptr(t):
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------------------
# raw C calls (integer addresses; return the status)
# ---------------------------------------------------------------------------

def moe_finalize_rmsnorm_raw(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                             scale, residual_out, normed_out, T, H, K, stream):
    """Direct C call with integer addresses; returns the status code."""
    return _lib.moe_finalize_rmsnorm(expert_out, perm_idx, topk_w, shared_out, residual, gamma,
                                     float(eps), float(scale), residual_out, normed_out,
                                     int(T), int(H), int(K), stream)


def moe_finalize_rmsnorm_checked_raw(expert_out, R, perm_idx, topk_w, shared_out, residual, gamma,
                                     eps, scale, residual_out, normed_out, bad_index, T, H, K,
                                     stream):
    """Direct C call of the checked entry point (bad_index may be 0/None)."""
    return _lib.moe_finalize_rmsnorm_checked(expert_out, int(R), perm_idx, topk_w, shared_out,
                                             residual, gamma, float(eps), float(scale),
                                             residual_out, normed_out, bad_index or None,
                                             int(T), int(H), int(K), stream)


def moe_finalize_rmsnorm_fp8_raw(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                                 scale, residual_out, normed_out, normed_fp8, fp8_scale, T, H, K,
                                 stream):
    """Direct C call with integer addresses (normed_out may be 0/None); returns the status."""
    return _lib.moe_finalize_rmsnorm_fp8(expert_out, perm_idx, topk_w, shared_out, residual, gamma,
                                         float(eps), float(scale), residual_out, normed_out or None,
                                         normed_fp8, fp8_scale, int(T), int(H), int(K), stream)


def moe_finalize_rmsnorm_fp8_checked_raw(expert_out, R, perm_idx, topk_w, shared_out, residual,
                                         gamma, eps, scale, residual_out, normed_out, normed_fp8,
                                         fp8_scale, bad_index, T, H, K, stream):
    """Direct C call with integer addresses (normed_out and bad_index may be
    0/None); returns the status."""
    return _lib.moe_finalize_rmsnorm_fp8_checked(
        expert_out, int(R), perm_idx, topk_w, shared_out, residual, gamma, float(eps),
        float(scale), residual_out, normed_out or None, normed_fp8, fp8_scale, bad_index or None,
        int(T), int(H), int(K), stream)


def residual_add_rmsnorm_raw(x, residual, gamma, eps, residual_out, normed_out, T, H, stream):
    """Direct C call with integer addresses; returns the status code."""
    return _lib.residual_add_rmsnorm(x, residual, gamma, float(eps), residual_out, normed_out,
                                     int(T), int(H), stream)


def residual_add_rmsnorm_fp8_raw(x, residual, gamma, eps, residual_out, normed_out, normed_fp8,
                                 fp8_scale, T, H, stream):
    """Direct C call with integer addresses (normed_out may be 0/None); returns the status."""
    return _lib.residual_add_rmsnorm_fp8(x, residual, gamma, float(eps), residual_out,
                                         normed_out or None, normed_fp8, fp8_scale, int(T), int(H),
                                         stream)


# ---------------------------------------------------------------------------
# tensor-level calls
# ---------------------------------------------------------------------------

def _bf16_outputs(T, H, ref, residual_out, normed_out):
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=_BF16, device=ref.device)
    if normed_out is None:
        normed_out = torch.empty((T, H), dtype=_BF16, device=ref.device)
    _check_dtypes(("residual_out", "normed_out"), (residual_out, normed_out), (_BF16, _BF16))
    _shape("residual_out", residual_out, (T, H))
    _shape("normed_out", normed_out, (T, H))
    return residual_out, normed_out


def _bad_index(ref, bad_index):
    if bad_index is None:
        return None
    _check_dtypes(("bad_index",), (bad_index,), (_I32,))
    if bad_index.dim() != 1 or bad_index.shape[0] < 1:
        raise ValueError("bad_index must be a one-dimensional int32 tensor of at least one element")
    return bad_index


def moe_finalize_rmsnorm(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale,
                         residual_out=None, normed_out=None, bad_index=None, stream=None):
    """Fused MoE finalize + residual add + RMSNorm on the current (or given) stream.

    expert_out [R, H] bf16, perm_idx [T, K] int32 (-1 = masked), topk_w [T, K] fp32,
    shared_out / residual [T, H] bf16, gamma [H] bf16; eps, scale are floats.
    residual_out / normed_out ([T, H] bf16) are allocated when not given;
    residual_out may be `residual` itself. An index at or past R is treated
    as masked; bad_index (an int32 GPU tensor, optional) is set to 1 when one
    occurs (never cleared). Returns (residual_out, normed_out).
    """
    ins = (expert_out, perm_idx, topk_w, shared_out, residual, gamma)
    _check_dtypes(_MOE_NAMES, ins, _MOE_IN)
    T, H, K, R = _moe_shapes(*ins)
    residual_out, normed_out = _bf16_outputs(T, H, residual, residual_out, normed_out)
    bad_index = _bad_index(residual, bad_index)
    ts = ins + (residual_out, normed_out) + (() if bad_index is None else (bad_index,))
    dev = _device_of(_MOE_NAMES + ("residual_out", "normed_out", "bad_index"), ts)
    _launch(dev, stream, _lib.moe_finalize_rmsnorm_checked, expert_out.data_ptr(), R,
            perm_idx.data_ptr(), topk_w.data_ptr(), shared_out.data_ptr(), residual.data_ptr(),
            gamma.data_ptr(), eps, scale, residual_out.data_ptr(), normed_out.data_ptr(),
            _ptr(bad_index), T, H, K)
    return residual_out, normed_out


def moe_finalize_rmsnorm_checked(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                                 scale, residual_out=None, normed_out=None, bad_index=None,
                                 stream=None):
    """moe_finalize_rmsnorm with the out-of-range flag always present:
    bad_index (a one-element int32 GPU tensor) is allocated zeroed when not
    given, and set to 1 if any token holds an index at or past R. Returns
    (residual_out, normed_out, bad_index)."""
    if bad_index is None:
        bad_index = torch.zeros((1,), dtype=_I32, device=residual.device)
    r, n = moe_finalize_rmsnorm(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                                scale, residual_out, normed_out, bad_index, stream)
    return r, n, bad_index


def _fp8_outputs(T, H, ref, residual_out, normed_fp8, fp8_scale, normed_out, bf16_normed):
    """Allocates the outputs of an FP8-output call that were not given and
    checks all of them: residual_out [T, H] bf16, normed_fp8 [T, H] E4M3 (or
    uint8), fp8_scale [T] fp32, and normed_out [T, H] bf16 when it is written
    (given, or asked for with bf16_normed)."""
    dev = ref.device
    if residual_out is None:
        residual_out = torch.empty((T, H), dtype=_BF16, device=dev)
    if normed_fp8 is None:
        normed_fp8 = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=dev)
    if fp8_scale is None:
        fp8_scale = torch.empty((T,), dtype=_F32, device=dev)
    if normed_out is None and bf16_normed:
        normed_out = torch.empty((T, H), dtype=_BF16, device=dev)
    _check_dtypes(("residual_out", "fp8_scale"), (residual_out, fp8_scale), (_BF16, _F32))
    if not isinstance(normed_fp8, torch.Tensor) or normed_fp8.dtype not in _FP8_CODES:
        raise ValueError("normed_fp8 must be a float8_e4m3fn (or uint8) tensor")
    _shape("residual_out", residual_out, (T, H))
    _shape("normed_fp8", normed_fp8, (T, H))
    _shape("fp8_scale", fp8_scale, (T,))
    if normed_out is not None:
        _check_dtypes(("normed_out",), (normed_out,), (_BF16,))
        _shape("normed_out", normed_out, (T, H))
    return residual_out, normed_fp8, fp8_scale, normed_out


def moe_finalize_rmsnorm_fp8(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps, scale,
                             residual_out=None, normed_fp8=None, fp8_scale=None, bf16_normed=False,
                             normed_out=None, bad_index=None, stream=None):
    """The fused op with the normalised output as dynamic per-token FP8 (E4M3).

    Returns (residual_out, normed_fp8 [T, H] torch.float8_e4m3fn, fp8_scale [T]
    float32, normed_out or None). The bf16 normed output is written only when
    bf16_normed is true or normed_out is given. An index at or past R is
    treated as masked, and sets bad_index (optional int32 GPU tensor) to 1.
    """
    ins = (expert_out, perm_idx, topk_w, shared_out, residual, gamma)
    _check_dtypes(_MOE_NAMES, ins, _MOE_IN)
    T, H, K, R = _moe_shapes(*ins)
    residual_out, normed_fp8, fp8_scale, normed_out = _fp8_outputs(
        T, H, residual, residual_out, normed_fp8, fp8_scale, normed_out, bf16_normed)
    bad_index = _bad_index(residual, bad_index)
    ts = ins + (residual_out, normed_fp8, fp8_scale)
    names = _MOE_NAMES + ("residual_out", "normed_fp8", "fp8_scale")
    if normed_out is not None:
        ts, names = ts + (normed_out,), names + ("normed_out",)
    if bad_index is not None:
        ts, names = ts + (bad_index,), names + ("bad_index",)
    dev = _device_of(names, ts)
    _launch(dev, stream, _lib.moe_finalize_rmsnorm_fp8_checked, expert_out.data_ptr(), R,
            perm_idx.data_ptr(), topk_w.data_ptr(), shared_out.data_ptr(), residual.data_ptr(),
            gamma.data_ptr(), eps, scale, residual_out.data_ptr(), _ptr(normed_out),
            normed_fp8.data_ptr(), fp8_scale.data_ptr(), _ptr(bad_index), T, H, K)
    return residual_out, normed_fp8, fp8_scale, normed_out


def moe_finalize_rmsnorm_fp8_checked(expert_out, perm_idx, topk_w, shared_out, residual, gamma,
                                     eps, scale, residual_out=None, normed_fp8=None,
                                     fp8_scale=None, bf16_normed=False, normed_out=None,
                                     bad_index=None, stream=None):
    """moe_finalize_rmsnorm_fp8 with the out-of-range flag always present
    (allocated zeroed when not given). Returns (residual_out, normed_fp8,
    fp8_scale, normed_out or None, bad_index)."""
    if bad_index is None:
        bad_index = torch.zeros((1,), dtype=_I32, device=residual.device)
    out = moe_finalize_rmsnorm_fp8(expert_out, perm_idx, topk_w, shared_out, residual, gamma, eps,
                                   scale, residual_out, normed_fp8, fp8_scale, bf16_normed,
                                   normed_out, bad_index, stream)
    return out + (bad_index,)


_DENSE_NAMES = ("x", "residual", "gamma")


def _dense_shapes(x, residual, gamma):
    if x.dim() != 2 or gamma.dim() != 1:
        raise ValueError("x and residual must be [T, H] and gamma [H]")
    T, H = x.shape
    _shape("residual", residual, (T, H))
    _shape("gamma", gamma, (H,))
    return T, H


def residual_add_rmsnorm(x, residual, gamma, eps, residual_out=None, normed_out=None, stream=None):
    """Dense residual add + RMSNorm (no routed part) on the current (or given) stream.

    x / residual [T, H] bf16, gamma [H] bf16. Outputs are allocated when not
    given; residual_out may be `residual` itself. Returns (residual_out, normed_out).
    """
    ins = (x, residual, gamma)
    _check_dtypes(_DENSE_NAMES, ins, (_BF16, _BF16, _BF16))
    T, H = _dense_shapes(*ins)
    residual_out, normed_out = _bf16_outputs(T, H, residual, residual_out, normed_out)
    dev = _device_of(_DENSE_NAMES + ("residual_out", "normed_out"), ins + (residual_out, normed_out))
    _launch(dev, stream, _lib.residual_add_rmsnorm, x.data_ptr(), residual.data_ptr(),
            gamma.data_ptr(), eps, residual_out.data_ptr(), normed_out.data_ptr(), T, H)
    return residual_out, normed_out


def residual_add_rmsnorm_fp8(x, residual, gamma, eps, residual_out=None, normed_fp8=None,
                             fp8_scale=None, bf16_normed=False, normed_out=None, stream=None):
    """Dense residual add + RMSNorm with the normalised output as dynamic
    per-token FP8 (E4M3).

    x / residual [T, H] bf16, gamma [H] bf16. Returns (residual_out, normed_fp8
    [T, H] torch.float8_e4m3fn, fp8_scale [T] float32, normed_out or None); the
    bf16 normed output is written only when bf16_normed is true or normed_out
    is given. residual_out may be `residual` itself.
    """
    ins = (x, residual, gamma)
    _check_dtypes(_DENSE_NAMES, ins, (_BF16, _BF16, _BF16))
    T, H = _dense_shapes(*ins)
    residual_out, normed_fp8, fp8_scale, normed_out = _fp8_outputs(
        T, H, residual, residual_out, normed_fp8, fp8_scale, normed_out, bf16_normed)
    ts = ins + (residual_out, normed_fp8, fp8_scale)
    names = _DENSE_NAMES + ("residual_out", "normed_fp8", "fp8_scale")
    if normed_out is not None:
        ts, names = ts + (normed_out,), names + ("normed_out",)
    dev = _device_of(names, ts)
    _launch(dev, stream, _lib.residual_add_rmsnorm_fp8, x.data_ptr(), residual.data_ptr(),
            gamma.data_ptr(), eps, residual_out.data_ptr(), _ptr(normed_out),
            normed_fp8.data_ptr(), fp8_scale.data_ptr(), T, H)
    return residual_out, normed_fp8, fp8_scale, normed_out
