"""Oracle: plain fp64 CPU definition of the fused MoE finalize + RMSNorm.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library never
imports it and it never imports the GPU library; they share no code.

The arithmetic lives in ``mfr_oracle.cpp`` (single-threaded C++17, fp64, one
rounding to bf16 per output). This module only marshals numpy arrays into it.
Source of the definitions: vLLM pull request #62174 (deferred MoE finalize for
GLM-5.x), sections Details and Validation, for finalize_rmsnorm; "Port the
validated GLM-5.2 H200 production path to latest vLLM", Ported behavior, for
the dense residual_rmsnorm, and Prepared experiment branches (dynamic
per-token FP8 activations) for fp8_quantize_rows. The header of
``mfr_oracle.cpp`` lists the readings taken where the pages are silent.

Parity pins: every function here is pinned by tests/test_oracle.py (hand cases,
closed forms, invariants, library special cases, exact brute force); none is
"parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build


class OracleIndexError(IndexError):
    """A non-negative permutation index is outside the rows of expert_out."""


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Handle on one build of the oracle library (the default build, or a
    test-built variant of the same source)."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.mfr_oracle_finalize_rmsnorm.restype = ctypes.c_int
        lib.mfr_oracle_finalize_rmsnorm.argtypes = [
            p, i64, p, p, p, p, p, ctypes.c_float, ctypes.c_float,
            i64, i64, i64, p, p, p, p,
        ]
        lib.mfr_oracle_residual_rmsnorm.restype = ctypes.c_int
        lib.mfr_oracle_residual_rmsnorm.argtypes = [p, p, p, ctypes.c_float, i64, i64, p, p, p, p]
        lib.mfr_oracle_fp8_quantize_rows.restype = None
        lib.mfr_oracle_fp8_quantize_rows.argtypes = [p, i64, i64, p, p, p]
        lib.mfr_oracle_rne_e4m3_from_f64.restype = None
        lib.mfr_oracle_rne_e4m3_from_f64.argtypes = [p, i64, p]
        lib.mfr_oracle_rne_bf16_from_f64.restype = None
        lib.mfr_oracle_rne_bf16_from_f64.argtypes = [p, i64, p]
        self.path = path
        self._lib = lib

    def finalize_rmsnorm(self, expert_out, perm_idx, topk_w, shared_out, residual, gamma,
                         eps, scale, want_exact=True):
        """Evaluate the fused op on host arrays.

        expert_out: uint16 [R, H] (bf16 bits); perm_idx: int32 [T, K];
        topk_w: float32 [T, K]; shared_out, residual: uint16 [T, H];
        gamma: uint16 [H]; eps, scale: fp32 values.
        Returns a dict with residual_out, normed_out (uint16 [T, H]) and, when
        want_exact, s and normed_exact (float64 [T, H], the unrounded values).
        """
        E = np.ascontiguousarray(expert_out, dtype=np.uint16)
        P = np.ascontiguousarray(perm_idx, dtype=np.int32)
        W = np.ascontiguousarray(topk_w, dtype=np.float32)
        S = np.ascontiguousarray(shared_out, dtype=np.uint16)
        X = np.ascontiguousarray(residual, dtype=np.uint16)
        G = np.ascontiguousarray(gamma, dtype=np.uint16)
        if P.ndim != 2:
            raise ValueError("perm_idx must be [T, K]")
        T, K = P.shape
        H = G.shape[0]
        R = E.shape[0] if E.ndim == 2 else 0
        if E.ndim == 2 and R > 0 and E.shape[1] != H:
            raise ValueError("expert_out width differs from gamma length")
        for name, a in (("shared_out", S), ("residual", X)):
            if a.shape != (T, H):
                raise ValueError(f"{name} has shape {a.shape}, expected {(T, H)}")
        if W.shape != (T, K):
            raise ValueError("topk_w shape differs from perm_idx shape")
        res_out = np.empty((T, H), dtype=np.uint16)
        nrm_out = np.empty((T, H), dtype=np.uint16)
        s = np.empty((T, H), dtype=np.float64) if want_exact else None
        ne = np.empty((T, H), dtype=np.float64) if want_exact else None
        if E.size == 0:
            E = np.zeros(1, dtype=np.uint16)  # R == 0: never read
        rc = self._lib.mfr_oracle_finalize_rmsnorm(
            _ptr(E), R, _ptr(P), _ptr(W), _ptr(S), _ptr(X), _ptr(G),
            float(np.float32(eps)), float(np.float32(scale)), T, H, K,
            _ptr(res_out), _ptr(nrm_out),
            _ptr(s) if want_exact else None, _ptr(ne) if want_exact else None)
        if rc == 2:
            raise OracleIndexError("perm_idx holds an index >= rows of expert_out")
        if rc != 0:
            raise ValueError(f"oracle rejected the shapes (status {rc})")
        out = {"residual_out": res_out, "normed_out": nrm_out}
        if want_exact:
            out["s"] = s
            out["normed_exact"] = ne
        return out

    def residual_rmsnorm(self, x, residual, gamma, eps, want_exact=True):
        """Dense residual add + RMSNorm (no routed part) on host arrays.

        x, residual: uint16 [T, H] (bf16 bits); gamma: uint16 [H]; eps: fp32 value.
        Same outputs as finalize_rmsnorm.
        """
        X = np.ascontiguousarray(x, dtype=np.uint16)
        R = np.ascontiguousarray(residual, dtype=np.uint16)
        G = np.ascontiguousarray(gamma, dtype=np.uint16)
        if X.ndim != 2 or R.shape != X.shape or G.shape != (X.shape[1],):
            raise ValueError("x and residual must be [T, H] and gamma [H]")
        T, H = X.shape
        res_out = np.empty((T, H), dtype=np.uint16)
        nrm_out = np.empty((T, H), dtype=np.uint16)
        s = np.empty((T, H), dtype=np.float64) if want_exact else None
        ne = np.empty((T, H), dtype=np.float64) if want_exact else None
        rc = self._lib.mfr_oracle_residual_rmsnorm(
            _ptr(X), _ptr(R), _ptr(G), float(np.float32(eps)), T, H, _ptr(res_out), _ptr(nrm_out),
            _ptr(s) if want_exact else None, _ptr(ne) if want_exact else None)
        if rc != 0:
            raise ValueError(f"oracle rejected the shapes (status {rc})")
        out = {"residual_out": res_out, "normed_out": nrm_out}
        if want_exact:
            out["s"] = s
            out["normed_exact"] = ne
        return out

    def fp8_quantize_rows(self, y):
        """Dynamic per-row E4M3 quantisation of float64 rows [T, H].

        Returns (codes uint8 [T, H], scales float64 [T], scaled float64 [T, H]),
        where scaled = y / scale before rounding.
        """
        Y = np.ascontiguousarray(y, dtype=np.float64)
        if Y.ndim != 2:
            raise ValueError("y must be [T, H]")
        T, H = Y.shape
        codes = np.empty((T, H), dtype=np.uint8)
        scales = np.empty(T, dtype=np.float64)
        scaled = np.empty((T, H), dtype=np.float64)
        self._lib.mfr_oracle_fp8_quantize_rows(_ptr(Y), T, H, _ptr(codes), _ptr(scales), _ptr(scaled))
        return codes, scales, scaled

    def rne_e4m3_from_f64(self, x):
        """Round float64 values to E4M3 codes (ties to even, saturating at 448)."""
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint8)
        self._lib.mfr_oracle_rne_e4m3_from_f64(_ptr(a), a.size, _ptr(out))
        return out

    def rne_bf16_from_f64(self, x):
        """Round float64 values to bf16 bit patterns (ties to even), elementwise."""
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self._lib.mfr_oracle_rne_bf16_from_f64(_ptr(a), a.size, _ptr(out))
        return out


_default = None


def default():
    """The oracle built from mfr_oracle.cpp (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def finalize_rmsnorm(*args, **kwargs):
    return default().finalize_rmsnorm(*args, **kwargs)


def residual_rmsnorm(*args, **kwargs):
    return default().residual_rmsnorm(*args, **kwargs)


def fp8_quantize_rows(y):
    return default().fp8_quantize_rows(y)


def rne_e4m3_from_f64(x):
    return default().rne_e4m3_from_f64(x)


def rne_bf16_from_f64(x):
    return default().rne_bf16_from_f64(x)
