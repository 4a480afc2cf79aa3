"""Helpers for the GPU parity tests: move synthetic inputs to the device, call
the HIP library through its binding, and compare with the oracle.

The tolerance is the one the op is specified to: every output element within
one bf16 ulp of the oracle's unrounded fp64 value,
    |gpu - ref| <= 2^-8 * |ref| + 1e-6,
plus an ulp distance of at most 1 from the oracle's own bf16 output wherever
|ref| >= 2^-8. Below that the absolute term governs: the fp32 sum carries an
absolute error of order 2^-24 times the magnitude of its addends (about 1e-6
here), which near a cancellation spans many bf16 ulps of the tiny result."""
import numpy as np
import torch

import oracle
import top_finalize_residual_amd as mfr

REL = 2.0 ** -8
ABS = 1e-6
ULP_CHECK_MIN = 2.0 ** -8


def dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).cuda()


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_device(d):
    return dict(expert_out=dev_bf16(d["expert_out"]),
                perm_idx=torch.from_numpy(np.ascontiguousarray(d["perm_idx"])).cuda(),
                topk_w=torch.from_numpy(np.ascontiguousarray(d["topk_w"])).cuda(),
                shared_out=dev_bf16(d["shared_out"]), residual=dev_bf16(d["residual"]),
                gamma=dev_bf16(d["gamma"]))


class forced:
    """Context manager: force a launch configuration, restore automatic after."""

    def __init__(self, path=0, vpt=0, store=0):
        self.args = (path, vpt, store)

    def __enter__(self):
        mfr.moe_finalize_rmsnorm_force(*self.args)
        return self

    def __exit__(self, *exc):
        mfr.moe_finalize_rmsnorm_force(0, 0, 0)
        return False


def run(dd, eps, scale, path=0, vpt=0, store=0, residual_out=None, normed_out=None):
    """One call on device tensors; returns host uint16 (residual_out, normed_out)."""
    with forced(path, vpt, store):
        r, n = mfr.moe_finalize_rmsnorm(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                        dd["shared_out"], dd["residual"], dd["gamma"], eps, scale,
                                        residual_out=residual_out, normed_out=normed_out)
    torch.cuda.synchronize()
    return host_u16(r), host_u16(n)


def bf16_f64(u16):
    with np.errstate(invalid="ignore"):
        return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
            np.float64)


def ulp_key(u16):
    """Monotone integer key of bf16 bit patterns (+0 and -0 map to 0)."""
    b = np.asarray(u16, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def oracle_for(d, tokens=None):
    """Oracle outputs for all tokens, or for the listed token indices."""
    if tokens is None:
        return oracle.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"],
                                       d["shared_out"], d["residual"], d["gamma"], d["eps"],
                                       d["scale"])
    tokens = np.asarray(tokens)
    return oracle.finalize_rmsnorm(d["expert_out"], d["perm_idx"][tokens], d["topk_w"][tokens],
                                   d["shared_out"][tokens], d["residual"][tokens], d["gamma"],
                                   d["eps"], d["scale"])


def assert_gate(gpu_u16, ref_exact, ref_bits, what):
    g = bf16_f64(gpu_u16)
    err = np.abs(g - ref_exact)
    bound = REL * np.abs(ref_exact) + ABS
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements outside the gate; first "
                             f"at {tuple(i)}: gpu {g[tuple(i)]!r} ref {ref_exact[tuple(i)]!r}")
    dist = np.abs(ulp_key(gpu_u16) - ulp_key(ref_bits))
    big = np.abs(ref_exact) >= ULP_CHECK_MIN
    worst = int(dist[big].max(initial=0))
    assert worst <= 1, f"{what}: {worst} ulp from the oracle's bf16 where |ref| >= 2^-8"


def check(d, res_u16, nrm_u16, tokens=None, ref=None):
    """Assert the GPU outputs (all tokens, or the listed ones) pass the gate."""
    if ref is None:
        ref = oracle_for(d, tokens)
    if tokens is not None:
        res_u16, nrm_u16 = res_u16[tokens], nrm_u16[tokens]
    assert_gate(res_u16, ref["s"], ref["residual_out"], "residual_out")
    assert_gate(nrm_u16, ref["normed_exact"], ref["normed_out"], "normed_out")
    return ref
