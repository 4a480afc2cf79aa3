"""Helpers for the GPU parity tests: move synthetic inputs to the device, call
the HIP library through its binding, and compare with the oracle.

The tolerance is the one the op is specified to: every output element within
one bf16 ulp of the oracle's unrounded fp64 value,
    |gpu - ref| <= 2^-8 * |ref| + 1e-6,
plus an ulp distance of at most 1 from the oracle's own bf16 output wherever
|ref| >= 2^-8. Below that the absolute term governs: the fp32 sum carries an
absolute error of order 2^-24 times the magnitude of its addends (about 1e-6
here), which near a cancellation spans many bf16 ulps of the tiny result."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import top_finalize_residual_amd as mfr
from top_finalize_residual_amd import tuning

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


forced = tuning.forced  # force a launch configuration on this thread, automatic after


def run(dd, eps, scale, path=0, vpt=0, store=0, residual_out=None, normed_out=None, api="c",
        residency=0, order=0):
    """One call on device tensors; returns host uint16 (residual_out, normed_out).

    api="c": the plain C entry point moe_finalize_rmsnorm on the tensors'
    addresses (the call the benchmark times); api="binding": the tensor-level
    binding, which goes through the checked entry point with R =
    expert_out.shape[0]."""
    with forced(path, vpt, store, residency, order):
        if api == "binding":
            r, n = mfr.moe_finalize_rmsnorm(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                            dd["shared_out"], dd["residual"], dd["gamma"], eps,
                                            scale, residual_out=residual_out,
                                            normed_out=normed_out)
        else:
            T, K = dd["perm_idx"].shape
            H = dd["gamma"].shape[0]
            r = torch.empty_like(dd["residual"]) if residual_out is None else residual_out
            n = torch.empty_like(dd["residual"]) if normed_out is None else normed_out
            rc = mfr.moe_finalize_rmsnorm_raw(
                *(dd[k].data_ptr() for k in ("expert_out", "perm_idx", "topk_w", "shared_out",
                                             "residual", "gamma")),
                eps, scale, r.data_ptr(), n.data_ptr(), T, H, K,
                torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise mfr.MFRError(rc)
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


def _workers():
    # the oracle's C entry point runs without the interpreter lock, so threads
    # over disjoint token ranges use every core given to the process (at most
    # 16, the CPU share of a one-GPU machine)
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_chunks(T, evaluate, chunk=1024):
    """Yield (t0, t1, ref) over the tokens [0, T) in chunks, where ref is
    evaluate(a, b) (an oracle call on tokens [a, b), returning a dict of
    per-token arrays) computed in threads over disjoint sub-ranges of the
    chunk and joined in token order. Bounded memory at any T."""
    n = _workers()
    with ThreadPoolExecutor(max_workers=n) as ex:
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            bounds = [(t0 + (t1 - t0) * i // n, t0 + (t1 - t0) * (i + 1) // n) for i in range(n)]
            bounds = [b for b in bounds if b[1] > b[0]]
            parts = list(ex.map(lambda b: evaluate(*b), bounds))
            yield t0, t1, {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def finalize_evaluator(d):
    """evaluate(a, b) for oracle_chunks: the oracle's fused op on tokens [a, b)."""
    def evaluate(a, b):
        return oracle.finalize_rmsnorm(d["expert_out"], d["perm_idx"][a:b], d["topk_w"][a:b],
                                       d["shared_out"][a:b], d["residual"][a:b], d["gamma"],
                                       d["eps"], d["scale"])
    return evaluate


def check_all_tokens(d, res_u16, nrm_u16, chunk=1024):
    """check() over every token of a large call, the oracle run in threads
    over token ranges."""
    for t0, t1, ref in oracle_chunks(d["perm_idx"].shape[0], finalize_evaluator(d), chunk):
        check(d, res_u16[t0:t1], nrm_u16[t0:t1], ref=ref)
