"""Calls so large that one dispatch cannot hold them: T workgroups of 64
threads (H = 8) pass 2^32 work-items once T > 2^26 - 1, and the library
enqueues several dispatches, each starting at a later token.

The inputs repeat with a prime period P, which does not divide the split
point. So every token of the large call must equal, bit for bit, the same
token of one P-token call, and that call is itself checked against the
oracle. Outputs are first filled with an all-ones pattern, so a token that no
dispatch wrote would show up as a mismatch. About 5 GB of device memory.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_finalize_residual_amd as mfr
from tests import gpu_util as gu
from tests.test_fp8_gpu import check_fp8

pytestmark = pytest.mark.gpu

H, K, P = 8, 2, 997
THREADS = 64  # one wave per token at H = 8, on either path
PER_DISPATCH = (2**32 - 1) // THREADS  # 67,108,863 tokens
T = PER_DISPATCH + 3001  # two dispatches: 67,108,863 tokens, then 3,001


def _small():
    return synth.generate(P, H, K, scale=2.5, seed=synth.BASE_SEED + 917)


def _tile(x, T):
    """x [P, ...] repeated along dim 0 to T rows (a contiguous prefix)."""
    reps = -(-T // x.shape[0])
    return x.unsqueeze(0).expand((reps,) + tuple(x.shape)).reshape((-1,) + tuple(x.shape[1:]))[:T]


def _periodic_equal(big, small):
    """Every row t of big equals row t % P of small, bit for bit."""
    q, rem = divmod(big.shape[0], small.shape[0])
    head = big[:q * small.shape[0]].view((q,) + tuple(small.shape))
    return bool((head == small.unsqueeze(0)).all()) and torch.equal(big[q * small.shape[0]:],
                                                                     small[:rem])


def _sentinel(shape, dtype):
    return torch.full(shape, -1, dtype=torch.int16 if dtype == torch.bfloat16 else torch.uint8,
                      device="cuda").view(dtype)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.uint8)


@pytest.fixture(scope="module")
def small():
    d = _small()
    dd = gu.to_device(d)
    return d, dd


def test_split_point_is_crossed():
    assert T * THREADS >= 2**32 and PER_DISPATCH % P != 0
    assert mfr.moe_finalize_rmsnorm_path(T, H, K) == mfr.PATH_STREAM


def test_fused_op_across_dispatches(small):
    d, dd = small
    r0, n0 = mfr.moe_finalize_rmsnorm(*(dd[k] for k in ("expert_out", "perm_idx", "topk_w",
                                                         "shared_out", "residual", "gamma")),
                                      d["eps"], d["scale"])
    torch.cuda.synchronize()
    gu.check(d, gu.host_u16(r0), gu.host_u16(n0))
    print(f"split dispatch: fused op, T={T}, H={H}, K={K}", flush=True)
    big = {k: _tile(dd[k], T) for k in ("perm_idx", "topk_w", "shared_out", "residual")}
    r = _sentinel((T, H), torch.bfloat16)
    n = _sentinel((T, H), torch.bfloat16)
    mfr.moe_finalize_rmsnorm(dd["expert_out"], big["perm_idx"], big["topk_w"], big["shared_out"],
                             big["residual"], dd["gamma"], d["eps"], d["scale"], residual_out=r,
                             normed_out=n)
    torch.cuda.synchronize()
    assert _periodic_equal(_bits(r), _bits(r0)), "residual_out differs from the P-token call"
    assert _periodic_equal(_bits(n), _bits(n0)), "normed_out differs from the P-token call"


def test_fp8_op_across_dispatches(small):
    d, dd = small
    args = [dd[k] for k in ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma")]
    r0, q0, s0, n0 = mfr.moe_finalize_rmsnorm_fp8(*args, d["eps"], d["scale"], bf16_normed=True)
    torch.cuda.synchronize()
    ref = gu.check(d, gu.host_u16(r0), gu.host_u16(n0))
    check_fp8(_bits(q0).cpu().numpy(), s0.cpu().numpy().astype(np.float64), ref, d["gamma"],
              d["eps"])
    print(f"split dispatch: FP8 op, T={T}, H={H}, K={K}", flush=True)
    big = {k: _tile(dd[k], T) for k in ("perm_idx", "topk_w", "shared_out", "residual")}
    r = _sentinel((T, H), torch.bfloat16)
    n = _sentinel((T, H), torch.bfloat16)
    q = _sentinel((T, H), torch.float8_e4m3fn)
    s = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    mfr.moe_finalize_rmsnorm_fp8(dd["expert_out"], big["perm_idx"], big["topk_w"],
                                 big["shared_out"], big["residual"], dd["gamma"], d["eps"],
                                 d["scale"], residual_out=r, normed_fp8=q, fp8_scale=s,
                                 bf16_normed=True, normed_out=n)
    torch.cuda.synchronize()
    assert _periodic_equal(_bits(r), _bits(r0)), "residual_out differs from the P-token call"
    assert _periodic_equal(_bits(n), _bits(n0)), "normed_out differs from the P-token call"
    assert _periodic_equal(_bits(q), _bits(q0)), "codes differ from the P-token call"
    assert _periodic_equal(s.view(torch.int32), s0.view(torch.int32)), "scales differ"


def test_dense_op_across_dispatches(small):
    d, dd = small
    r0, n0 = mfr.residual_add_rmsnorm(dd["shared_out"], dd["residual"], dd["gamma"], d["eps"])
    torch.cuda.synchronize()
    ref = oracle.residual_rmsnorm(d["shared_out"], d["residual"], d["gamma"], d["eps"])
    gu.assert_gate(gu.host_u16(r0), ref["s"], ref["residual_out"], "residual_out")
    gu.assert_gate(gu.host_u16(n0), ref["normed_exact"], ref["normed_out"], "normed_out")
    print(f"split dispatch: dense op, T={T}, H={H}", flush=True)
    x, res = _tile(dd["shared_out"], T), _tile(dd["residual"], T)
    r = _sentinel((T, H), torch.bfloat16)
    n = _sentinel((T, H), torch.bfloat16)
    mfr.residual_add_rmsnorm(x, res, dd["gamma"], d["eps"], residual_out=r, normed_out=n)
    torch.cuda.synchronize()
    assert _periodic_equal(_bits(r), _bits(r0)), "residual_out differs from the P-token call"
    assert _periodic_equal(_bits(n), _bits(n0)), "normed_out differs from the P-token call"
