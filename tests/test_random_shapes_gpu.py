"""Seeded random sweep of shapes against the oracle: T up to 600, any H that is
a multiple of 8 up to 8192, K from 1 to 16, masked fractions from none to all,
random scale and eps, on the launch path the library chooses. Each shape runs
the fused op (bf16 output), the FP8-output call, its row-checked form, and the
dense tail with both outputs on the shape's shared_out as x. The shapes are
drawn once from a fixed seed, so every run checks the same set."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_finalize_residual_amd as mfr
from tests import gpu_util as gu
from tests.test_fp8_gpu import check_fp8

pytestmark = pytest.mark.gpu


def _shapes(n=80, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([1, 2, 3, 5, 17, 64, 255, 256, 257, 300, 511, 600]))
        H = int(8 * rng.integers(1, 1025))
        K = int(rng.integers(1, 17))
        mask = float(rng.choice([0.0, 0.1, 0.5, 1.0]))
        scale = float(rng.choice([0.5, 1.0, 2.5, 8.0]))
        eps = float(rng.choice([1e-6, 1e-5, 1e-3]))
        out.append((i, T, H, K, mask, scale, eps))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("i,T,H,K,mask,scale,eps", SHAPES,
                         ids=[f"{s[0]}-T{s[1]}-H{s[2]}-K{s[3]}-m{s[4]}" for s in SHAPES])
def test_random_shape(i, T, H, K, mask, scale, eps):
    d = synth.generate(T, H, K, scale=scale, eps=eps, mask_frac=mask, seed=5000 + i,
                       extra_rows=int(i % 3))
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"])
    ref = gu.check(d, r, n)
    rf, q, sc, nf = mfr.moe_finalize_rmsnorm_fp8(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                                 dd["shared_out"], dd["residual"], dd["gamma"],
                                                 d["eps"], d["scale"], bf16_normed=True)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_u16(rf), r) and np.array_equal(gu.host_u16(nf), n)
    check_fp8(q.view(torch.uint8).cpu().numpy(), sc.cpu().numpy().astype(np.float64), ref,
              d["gamma"], d["eps"])
    # the row-checked form, told the true row count: the same outputs, no flag
    rc_, qc, scc, nc, bad = mfr.moe_finalize_rmsnorm_fp8_checked(
        dd["expert_out"], dd["perm_idx"], dd["topk_w"], dd["shared_out"], dd["residual"],
        dd["gamma"], d["eps"], d["scale"], bf16_normed=True)
    torch.cuda.synchronize()
    assert torch.equal(rc_.view(torch.int16), rf.view(torch.int16))
    assert torch.equal(qc.view(torch.uint8), q.view(torch.uint8))
    assert torch.equal(scc.view(torch.int32), sc.view(torch.int32))
    assert torch.equal(nc.view(torch.int16), nf.view(torch.int16)) and int(bad.item()) == 0
    # the dense tail on the same shape: bf16 outputs against its oracle, FP8 codes and scales
    r2, q2, sc2, n2 = mfr.residual_add_rmsnorm_fp8(dd["shared_out"], dd["residual"], dd["gamma"],
                                                   d["eps"], bf16_normed=True)
    torch.cuda.synchronize()
    dref = oracle.residual_rmsnorm(d["shared_out"], d["residual"], d["gamma"], d["eps"])
    gu.assert_gate(gu.host_u16(r2), dref["s"], dref["residual_out"], "dense residual_out")
    gu.assert_gate(gu.host_u16(n2), dref["normed_exact"], dref["normed_out"], "dense normed_out")
    check_fp8(q2.view(torch.uint8).cpu().numpy(), sc2.cpu().numpy().astype(np.float64), dref,
              d["gamma"], d["eps"])
