"""GPU parity of the dense residual add + RMSNorm (no routed part) against its
oracle, plus bit-exact relations to the fused finalize."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_finalize_residual_amd as mfr
from top_finalize_residual_amd import tuning
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run_dense(d, path=0, vpt=0, store=0, residual_out=None, x=None, residual=None):
    x = gu.dev_bf16(d["x"]) if x is None else x
    residual = gu.dev_bf16(d["residual"]) if residual is None else residual
    with gu.forced(path, vpt, store):
        r, n = mfr.residual_add_rmsnorm(x, residual, gu.dev_bf16(d["gamma"]), d["eps"],
                                        residual_out=residual_out)
    torch.cuda.synchronize()
    return gu.host_u16(r), gu.host_u16(n)


def check_dense(d, r, n, tokens=None):
    if tokens is None:
        ref = oracle.residual_rmsnorm(d["x"], d["residual"], d["gamma"], d["eps"])
    else:
        ref = oracle.residual_rmsnorm(d["x"][tokens], d["residual"][tokens], d["gamma"], d["eps"])
        r, n = r[tokens], n[tokens]
    gu.assert_gate(r, ref["s"], ref["residual_out"], "residual_out")
    gu.assert_gate(n, ref["normed_exact"], ref["normed_out"], "normed_out")
    return ref


CASES = [(1, 2048), (4, 2048), (64, 2048), (1, 6144), (28, 6144), (512, 6144), (2048, 6144),
         (3, 8), (5, 24), (7, 1000), (33, 6152), (2, 16384), (300, 520)]


@pytest.mark.parametrize("path", [0, mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["auto", "token", "stream"])
@pytest.mark.parametrize("T,H", CASES, ids=[f"T{t}-H{h}" for t, h in CASES])
def test_dense_parity(T, H, path):
    d = synth.dense_inputs(T, H, seed=5000 + T + H)
    r, n = run_dense(d, path=path)
    ref = check_dense(d, r, n)
    # x + residual of two bf16 values is exact in fp32 whenever their exponents
    # are within 24 of each other, so residual_out is then the exact rounding
    sx, sr = gu.bf16_f64(d["x"]), gu.bf16_f64(d["residual"])
    exact32 = (sx + sr).astype(np.float32).astype(np.float64) == sx + sr
    assert np.array_equal(gu.bf16_f64(r[exact32]), gu.bf16_f64(ref["residual_out"][exact32]))


def test_dense_prefill_full_size():
    """The dense tail on an 8192-token chunk (1% of residual rows x100): every
    token against the oracle (threads over token ranges)."""
    d = synth.dense_inputs(8192, 6144, seed=synth.seed_for("prefill", 8192), spike_frac=0.01)
    r, n = run_dense(d)

    def evaluate(a, b):
        return oracle.residual_rmsnorm(d["x"][a:b], d["residual"][a:b], d["gamma"], d["eps"])
    for t0, t1, ref in gu.oracle_chunks(8192, evaluate):
        gu.assert_gate(r[t0:t1], ref["s"], ref["residual_out"], "residual_out")
        gu.assert_gate(n[t0:t1], ref["normed_exact"], ref["normed_out"], "normed_out")


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_dense_in_place_and_store_policies(path):
    d = synth.dense_inputs(512, 6144, seed=8)
    r0, n0 = run_dense(d, path=path)
    for store in (tuning.STORE_WRITE_BACK, tuning.STORE_WRITE_THROUGH):
        r1, n1 = run_dense(d, path=path, store=store)
        assert np.array_equal(r0, r1) and np.array_equal(n0, n1)
    resid = gu.dev_bf16(d["residual"])
    r2, n2 = run_dense(d, path=path, residual=resid, residual_out=resid)
    assert np.array_equal(r0, r2) and np.array_equal(n0, n2)
    assert np.array_equal(gu.host_u16(resid), r0)


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_dense_equals_fused_with_all_slots_masked(path):
    """Same launch shape, same sum-of-squares tree: the dense op and the fused
    finalize with every slot masked (shared = x) agree bit for bit, up to the
    sign of an exact zero."""
    d = synth.generate(64, 6144, 8, scale=2.5, seed=21)
    d["perm_idx"][:] = -1
    dd = gu.to_device(d)
    rf, nf = gu.run(dd, d["eps"], d["scale"], path=path)
    rd, nd = run_dense(dict(x=d["shared_out"], residual=d["residual"], gamma=d["gamma"],
                            eps=d["eps"]), path=path)
    assert np.array_equal(gu.bf16_f64(rf), gu.bf16_f64(rd))
    assert np.array_equal(gu.bf16_f64(nf), gu.bf16_f64(nd))


def test_dense_graph_replay():
    d = synth.dense_inputs(28, 6144, seed=9)
    r_eager, n_eager = run_dense(d)
    x, res, g = gu.dev_bf16(d["x"]), gu.dev_bf16(d["residual"]), gu.dev_bf16(d["gamma"])
    r_out, n_out = torch.empty_like(x), torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mfr.residual_add_rmsnorm(x, res, g, d["eps"], residual_out=r_out, normed_out=n_out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(3):
            mfr.residual_add_rmsnorm(x, res, g, d["eps"], residual_out=r_out, normed_out=n_out)
    for i in range(10):
        r_out.fill_(0)
        n_out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_u16(r_out), r_eager), i
        assert np.array_equal(gu.host_u16(n_out), n_eager), i


# --- the dense tail with FP8 output --------------------------------------

def run_dense_fp8(d, path=0, vpt=0, store=0, bf16_normed=True):
    x, res, g = gu.dev_bf16(d["x"]), gu.dev_bf16(d["residual"]), gu.dev_bf16(d["gamma"])
    with gu.forced(path, vpt, store):
        r, q, sc, n = mfr.residual_add_rmsnorm_fp8(x, res, g, d["eps"], bf16_normed=bf16_normed)
    torch.cuda.synchronize()
    return (gu.host_u16(r), q.view(torch.uint8).cpu().numpy(), sc.cpu().numpy().astype(np.float64),
            None if n is None else gu.host_u16(n))


FP8_CASES = [(1, 6144), (28, 6144), (512, 6144), (3, 8), (7, 1000), (33, 6152), (2, 16384)]


@pytest.mark.parametrize("path", [0, mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["auto", "token", "stream"])
@pytest.mark.parametrize("T,H", FP8_CASES, ids=[f"T{t}-H{h}" for t, h in FP8_CASES])
def test_dense_fp8_parity(T, H, path):
    """Codes and scales against the oracle's per-token E4M3 quantisation of
    its exact normed rows; the bf16 outputs bit-identical to the plain dense
    call."""
    from tests.test_fp8_gpu import check_fp8
    d = synth.dense_inputs(T, H, seed=7000 + T + H)
    r, q, sc, n = run_dense_fp8(d, path=path)
    r0, n0 = run_dense(d, path=path)
    assert np.array_equal(r, r0) and np.array_equal(n, n0)
    ref = oracle.residual_rmsnorm(d["x"], d["residual"], d["gamma"], d["eps"])
    check_fp8(q, sc, ref, d["gamma"], d["eps"])
    # without the bf16 normed output: the same codes and scales
    r2, q2, sc2, n2 = run_dense_fp8(d, path=path, bf16_normed=False)
    assert n2 is None and np.array_equal(r2, r) and np.array_equal(q2, q)
    assert np.array_equal(sc2, sc)


def test_dense_fp8_prefill_full_size():
    """The dense tail with FP8 output on an 8192-token chunk (1% of residual
    rows x100): every token's codes, scale and residual_out against the
    oracle (threads over token ranges)."""
    from tests.test_fp8_gpu import check_fp8
    d = synth.dense_inputs(8192, 6144, seed=synth.seed_for("prefill", 8192), spike_frac=0.01)
    r, q, sc, _ = run_dense_fp8(d, bf16_normed=False)

    def evaluate(a, b):
        return oracle.residual_rmsnorm(d["x"][a:b], d["residual"][a:b], d["gamma"], d["eps"])
    for t0, t1, ref in gu.oracle_chunks(8192, evaluate):
        gu.assert_gate(r[t0:t1], ref["s"], ref["residual_out"], "residual_out")
        check_fp8(q[t0:t1], sc[t0:t1], ref, d["gamma"], d["eps"])


def test_dense_fp8_graph_replay():
    d = synth.dense_inputs(64, 6144, seed=71)
    x, res, g = gu.dev_bf16(d["x"]), gu.dev_bf16(d["residual"]), gu.dev_bf16(d["gamma"])
    r0, q0, s0, _ = mfr.residual_add_rmsnorm_fp8(x, res, g, d["eps"])
    ro, q, s = torch.empty_like(r0), torch.empty_like(q0), torch.empty_like(s0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mfr.residual_add_rmsnorm_fp8(x, res, g, d["eps"], residual_out=ro, normed_fp8=q,
                                     fp8_scale=s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mfr.residual_add_rmsnorm_fp8(x, res, g, d["eps"], residual_out=ro, normed_fp8=q,
                                     fp8_scale=s)
    for _ in range(5):
        ro.zero_()
        q.view(torch.uint8).zero_()
        s.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ro.view(torch.int16), r0.view(torch.int16))
        assert torch.equal(q.view(torch.uint8), q0.view(torch.uint8))
        assert torch.equal(s.view(torch.int32), s0.view(torch.int32))
