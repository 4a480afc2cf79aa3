"""GPU parity of the persistent multi-token path: a grid sized to the GPU,
each workgroup walking tokens blockIdx.x, blockIdx.x + G, ... with the next
token's loads in flight while it finishes the current one.

The grid is forced smaller through the tuning interface's residency cap, so
that each workgroup walks between one and several tens of tokens and the walk
ends on either of the two register buffers. residual_out is compared bit for
bit with the one-token-per-workgroup paths (s is formed the same way in every
layout); normed_out against the oracle at the gate."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_finalize_residual_amd as mfr
from top_finalize_residual_amd import tuning
from tests import gpu_util as gu
from tests.test_fp8_gpu import check_fp8, run_fp8

pytestmark = pytest.mark.gpu

P = mfr.PATH_PERSIST
CONFIG_CASES = [(cfg, T) for cfg in ("tiny", "decode", "decode_masked", "batch512")
                for T in synth.CONFIGS[cfg]["Ts"]]


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def test_path_query_and_fallback():
    """Forced, the persistent path serves H <= 6144 and K <= 8; other shapes
    fall back to the automatic path."""
    with tuning.forced(P):
        assert mfr.moe_finalize_rmsnorm_path(8192, 6144, 8) == P
        assert mfr.moe_finalize_rmsnorm_path(4, 2048, 6) == P
        assert mfr.moe_finalize_rmsnorm_path(8192, 6152, 8) == mfr.PATH_STREAM
        assert mfr.moe_finalize_rmsnorm_path(8192, 6144, 9) == mfr.PATH_STREAM
        assert mfr.moe_finalize_rmsnorm_path(4, 6144, 9) == mfr.PATH_TOKEN


@pytest.mark.parametrize("cfg,T", CONFIG_CASES, ids=[f"{c}-T{t}" for c, t in CONFIG_CASES])
def test_config_parity(cfg, T):
    d = synth.config_inputs(cfg, T)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=P)
    gu.check(d, r, n)
    r0, _ = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_STREAM)
    assert np.array_equal(r, r0)


@pytest.mark.parametrize("residency", [1, 2, 3])
@pytest.mark.parametrize("T", [1, 255, 256, 257, 511, 512, 513, 1000, 2047])
def test_walk_lengths(T, residency):
    """T against grids of 256 x residency workgroups (one CU's worth each):
    a workgroup walks from one token to about eight, ending on either
    buffer, and T below the grid gives one token per workgroup."""
    d = synth.generate(T, 2048, 8, scale=2.5, mask_frac=0.05, seed=5100 + T)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=P, residency=residency)
    gu.check(d, r, n)
    r0, _ = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_STREAM)
    assert np.array_equal(r, r0)


def test_long_walks():
    """One workgroup per CU: T = 8192 gives walks of 32 tokens on 256 CUs,
    and a ragged T of 31 CUs' worth plus 7 walks of 31 and 32."""
    for T, res in ((8192, 1), (31 * _cus() + 7, 1)):
        d = synth.generate(T, 2048, 8, scale=2.5, seed=5200 + T)
        dd = gu.to_device(d)
        r, n = gu.run(dd, d["eps"], d["scale"], path=P, residency=res)
        gu.check_all_tokens(d, r, n)


def test_prefill_chunk_full_size():
    """The 8192-token prefill chunk on the persistent path, every token
    against the oracle; residual_out bit-identical to the stream path."""
    d = synth.config_inputs("prefill", 8192)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=P)
    r0, _ = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_STREAM)
    del dd
    assert np.array_equal(r, r0)
    gu.check_all_tokens(d, r, n)


RAGGED = [(3, 16, 2), (7, 1000, 5), (33, 2056, 7), (300, 520, 4), (65, 6144, 8), (17, 4096, 1)]


@pytest.mark.parametrize("store", [tuning.STORE_WRITE_BACK, tuning.STORE_WRITE_THROUGH],
                         ids=["write_back", "write_through"])
@pytest.mark.parametrize("T,H,K", RAGGED, ids=[f"T{t}-H{h}-K{k}" for t, h, k in RAGGED])
def test_ragged_shapes(T, H, K, store):
    d = synth.generate(T, H, K, scale=2.5, mask_frac=0.1, seed=5300 + T + H + K, extra_rows=3)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=P, store=store, residency=1)
    gu.check(d, r, n)


@pytest.mark.parametrize("bf16_normed", [False, True], ids=["fp8", "fp8+bf16"])
@pytest.mark.parametrize("cfg,T", [("decode", 28), ("batch512", 512)])
def test_fp8(cfg, T, bf16_normed):
    d = synth.config_inputs(cfg, T)
    dd = gu.to_device(d)
    r, q, sc, n = run_fp8(dd, d, path=P, bf16_normed=bf16_normed, residency=1)
    check_fp8(q, sc, gu.oracle_for(d), d["gamma"], d["eps"])
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=P, residency=1)
    assert np.array_equal(r, r0)
    if bf16_normed:
        assert np.array_equal(n, n0)


def test_fp8_prefill_full_size():
    d = synth.config_inputs("prefill", 8192)
    dd = gu.to_device(d)
    r, q, sc, _ = run_fp8(dd, d, path=P)
    del dd
    for t0, t1, ref in gu.oracle_chunks(8192, gu.finalize_evaluator(d)):
        check_fp8(q[t0:t1], sc[t0:t1], ref, d["gamma"], d["eps"])
        gu.assert_gate(r[t0:t1], ref["s"], ref["residual_out"], "residual_out")


@pytest.mark.parametrize("T,H", [(1, 6144), (512, 6144), (1000, 2048), (8192, 6144)])
def test_dense(T, H):
    """The dense tail (bf16 and FP8 output) on the persistent path against the
    oracle, and bit-identical to the stream path's residual_out."""
    d = synth.dense_inputs(T, H, seed=5400 + T + H, spike_frac=0.01)
    x, res, g = gu.dev_bf16(d["x"]), gu.dev_bf16(d["residual"]), gu.dev_bf16(d["gamma"])
    with tuning.forced(P):
        r, n = mfr.residual_add_rmsnorm(x, res, g, d["eps"])
        r8, q, sc, n8 = mfr.residual_add_rmsnorm_fp8(x, res, g, d["eps"], bf16_normed=True)
    with tuning.forced(mfr.PATH_STREAM):
        r0, _ = mfr.residual_add_rmsnorm(x, res, g, d["eps"])
    torch.cuda.synchronize()
    r, n, r8, n8, r0 = (gu.host_u16(a) for a in (r, n, r8, n8, r0))
    assert np.array_equal(r, r0) and np.array_equal(r8, r) and np.array_equal(n8, n)
    q = q.view(torch.uint8).cpu().numpy()
    sc = sc.cpu().numpy().astype(np.float64)

    def evaluate(a, b):
        return oracle.residual_rmsnorm(d["x"][a:b], d["residual"][a:b], d["gamma"], d["eps"])
    for t0, t1, ref in gu.oracle_chunks(T, evaluate):
        gu.assert_gate(r[t0:t1], ref["s"], ref["residual_out"], "residual_out")
        gu.assert_gate(n[t0:t1], ref["normed_exact"], ref["normed_out"], "normed_out")
        check_fp8(q[t0:t1], sc[t0:t1], ref, d["gamma"], d["eps"])


@pytest.mark.parametrize("K", [8, 5], ids=["top8", "anyK"])
def test_checked_masks_and_flags_out_of_range_indices(K):
    """The checked entry point on the persistent path: an index at or past R
    is masked (the output equals the call with that slot masked) and raises
    the flag; with every index in range the flag stays clear and the outputs
    are those of the plain call."""
    T, H = 700, 2048
    d = synth.generate(T, H, K, scale=2.5, seed=5500 + K)
    dd = gu.to_device(d)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    with tuning.forced(P, 0, 0, residency=1):
        r, n = mfr.moe_finalize_rmsnorm(*(dd[k] for k in ("expert_out", "perm_idx", "topk_w",
                                                          "shared_out", "residual", "gamma")),
                                        d["eps"], d["scale"], bad_index=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=P, residency=1)
    assert np.array_equal(gu.host_u16(r), r0) and np.array_equal(gu.host_u16(n), n0)
    bad = d["perm_idx"].copy()
    bad[[3, 400, 699], [0, K - 1, 1]] = d["R"] + np.array([0, 5, 1 << 20])
    masked = d["perm_idx"].copy()
    masked[[3, 400, 699], [0, K - 1, 1]] = -1
    dd_bad = dict(dd, perm_idx=torch.from_numpy(bad).cuda())
    with tuning.forced(P, 0, 0, residency=1):
        r, n = mfr.moe_finalize_rmsnorm(*(dd_bad[k] for k in ("expert_out", "perm_idx", "topk_w",
                                                              "shared_out", "residual", "gamma")),
                                        d["eps"], d["scale"], bad_index=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1
    r1, n1 = gu.run(dict(dd, perm_idx=torch.from_numpy(masked).cuda()), d["eps"], d["scale"],
                    path=P, residency=1)
    assert np.array_equal(gu.host_u16(r), r1) and np.array_equal(gu.host_u16(n), n1)


def test_graph_replay():
    """The persistent call captured into a graph replays like the eager call,
    with eager work and synchronisations between the replays."""
    d = synth.config_inputs("batch512", 512)
    dd = gu.to_device(d)
    r_eager, n_eager = gu.run(dd, d["eps"], d["scale"], path=P)
    r_out, n_out = torch.empty_like(dd["residual"]), torch.empty_like(dd["residual"])
    T, K = d["T"], d["K"]

    def call():
        rc = mfr.moe_finalize_rmsnorm_raw(
            *(dd[k].data_ptr() for k in ("expert_out", "perm_idx", "topk_w", "shared_out",
                                         "residual", "gamma")),
            d["eps"], d["scale"], r_out.data_ptr(), n_out.data_ptr(), T, d["H"], K,
            torch.cuda.current_stream().cuda_stream)
        assert rc == 0
    with tuning.forced(P):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
            call()
    for i in range(10):
        r_out.fill_(0)
        n_out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_u16(r_out), r_eager), i
        assert np.array_equal(gu.host_u16(n_out), n_eager), i


def test_extreme_rows():
    """Rows outside the fp32 range of the sum of squares take the fp64
    normalisation on this path too, within walks of several tokens (the
    pattern of scaled tokens repeated 40 times, on one workgroup per CU)."""
    from tests.test_range_gpu import EXPS, check_rows, extreme_inputs
    d = extreme_inputs(seed=5600, exps=EXPS * 40)
    r, n = gu.run(gu.to_device(d), d["eps"], d["scale"], path=P, residency=1)
    check_rows(d, r, n)


def test_checked_fp8_calls_take_the_automatic_path():
    """The persistent kernel does not serve the checked entry points with FP8
    output: forced onto it, those calls run the automatic path, bit for bit
    the same as with no override."""
    T, H, K = 700, 6144, 8
    d = synth.generate(T, H, K, scale=2.5, seed=5700)
    dd = gu.to_device(d)
    with tuning.forced(P):
        forced = run_fp8(dd, d, bf16_normed=True, api="binding")
    auto = run_fp8(dd, d, bf16_normed=True, api="binding")
    for a, b in zip(forced, auto):
        assert np.array_equal(a, b)
    check_fp8(forced[1], forced[2], gu.oracle_for(d), d["gamma"], d["eps"])
