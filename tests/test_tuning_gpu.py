"""The tuning interface's placement knobs on the GPU: a cap on the
workgroups per CU of the grid paths (LDS reserved at launch), per-XCD token
ranges, and the non-temporal output encodings. None of them may change a
result, so every output is compared bit for bit with the automatic launch of
the same path, and the automatic launch against the oracle at the gate.

The knobs exist to measure alternatives to the shipped launch (the
benchmark's --alternatives mode); these tests make sure that what is
measured computes the op."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth
import top_finalize_residual_amd as mfr
from top_finalize_residual_amd import tuning
from tests import gpu_util as gu
from tests.test_fp8_gpu import run_fp8

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
XCD = tuning.ORDER_XCD_RANGES
KNOBS = {
    "no-cap": dict(residency=64),
    "cap1": dict(residency=1),
    "cap2": dict(residency=2),
    "xcd": dict(order=XCD),
    "nt": dict(store=tuning.STORE_NONTEMPORAL),
    "nt-wt": dict(store=tuning.STORE_NONTEMPORAL_WRITE_THROUGH),
    "all": dict(residency=2, order=XCD, store=tuning.STORE_NONTEMPORAL_WRITE_THROUGH),
}
# ragged T around the 8 XCDs and the 256 CUs, H of one to four vectors per thread
SHAPES = [(1, 6144), (7, 2048), (9, 6144), (28, 6144), (257, 2048), (513, 6144), (1000, 4096)]


@pytest.fixture(scope="module")
def inputs():
    cache = {}

    def get(T, H, K=8):
        if (T, H, K) not in cache:
            d = synth.generate(T, H, K, scale=2.5, mask_frac=0.05,
                               seed=synth.BASE_SEED + 7000 + T + H + K, extra_rows=5)
            cache[(T, H, K)] = (d, gu.to_device(d))
        return cache[(T, H, K)]
    return get


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
@pytest.mark.parametrize("T,H", SHAPES, ids=[f"T{t}-H{h}" for t, h in SHAPES])
def test_fused_op_unchanged(inputs, T, H, path):
    d, dd = inputs(T, H)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    gu.check(d, r0, n0)
    for name, kw in KNOBS.items():
        r, n = gu.run(dd, d["eps"], d["scale"], path=path, **kw)
        assert np.array_equal(r, r0), name
        assert np.array_equal(n, n0), name


@pytest.mark.parametrize("T,H,K", [(9, 6144, 6), (513, 2048, 5), (1000, 6144, 8)])
def test_other_variants_unchanged(inputs, T, H, K):
    """Any K, the FP8 output and the checked entry point under the cap and
    the token ranges; the non-temporal encodings fall back to the automatic
    policy for them, which must not change a result either."""
    d, dd = inputs(T, H, K)
    base = run_fp8(dd, d, bf16_normed=True)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], api="binding")
    for name, kw in KNOBS.items():
        got = run_fp8(dd, d, bf16_normed=True, **kw)
        for a, b in zip(got, base):
            assert np.array_equal(a, b), name
        r, n = gu.run(dd, d["eps"], d["scale"], api="binding", **kw)
        assert np.array_equal(r, r0) and np.array_equal(n, n0), name


def test_dense_unchanged():
    T, H = 1000, 6144
    dd = synth.dense_inputs(T, H, seed=synth.BASE_SEED + 7100, spike_frac=0.01)
    x, res, g = gu.dev_bf16(dd["x"]), gu.dev_bf16(dd["residual"]), gu.dev_bf16(dd["gamma"])
    r0, n0 = mfr.residual_add_rmsnorm(x, res, g, dd["eps"])
    torch.cuda.synchronize()
    r0, n0 = gu.host_u16(r0), gu.host_u16(n0)
    for name, kw in KNOBS.items():
        with tuning.forced(**kw):
            r, n = mfr.residual_add_rmsnorm(x, res, g, dd["eps"])
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_u16(r), r0) and np.array_equal(gu.host_u16(n), n0), name


def test_prefill_chunk_unchanged():
    """The 8192-token chunk (32 tokens per CU) under each knob, bit for bit."""
    d = synth.config_inputs("prefill", 8192)
    dd = gu.to_device(d)
    r0, n0 = gu.run(dd, d["eps"], d["scale"])
    for name, kw in KNOBS.items():
        r, n = gu.run(dd, d["eps"], d["scale"], **kw)
        assert np.array_equal(r, r0) and np.array_equal(n, n0), name


_LOG_SCRIPT = r"""
import torch, synth, sys
from tests import gpu_util as gu
from tests.test_fp8_gpu import run_fp8
for T in (600, 2048):
    d = synth.generate(T, 6144, 8, scale=2.5, seed=11)
    dd = gu.to_device(d)
    for cap in (0, 1, 2, 3, 8):
        print(f"case=T{T}/bf16/cap{cap}", file=sys.stderr, flush=True)
        gu.run(dd, d["eps"], d["scale"], residency=cap)
    print(f"case=T{T}/fp8/cap0", file=sys.stderr, flush=True)
    run_fp8(dd, d)
"""


def test_cap_reserves_lds_only_below_the_kernel_residency():
    """H = 6144 (the 256-thread stream kernel, 3 workgroups per CU by its
    registers): a cap of 1 or 2 reserves LDS at launch, a cap of 3 or more
    none. Automatic (0): no cap at T = 600, a cap of 2 at T = 2048 for the
    bf16 and the FP8 output. Read from the library's launch log in a child
    process."""
    env = dict(os.environ, MFR_LOG="1", PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", _LOG_SCRIPT], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    lds = {}
    case = None
    for ln in out.stderr.splitlines():
        if ln.startswith("case="):
            case = ln[5:]
        elif "reserved_lds=" in ln and case is not None:
            lds[case] = int(ln.split("reserved_lds=")[1].split()[0])
    assert len(lds) == 12, out.stderr[-3000:]
    for T in (600, 2048):
        c = {cap: lds[f"T{T}/bf16/cap{cap}"] for cap in (0, 1, 2, 3, 8)}
        assert c[3] == 0 and c[8] == 0 and c[1] > c[2] > 0, (T, c)
    assert lds["T600/bf16/cap0"] == 0 and lds["T600/fp8/cap0"] == 0
    assert lds["T2048/bf16/cap0"] == lds["T2048/bf16/cap2"]
    assert lds["T2048/fp8/cap0"] > 0


_GRAPH_FIRST = r"""
import numpy as np, torch, synth
from tests import gpu_util as gu
import top_finalize_residual_amd as mfr
d = synth.generate(2048, 6144, 8, scale=2.5, seed=21)
dd = gu.to_device(d)
r, n = torch.empty_like(dd["residual"]), torch.empty_like(dd["residual"])
args = [dd[k].data_ptr() for k in ("expert_out", "perm_idx", "topk_w", "shared_out", "residual",
                                   "gamma")]


def call():
    rc = mfr.moe_finalize_rmsnorm_raw(*args, d["eps"], d["scale"], r.data_ptr(), n.data_ptr(),
                                      2048, 6144, 8, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, rc


g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):  # the process's first launch: the cap is looked up during capture
    call()
outs = []
for i in range(3):
    r.fill_(0)
    n.fill_(0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    outs.append((gu.host_u16(r), gu.host_u16(n)))
r0, n0 = gu.run(dd, d["eps"], d["scale"])
for rr, nn in outs:
    assert np.array_equal(rr, r0) and np.array_equal(nn, n0)
print("graph-first ok", flush=True)
"""


def test_first_capped_launch_inside_a_graph_capture():
    """A process whose first launch of the capped stream kernel happens
    during graph capture: the occupancy and attribute queries behind the cap
    are made inside the capture, and every replay equals the eager call."""
    env = dict(os.environ, PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", _GRAPH_FIRST], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and "graph-first ok" in out.stdout, out.stderr[-3000:]


@pytest.mark.parametrize("T,H", [(2048, 6144), (2049, 5128), (3001, 5632)],
                         ids=["T2048-H6144", "T2049-H5128", "T3001-H5632"])
def test_capped_shapes_against_the_oracle(T, H):
    """Shapes the automatic per-CU cap applies to (the 3-vector stream kernel
    above H = 5120 from T = 2048), with bf16 and with FP8-only output, every
    token against the oracle."""
    from tests.test_fp8_gpu import check_fp8
    d = synth.generate(T, H, 8, scale=2.5, mask_frac=0.03, seed=synth.BASE_SEED + 7300 + T + H,
                       extra_rows=2)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"])
    gu.check_all_tokens(d, r, n)
    rq, q, sc, _ = run_fp8(dd, d)
    assert np.array_equal(rq, r)
    for t0, t1, ref in gu.oracle_chunks(T, gu.finalize_evaluator(d)):
        check_fp8(q[t0:t1], sc[t0:t1], ref, d["gamma"], d["eps"])
