"""GPU parity of the fused op's dynamic per-token FP8 output against the oracle
(finalize, then per-token E4M3 quantisation of the exact normed rows).

Codes are compared exactly, except next to a rounding tie: the GPU forms y and
the scale in fp32, so its y / scale carries the fp32 error of the sum s (the
same 1e-6 absolute floor the bf16 gate allows, carried through the
normalisation and the scale) plus a relative 2^-18. Where the exact y / scale
lies that close to the midpoint between two E4M3 neighbours, either is a
correct rounding and the GPU's code may be the other one. Scales agree to
fp32 accuracy: a relative 2^-20, plus the spacing 2^-149 of fp32 subnormals
for the scale of a row whose largest value is tiny."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_finalize_residual_amd as mfr
from top_finalize_residual_amd import tuning
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SCALE_REL = 2.0 ** -20
SCALE_ABS = 2.0 ** -149  # spacing of fp32 subnormals
TIE_REL = 2.0 ** -18


def e4m3_key(codes):
    """Monotone integer key of E4M3 codes (+0 and -0 map to 0)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def e4m3_values(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def run_fp8(dd, d, path=0, vpt=0, store=0, bf16_normed=False, api="c", residency=0, order=0):
    """One FP8-output call; returns host (residual_out, codes, scales, normed_out
    or None). api="c": the plain C entry point moe_finalize_rmsnorm_fp8 (the
    call the benchmark times); api="binding": the tensor-level binding, which
    goes through the checked entry point."""
    with gu.forced(path, vpt, store, residency, order):
        if api == "binding":
            r, q, sc, n = mfr.moe_finalize_rmsnorm_fp8(
                dd["expert_out"], dd["perm_idx"], dd["topk_w"], dd["shared_out"], dd["residual"],
                dd["gamma"], d["eps"], d["scale"], bf16_normed=bf16_normed)
        else:
            T, K = dd["perm_idx"].shape
            H = dd["gamma"].shape[0]
            r = torch.empty_like(dd["residual"])
            n = torch.empty_like(dd["residual"]) if bf16_normed else None
            q = torch.empty((T, H), dtype=torch.float8_e4m3fn, device="cuda")
            sc = torch.empty((T,), dtype=torch.float32, device="cuda")
            rc = mfr.moe_finalize_rmsnorm_fp8_raw(
                *(dd[k].data_ptr() for k in ("expert_out", "perm_idx", "topk_w", "shared_out",
                                             "residual", "gamma")),
                d["eps"], d["scale"], r.data_ptr(), None if n is None else n.data_ptr(),
                q.data_ptr(), sc.data_ptr(), T, H, K, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise mfr.MFRError(rc)
    torch.cuda.synchronize()
    return (gu.host_u16(r), q.view(torch.uint8).cpu().numpy(), sc.cpu().numpy().astype(np.float64),
            None if n is None else gu.host_u16(n))


def check_fp8(codes, scales, ref, gamma, eps, abs_floor=None):
    """ref: the oracle's finalize outputs (s, normed_exact) for these rows.
    abs_floor: the absolute error the GPU's fp32 s may carry, per row or for
    all rows (default gu.ABS, right for inputs of order one; a row scaled by
    c carries c times that)."""
    normed_exact = ref["normed_exact"]
    want, want_scale, scaled = oracle.fp8_quantize_rows(normed_exact)
    assert np.all(np.abs(scales - want_scale) <= SCALE_REL * want_scale + SCALE_ABS), "scale"
    diff = np.abs(e4m3_key(codes) - e4m3_key(want))
    assert diff.max(initial=0) <= 1, f"codes {int(diff.max())} steps apart"
    if diff.any():
        # the exact value must sit at the midpoint of the two codes, within the
        # error the GPU's fp32 y / scale may carry there
        s = ref["s"]
        rstd = 1.0 / np.sqrt(np.mean(s * s, axis=1, keepdims=True) + eps)
        g = np.abs(gu.bf16_f64(gamma))[None, :]
        floor = gu.ABS if abs_floor is None else np.reshape(abs_floor, (-1, 1))
        tol = floor * rstd * g / want_scale[:, None] + TIE_REL * np.abs(scaled)
        a, b = e4m3_values(codes[diff == 1]), e4m3_values(want[diff == 1])
        v = scaled[diff == 1]
        assert np.all(np.abs(v - (a + b) / 2) <= tol[diff == 1]), "code differs away from a tie"
    assert not np.any((codes & 0x7F) == 0x7F), "NaN code"
    # the element of largest magnitude of every row with a finite nonzero scale
    # encodes to exactly +-448 (0x7E): the factor keeps it from passing 448, and
    # no lower code is within a step of it
    live = np.isfinite(want_scale) & (want_scale > 0) & (want_scale != 1.0)
    if live.any():
        top = (codes[live] & 0x7F).max(axis=1)
        assert np.all(top == 0x7E), "row maximum not at 448"
    return want


CASES = [("tiny", 4), ("decode", 1), ("decode", 28), ("decode", 64), ("decode_masked", 64),
         ("batch512", 512)]


@pytest.mark.parametrize("path", [0, mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["auto", "token", "stream"])
@pytest.mark.parametrize("cfg,T", CASES, ids=[f"{c}-T{t}" for c, t in CASES])
def test_fp8_parity(cfg, T, path):
    d = synth.config_inputs(cfg, T)
    dd = gu.to_device(d)
    r, q, sc, n = run_fp8(dd, d, path=path, bf16_normed=True)
    ref = gu.oracle_for(d)
    check_fp8(q, sc, ref, d["gamma"], d["eps"])
    # the bf16 outputs are those of the plain call
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    assert np.array_equal(r, r0) and np.array_equal(n, n0)


def test_fp8_without_bf16_normed_and_store_policies():
    d = synth.config_inputs("batch512", 512)
    dd = gu.to_device(d)
    r1, q1, s1, n1 = run_fp8(dd, d)
    assert n1 is None
    for store in (tuning.STORE_WRITE_BACK, tuning.STORE_WRITE_THROUGH):
        r2, q2, s2, _ = run_fp8(dd, d, store=store, bf16_normed=True)
        assert np.array_equal(r1, r2) and np.array_equal(q1, q2) and np.array_equal(s1, s2)
    check_fp8(q1, s1, gu.oracle_for(d), d["gamma"], d["eps"])


def test_fp8_prefill_full_size():
    """The FP8-output call on the 8192-token prefill chunk: every token's codes,
    scale and residual_out against the oracle (threads over token ranges)."""
    d = synth.config_inputs("prefill", 8192)
    dd = gu.to_device(d)
    r, q, sc, _ = run_fp8(dd, d)
    del dd
    for t0, t1, ref in gu.oracle_chunks(8192, gu.finalize_evaluator(d)):
        check_fp8(q[t0:t1], sc[t0:t1], ref, d["gamma"], d["eps"])
        gu.assert_gate(r[t0:t1], ref["s"], ref["residual_out"], "residual_out")


RAGGED = [(3, 16, 2), (7, 1000, 5), (33, 2056, 9), (17, 6152, 16), (2, 16384, 16)]


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
@pytest.mark.parametrize("T,H,K", RAGGED, ids=[f"T{t}-H{h}-K{k}" for t, h, k in RAGGED])
def test_fp8_ragged(T, H, K, path):
    d = synth.generate(T, H, K, scale=2.5, mask_frac=0.1, seed=700 + T + H)
    dd = gu.to_device(d)
    r, q, sc, _ = run_fp8(dd, d, path=path)
    check_fp8(q, sc, gu.oracle_for(d), d["gamma"], d["eps"])


def test_fp8_zero_row():
    """A token whose sum is exactly zero: scale 1, every code zero."""
    d = synth.generate(4, 2048, 8, scale=1.0, seed=71)
    d["topk_w"][1] = 0.0
    d["residual"][1] = d["shared_out"][1] ^ np.uint16(0x8000)
    dd = gu.to_device(d)
    r, q, sc, _ = run_fp8(dd, d)
    assert sc[1] == 1.0 and np.all(e4m3_key(q[1]) == 0)
    check_fp8(q, sc, gu.oracle_for(d), d["gamma"], d["eps"])


def test_fp8_tiny_row():
    """A token whose sum is made of bf16 subnormals no larger than 7 * 2^-133
    (shared and routed parts zero, eps 1e-4): its amax lies far below
    448 / FLT_MAX, so 448 / amax overflows fp32. Every code still matches the
    oracle (this row's sum is exact, so a code may differ only at a tie, to
    fp32 rounding of the scaled value), zeros stay zero and no NaN code
    appears."""
    T, H, t = 4, 2048, 2
    d = synth.generate(T, H, 8, scale=1.0, seed=72)
    d["eps"] = float(np.float32(1e-4))
    d["topk_w"][t] = 0.0
    d["shared_out"][t] = 0
    rng = np.random.default_rng(3)
    mant = rng.integers(0, 8, size=H).astype(np.uint16)
    sign = rng.integers(0, 2, size=H).astype(np.uint16) << np.uint16(15)
    d["residual"][t] = sign | mant
    dd = gu.to_device(d)
    r, q, sc, _ = run_fp8(dd, d)
    ref = gu.oracle_for(d)
    want, want_scale, scaled = oracle.fp8_quantize_rows(ref["normed_exact"])
    amax = want_scale[t] * 448.0
    assert 448.0 / amax > np.finfo(np.float32).max  # the case under test
    check_fp8(q, sc, ref, d["gamma"], d["eps"])
    diff = np.abs(e4m3_key(q[t]) - e4m3_key(want[t]))
    assert diff.max() <= 1
    i = np.nonzero(diff)[0]
    mid = (e4m3_values(q[t][i]) + e4m3_values(want[t][i])) / 2
    assert np.all(np.abs(scaled[t][i] - mid) <= TIE_REL * np.abs(scaled[t][i]))
    zero = (d["residual"][t] & 0x7FFF) == 0
    assert zero.any() and np.all(e4m3_key(q[t][zero]) == 0)


def test_fp8_nan_gamma_element():
    """A NaN in gamma makes that column of y NaN: its codes are the NaN code;
    amax is taken over the other values (as the oracle takes it), so every
    other code and the scales match the oracle."""
    T, H, col = 8, 2048, 100
    d = synth.generate(T, H, 8, scale=2.5, seed=73)
    d["gamma"] = d["gamma"].copy()
    d["gamma"][col] = 0x7FC0
    dd = gu.to_device(d)
    r, q, sc, _ = run_fp8(dd, d)
    ref = gu.oracle_for(d)
    assert np.all((q[:, col] & 0x7F) == 0x7F)
    keep = np.arange(H) != col
    sub = dict(s=ref["s"][:, keep], normed_exact=ref["normed_exact"][:, keep])
    check_fp8(q[:, keep], sc, sub, d["gamma"][keep], d["eps"])


def test_fp8_graph_replay():
    """The FP8-output call captured into a graph replays like the eager call,
    codes and scales bit for bit, with eager work and synchronisations
    between the replays."""
    d = synth.config_inputs("decode", 28)
    dd = gu.to_device(d)
    r0, q0, s0, n0 = run_fp8(dd, d, bf16_normed=True)
    T, H = d["T"], d["H"]
    ro = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    no = torch.empty_like(ro)
    q = torch.empty((T, H), dtype=torch.float8_e4m3fn, device="cuda")
    sc = torch.empty((T,), dtype=torch.float32, device="cuda")

    def call():
        mfr.moe_finalize_rmsnorm_fp8(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                     dd["shared_out"], dd["residual"], dd["gamma"], d["eps"],
                                     d["scale"], residual_out=ro, normed_fp8=q, fp8_scale=sc,
                                     normed_out=no)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(10):
        ro.fill_(0)
        no.fill_(0)
        q.view(torch.uint8).fill_(0)
        sc.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_u16(ro), r0), i
        assert np.array_equal(gu.host_u16(no), n0), i
        assert np.array_equal(q.view(torch.uint8).cpu().numpy(), q0), i
        assert np.array_equal(sc.cpu().numpy().astype(np.float64), s0), i
