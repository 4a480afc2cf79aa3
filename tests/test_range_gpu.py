"""GPU parity at the edges of the fp32 range of the sum of squares.

The kernels accumulate s in fp32 and take its sum of squares in fp32. Where
that sum overflows (|s| above about 2^64 / sqrt(H)) or is too small to decide
rstd (eps = 0 and squares that are fp32 subnormals or flush to zero), the
kernel normalises the row again with an fp64 sum of squares. These rows must
still match the oracle's fp64 definition at the usual gate.

Extreme rows are made by scaling a token of the synthetic workload by an exact
power of two c = 2^k (its residual, shared output and gathered expert rows), so
the kernel's fp32 s is c times that of the unscaled token wherever the scaled
bf16 inputs stay normal; the absolute error floor of the gate scales with c
too. Every kernel variant that carries the branch is run: both launch paths,
every vectors-per-thread shape, top-8 and any-K routing, the checked entry
point, the FP8 outputs and the dense tail."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_finalize_residual_amd as mfr
from tests import gpu_util as gu
from tests.test_fp8_gpu import check_fp8, run_fp8

pytestmark = pytest.mark.gpu

# log2 of the per-token scale: ordinary rows (0, 30, -30) beside rows whose
# fp32 sum of squares overflows (60 and up) or underflows (-60 and down)
EXPS = (0, 60, 70, 90, 110, 120, -60, -70, -90, -110, -120, 30, -30, 0)
F32_MAX = float(np.finfo(np.float32).max)


def _scale_bf16(u16, c):
    return synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(u16) * np.float32(c))


def extreme_inputs(H=2048, K=8, seed=4100, eps=0.0, exps=EXPS):
    d = synth.generate(len(exps), H, K, scale=2.5, seed=seed)
    d["eps"] = float(np.float32(eps))
    E, S, X = d["expert_out"].copy(), d["shared_out"].copy(), d["residual"].copy()
    c = np.array([2.0 ** k for k in exps])
    for t, ct in enumerate(c):
        rows = d["perm_idx"][t][d["perm_idx"][t] >= 0]
        E[rows] = _scale_bf16(E[rows], ct)
        S[t] = _scale_bf16(S[t], ct)
        X[t] = _scale_bf16(X[t], ct)
    d.update(expert_out=E, shared_out=S, residual=X)
    d["row_scale"] = c
    return d


# Half the spacing of the bf16 subnormals (2^-133): below 2^-126 the output
# format itself cannot come closer to a value than this, whatever the
# arithmetic, so a relative bound alone cannot hold there.
BF16_SUBNORMAL_HALF_STEP = 2.0 ** -134


def assert_gate_rows(gpu_u16, ref_exact, ref_bits, row_scale, what):
    """|gpu - ref| <= 2^-8 |ref| + 1e-6 * c_t (+ half a bf16 subnormal step)
    on every element of token t, and at most one bf16 step from the oracle's
    own bf16 rounding wherever |ref| >= 2^-8 c_t (below that, the fp32 error
    of a cancelling sum spans several steps of the small result, as in the
    ordinary gate)."""
    g = gu.bf16_f64(gpu_u16)
    bound = gu.REL * np.abs(ref_exact) + gu.ABS * row_scale[:, None] + BF16_SUBNORMAL_HALF_STEP
    bad = ~(np.abs(g - ref_exact) <= bound)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the gate; first at {i}: "
                             f"gpu {g[i]!r} ref {ref_exact[i]!r} (row scale {row_scale[i[0]]!r})")
    dist = np.abs(gu.ulp_key(gpu_u16) - gu.ulp_key(ref_bits))
    big = np.abs(ref_exact) >= gu.ULP_CHECK_MIN * row_scale[:, None]
    worst = int(dist[big].max(initial=0))
    assert worst <= 1, f"{what}: {worst} bf16 steps from the oracle"


def check_rows(d, r, n, ref=None):
    if ref is None:
        ref = gu.oracle_for(d)
    assert_gate_rows(r, ref["s"], ref["residual_out"], d["row_scale"], "residual_out")
    assert_gate_rows(n, ref["normed_exact"], ref["normed_out"], np.ones_like(d["row_scale"]),
                     "normed_out")
    return ref


def test_the_cases_reach_both_ends_of_the_range():
    """Host-side check of the construction: the scaled tokens' fp32 sums of
    squares do overflow, or do fall below the fp32 normal range, while the
    sums s themselves stay finite."""
    d = extreme_inputs()
    ref = gu.oracle_for(d)
    ss = np.sum(ref["s"] ** 2, axis=1)
    for t, k in enumerate(EXPS):
        assert np.all(np.abs(ref["s"][t]) < F32_MAX), k
        if k >= 60:
            assert ss[t] > F32_MAX, k
        if k <= -60:
            assert ss[t] / d["H"] < 2.0 ** -100, k


@pytest.mark.parametrize("K", [8, 6], ids=["top8", "anyK"])
@pytest.mark.parametrize("path,vpt", [(mfr.PATH_TOKEN, v) for v in (1, 2, 3, 4)] +
                         [(mfr.PATH_STREAM, v) for v in (1, 2, 3, 4)] + [(0, 0)],
                         ids=[f"token-v{v}" for v in (1, 2, 3, 4)] +
                             [f"stream-v{v}" for v in (1, 2, 3, 4)] + ["auto"])
def test_extreme_rows_bf16(path, vpt, K):
    d = extreme_inputs(K=K, seed=4100 + K)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=path, vpt=vpt)
    check_rows(d, r, n)
    # the ordinary tokens are untouched by their extreme neighbours: the same
    # bits as in a call made of ordinary tokens only
    plain = synth.generate(len(EXPS), d["H"], K, scale=2.5, seed=4100 + K)
    plain["eps"] = d["eps"]
    r0, n0 = gu.run(gu.to_device(plain), d["eps"], d["scale"], path=path, vpt=vpt)
    for t, k in enumerate(EXPS):
        if k == 0:
            assert np.array_equal(r[t], r0[t]) and np.array_equal(n[t], n0[t]), t
        # normalisation is scale-invariant: within one bf16 step of the
        # ordinary token's normed row (wherever the scaled inputs stayed exact)
        if abs(k) <= 90:
            dist = np.abs(gu.ulp_key(n[t]) - gu.ulp_key(n0[t]))
            assert dist.max() <= 1, (t, k)


@pytest.mark.parametrize("eps", [0.0, 1e-40, 1e-6], ids=["eps0", "eps_subnormal", "eps1e-6"])
@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_extreme_rows_eps(path, eps):
    """eps = 0, an fp32-subnormal eps and the usual 1e-6: with eps of normal
    size the tiny rows are dominated by it (and need no second pass); with
    eps = 0 or subnormal they are normalised by their own mean square."""
    d = extreme_inputs(eps=eps, seed=4200)
    r, n = gu.run(gu.to_device(d), d["eps"], d["scale"], path=path)
    check_rows(d, r, n)


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_subnormal_only_rows_eps_zero(path):
    """Tokens whose s is made of bf16 subnormals only (at most 127 * 2^-133;
    shared output and routed part zero) with eps = 0: every square flushes to
    zero in fp32, and the fp32 rstd would be infinite. The normed rows match
    the oracle, and residual_out is exactly the input (s is exact)."""
    T, H = 6, 2048
    d = synth.generate(T, H, 8, scale=1.0, seed=4300)
    d["eps"] = 0.0
    rng = np.random.default_rng(43)
    for t in (1, 2, 4):
        d["topk_w"][t] = 0.0
        d["shared_out"][t] = 0
        mant = rng.integers(1, 128, size=H).astype(np.uint16)
        sign = rng.integers(0, 2, size=H).astype(np.uint16) << np.uint16(15)
        d["residual"][t] = sign | mant
    r, n = gu.run(gu.to_device(d), 0.0, d["scale"], path=path)
    ref = gu.oracle_for(d)
    gu.check(d, r, n, ref=ref)
    for t in (1, 2, 4):
        assert np.array_equal(r[t] & 0x7FFF, d["residual"][t] & 0x7FFF)
        assert np.all(np.isfinite(gu.bf16_f64(n[t])))
        assert np.abs(gu.bf16_f64(n[t])).max() > 0.5  # normalised to order one


@pytest.mark.parametrize("bf16_normed", [False, True], ids=["fp8", "fp8+bf16"])
@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_extreme_rows_fp8(path, bf16_normed):
    """The FP8-output call on the same rows: codes and scales against the
    oracle's quantisation of its exact normed rows; the bf16 outputs those of
    the plain call."""
    d = extreme_inputs(seed=4400)
    dd = gu.to_device(d)
    r, q, sc, n = run_fp8(dd, d, path=path, bf16_normed=bf16_normed)
    ref = gu.oracle_for(d)
    check_fp8(q, sc, ref, d["gamma"], d["eps"], abs_floor=gu.ABS * d["row_scale"])
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    assert np.array_equal(r, r0)
    if bf16_normed:
        assert np.array_equal(n, n0)


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_extreme_rows_checked_binding(path):
    """The tensor binding (the checked entry point) and its FP8 form on the
    same rows give the bits of the plain C calls."""
    d = extreme_inputs(seed=4500)
    dd = gu.to_device(d)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    r1, n1 = gu.run(dd, d["eps"], d["scale"], path=path, api="binding")
    assert np.array_equal(r0, r1) and np.array_equal(n0, n1)
    a = run_fp8(dd, d, path=path, bf16_normed=True)
    b = run_fp8(dd, d, path=path, bf16_normed=True, api="binding")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_extreme_rows_dense(path):
    """The dense tail (x + residual, no routed part) on scaled rows, bf16 and
    FP8 output, against the oracle."""
    T, H = len(EXPS), 2048
    d = synth.dense_inputs(T, H, seed=4600)
    d["eps"] = 0.0
    c = np.array([2.0 ** k for k in EXPS])
    for t, ct in enumerate(c):
        d["x"][t] = _scale_bf16(d["x"][t], ct)
        d["residual"][t] = _scale_bf16(d["residual"][t], ct)
    x, res, g = gu.dev_bf16(d["x"]), gu.dev_bf16(d["residual"]), gu.dev_bf16(d["gamma"])
    with gu.forced(path, 0, 0):
        r, n = mfr.residual_add_rmsnorm(x, res, g, 0.0)
        r8, q, sc, n8 = mfr.residual_add_rmsnorm_fp8(x, res, g, 0.0, bf16_normed=True)
    torch.cuda.synchronize()
    ref = oracle.residual_rmsnorm(d["x"], d["residual"], d["gamma"], 0.0)
    assert_gate_rows(gu.host_u16(r), ref["s"], ref["residual_out"], c, "residual_out")
    assert_gate_rows(gu.host_u16(n), ref["normed_exact"], ref["normed_out"], np.ones_like(c),
                     "normed_out")
    assert np.array_equal(gu.host_u16(r8), gu.host_u16(r))
    assert np.array_equal(gu.host_u16(n8), gu.host_u16(n))
    check_fp8(q.view(torch.uint8).cpu().numpy(), sc.cpu().numpy().astype(np.float64), ref,
              d["gamma"], 0.0, abs_floor=gu.ABS * c)


def test_overflowing_s_is_infinite_on_both_sides():
    """Beyond the range: a token whose residual and shared output are both
    near the top of the bf16 range, so their sum leaves fp32. residual_out is
    infinite there on both sides (the oracle's fp64 s rounds to infinity in
    bf16 as well), and that element's normed value is NaN on the GPU
    (inf / inf). The other tokens are untouched."""
    d = synth.generate(3, 2048, 8, scale=2.5, seed=4700)
    big = synth.f32_to_bf16_bits(np.array([3.0e38], dtype=np.float32))[0]
    d["residual"][1, 9] = big
    d["shared_out"][1, 9] = big
    r, n = gu.run(gu.to_device(d), d["eps"], d["scale"])
    ref = gu.oracle_for(d)
    assert np.isinf(gu.bf16_f64(r[1, 9])) and np.isinf(gu.bf16_f64(ref["residual_out"][1, 9]))
    assert np.isnan(gu.bf16_f64(n[1, 9]))
    keep = np.array([0, 2])
    gu.check(d, r[keep], n[keep], ref={k: v[keep] for k, v in ref.items()})
