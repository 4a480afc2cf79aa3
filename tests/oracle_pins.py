"""Pins for the oracle: checks that tie it to something other than itself.

Each pin takes an oracle handle (``oracle.Oracle``) and raises AssertionError
when the oracle disagrees with:
  * hand-computed cases (tests/golden/hand_cases.json),
  * exact rational brute force on tiny dyadic inputs,
  * library special cases (scipy.sparse matmul for the top-k sum, torch's
    rms_norm for the normalisation, torch's fp32->bf16 converter for rounding),
  * closed forms and invariants of the definition.
The same pins run against deliberately broken builds of the oracle source in
test_oracle_mutants.py, to show that plausible mistakes are caught.
"""
import json
import os
from fractions import Fraction

import numpy as np
import scipy.sparse
import torch

import synth
from tests import exact

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")
NAN_BF16 = 0x7FC0


def _bits(values):
    """bf16 bits of values that are exactly bf16 (checked)."""
    out = np.array([exact.fraction_to_bf16_bits(Fraction(str(v))) for v in np.ravel(values)],
                   dtype=np.uint16).reshape(np.shape(values))
    back = exact.bf16_values(out)
    assert np.array_equal(back, np.asarray(values, dtype=np.float64)), "fixture value is not bf16"
    return out


def _is_nan_bits(b):
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


# --------------------------------------------------------------------------
# Rounding double -> bf16
# --------------------------------------------------------------------------

def pin_rne_roundtrip(o):
    """Every bf16 value converts back to its own bit pattern; NaN stays NaN."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = exact.bf16_values(bits)
    out = o.rne_bf16_from_f64(vals)
    nan = _is_nan_bits(bits)
    assert np.array_equal(out[~nan], bits[~nan])
    assert np.all(_is_nan_bits(out[nan]))
    assert np.array_equal(out[nan] & 0x8000, bits[nan] & 0x8000), "NaN sign lost"


def pin_rne_midpoints(o):
    """Midpoints between neighbours round to the even pattern; a nudge either
    way rounds to the nearer neighbour. Covers zero, subnormals and normals."""
    lo = np.arange(0, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    hi = lo + np.uint16(1)
    a, c = exact.bf16_values(lo), exact.bf16_values(hi)
    m = (a + c) / 2.0  # exact: neighbours have at most 8 significant bits
    even = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(o.rne_bf16_from_f64(m), even)
    assert np.array_equal(o.rne_bf16_from_f64(np.nextafter(m, np.inf)), hi)
    assert np.array_equal(o.rne_bf16_from_f64(np.nextafter(m, 0.0)), lo)
    assert np.array_equal(o.rne_bf16_from_f64(-m), even | np.uint16(0x8000))


def pin_rne_overflow_and_specials(o):
    thr = (2.0 - 2.0 ** -8) * 2.0 ** 127  # midpoint between the largest bf16 and 2^128
    x = np.array([thr, np.nextafter(thr, 0.0), -thr, 2.0 ** 200, np.inf, -np.inf, 0.0, -0.0,
                  2.0 ** -134, np.nextafter(2.0 ** -134, 1.0), 3 * 2.0 ** -134, 2.0 ** -140])
    want = np.array([0x7F80, 0x7F7F, 0xFF80, 0x7F80, 0x7F80, 0xFF80, 0x0000, 0x8000,
                     0x0000, 0x0001, 0x0002, 0x0000], dtype=np.uint16)
    assert np.array_equal(o.rne_bf16_from_f64(x), want)


def pin_rne_vs_torch(o):
    """Library special case: for doubles that are binary32 values, rounding
    to bf16 equals torch's float32 -> bfloat16 conversion."""
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.rne_bf16_from_f64(f.astype(np.float64)), ref)


def pin_rne_vs_exact_random(o):
    """Doubles that are not binary32 values, against exact rational rounding."""
    rng = np.random.default_rng(11)
    mant = rng.random(3000) + 1.0
    e = rng.integers(-140, 130, size=3000)
    x = np.ldexp(mant, e) * np.where(rng.random(3000) < 0.5, -1.0, 1.0)
    got = o.rne_bf16_from_f64(x)
    want = np.array([exact.fraction_to_bf16_bits(Fraction(float(v))) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# The fused op
# --------------------------------------------------------------------------

def _hand_case_arrays(case, eps):
    rows = np.asarray(case["rows"], dtype=np.float64)
    return dict(
        expert_out=_bits(rows),
        perm_idx=np.asarray(case["perm_idx"], dtype=np.int32),
        topk_w=np.asarray(case["topk_w"], dtype=np.float32),
        shared_out=_bits(np.asarray(case["shared"], dtype=np.float64)),
        residual=_bits(np.asarray(case["residual"], dtype=np.float64)),
        gamma=_bits(np.asarray(case["gamma"], dtype=np.float64)),
        eps=eps, scale=case["scale"])


def hand_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def dense_hand_cases():
    with open(GOLDEN) as f:
        return json.load(f)["dense_cases"]


def pin_hand_cases(o):
    for case in hand_cases():
        for eps in case["eps_values"]:
            a = _hand_case_arrays(case, eps)
            out = o.finalize_rmsnorm(**a)
            want_r = _bits(np.asarray(case["residual_out"], dtype=np.float64))
            want_n = _bits(np.asarray(case["normed_out"], dtype=np.float64))
            assert np.array_equal(out["residual_out"], want_r), (case["name"], eps, "residual_out")
            assert np.array_equal(out["normed_out"], want_n), (case["name"], eps, "normed_out")


def _near_tie(q, rel=2.0 ** -48):
    """True if the exact value q lies within rel*|q| of a bf16 rounding tie."""
    if q == 0:
        return False
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 7)
    n = a / quantum
    frac = n - (n.numerator // n.denominator)
    return abs(frac - Fraction(1, 2)) * quantum <= Fraction(rel) * a


def random_dyadic_case(rng):
    T = int(rng.integers(1, 4))
    H = int(rng.choice([8, 16]))
    K = int(rng.integers(1, 4))
    R = T * K + int(rng.integers(0, 3))
    rows = rng.integers(-32, 33, size=(R, H)) / 8.0
    perm = rng.integers(0, R, size=(T, K)).astype(np.int32)
    perm[rng.random((T, K)) < 0.2] = -1
    w = (rng.integers(0, 17, size=(T, K)) / 16.0).astype(np.float32)
    shared = rng.integers(-32, 33, size=(T, H)) / 8.0
    resid = rng.integers(-32, 33, size=(T, H)) / 8.0
    gamma = rng.integers(1, 17, size=H) / 8.0
    scale = float(rng.choice([0.5, 1.0, 2.0]))
    eps = float(rng.choice([0.0, 2.0 ** -10, float(np.float32(1e-6))]))
    return dict(rows=rows, perm=perm, w=w, shared=shared, resid=resid, gamma=gamma,
                scale=scale, eps=eps, T=T, H=H, K=K)


def pin_bruteforce_exact(o, n_cases=60, seed=2026):
    """Exact brute force on tiny dyadic inputs: exact s (rationals) rounded to
    bf16, and the normed value from a 60-digit square root, rounded to bf16."""
    rng = np.random.default_rng(seed)
    for ci in range(n_cases):
        c = random_dyadic_case(rng)
        out = o.finalize_rmsnorm(_bits(c["rows"]), c["perm"], c["w"], _bits(c["shared"]),
                                 _bits(c["resid"]), _bits(c["gamma"]), c["eps"], c["scale"])
        for t in range(c["T"]):
            s, normed = exact.exact_token(c["rows"].tolist(), c["perm"][t].tolist(),
                                          [float(x) for x in c["w"][t]], c["shared"][t].tolist(),
                                          c["resid"][t].tolist(), c["gamma"].tolist(),
                                          c["eps"], c["scale"])
            for h in range(c["H"]):
                assert out["s"][t, h] == float(s[h]), (ci, t, h, "s")
                assert out["residual_out"][t, h] == exact.fraction_to_bf16_bits(s[h]), (ci, t, h)
                if normed[h] is None:
                    assert _is_nan_bits(out["normed_out"][t, h]), (ci, t, h, "0/0")
                    continue
                want = exact.fraction_to_bf16_bits(normed[h])
                if out["normed_out"][t, h] != want:
                    assert _near_tie(normed[h]), (ci, t, h, "normed")


def _csr_weights(perm, w, R):
    T, K = perm.shape
    tt, kk = np.nonzero(perm >= 0)
    return scipy.sparse.csr_matrix((w[tt, kk].astype(np.float64), (tt, perm[tt, kk])), shape=(T, R))


def pin_sparse_matmul(o):
    """Library special case: the routed part equals scale * (W @ E) with W the
    sparse [T, R] matrix of routing weights (scipy.sparse, fp64)."""
    for cfg, T in (("tiny", 4), ("decode_masked", 64), ("decode_masked", 1)):
        d = synth.config_inputs(cfg, T)
        out = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                                 d["residual"], d["gamma"], d["eps"], d["scale"])
        E = exact.bf16_values(d["expert_out"])
        W = _csr_weights(d["perm_idx"], d["topk_w"], d["R"])
        sh, rs = exact.bf16_values(d["shared_out"]), exact.bf16_values(d["residual"])
        ref = d["scale"] * (W @ E) + sh + rs
        mag = abs(d["scale"]) * (abs(W) @ abs(E)) + abs(sh) + abs(rs)
        assert np.all(np.abs(out["s"] - ref) <= 1e-12 * mag + 1e-300), (cfg, T)


def pin_rms_norm_library(o):
    """Library special case: torch.nn.functional.rms_norm in float64 on the
    oracle's unrounded sum reproduces its unrounded normed value."""
    for cfg, T in (("tiny", 4), ("decode_masked", 64), ("decode", 4)):
        d = synth.config_inputs(cfg, T)
        out = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                                 d["residual"], d["gamma"], d["eps"], d["scale"])
        g = torch.from_numpy(exact.bf16_values(d["gamma"]))
        ref = torch.nn.functional.rms_norm(torch.from_numpy(out["s"]), (d["H"],), weight=g,
                                           eps=d["eps"]).numpy()
        assert np.all(np.abs(out["normed_exact"] - ref) <= 1e-12 * np.abs(ref) + 1e-300), (cfg, T)


def pin_closed_form_k1(o):
    """K = 1 with weight 1: s = residual + shared + scale * row (exact rationals),
    normed = s / sqrt(mean(s^2) + eps) * gamma (separate fp64 evaluation)."""
    d = synth.generate(4, 256, 1, scale=2.5, seed=99)
    d["topk_w"][:] = 1.0
    out = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                             d["residual"], d["gamma"], d["eps"], d["scale"])
    E, sh, rs = (exact.bf16_values(d[k]) for k in ("expert_out", "shared_out", "residual"))
    g = exact.bf16_values(d["gamma"])
    for t in range(4):
        row = E[d["perm_idx"][t, 0]]
        for h in range(256):
            q = Fraction(float(rs[t, h])) + Fraction(float(sh[t, h])) + Fraction(d["scale"]) * Fraction(float(row[h]))
            assert out["residual_out"][t, h] == exact.fraction_to_bf16_bits(q), (t, h)
    s = out["s"]
    y = s / np.sqrt(np.mean(s * s, axis=1, keepdims=True) + d["eps"]) * g
    assert np.all(np.abs(out["normed_exact"] - y) <= 1e-13 * np.abs(y))


def pin_slot_permutation(o):
    """Permuting the K slots of a token (index and weight together) leaves the
    outputs unchanged."""
    rng = np.random.default_rng(5)
    for cfg, T in (("tiny", 4), ("decode_masked", 64)):
        d = synth.config_inputs(cfg, T)
        base = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                                  d["residual"], d["gamma"], d["eps"], d["scale"])
        order = np.argsort(rng.random(d["perm_idx"].shape), axis=1)
        p2 = np.take_along_axis(d["perm_idx"], order, axis=1)
        w2 = np.take_along_axis(d["topk_w"], order, axis=1)
        out = o.finalize_rmsnorm(d["expert_out"], p2, w2, d["shared_out"], d["residual"],
                                 d["gamma"], d["eps"], d["scale"])
        assert np.array_equal(out["residual_out"], base["residual_out"])
        assert np.array_equal(out["normed_out"], base["normed_out"])
        assert np.all(np.abs(out["s"] - base["s"]) <= 1e-13 * np.abs(base["s"]) + 1e-12)


def pin_zero_routed(o):
    """All weights zero, or all slots masked: residual_out = RNE(shared + residual)."""
    d = synth.generate(4, 512, 8, scale=2.5, seed=3)
    sh, rs = exact.bf16_values(d["shared_out"]), exact.bf16_values(d["residual"])
    want = np.array([exact.fraction_to_bf16_bits(Fraction(float(a)) + Fraction(float(b)))
                     for a, b in zip(sh.ravel(), rs.ravel())], dtype=np.uint16).reshape(sh.shape)
    for variant in ("zero_weights", "all_masked"):
        p, w = d["perm_idx"].copy(), d["topk_w"].copy()
        if variant == "zero_weights":
            w[:] = 0.0
        else:
            p[:] = -1
        out = o.finalize_rmsnorm(d["expert_out"], p, w, d["shared_out"], d["residual"],
                                 d["gamma"], d["eps"], d["scale"])
        assert np.array_equal(out["residual_out"], want), variant


def pin_scale_invariance(o):
    """shared, residual and scale times c = 2^j, eps times c^2: residual_out
    scales by exactly c and normed_out is unchanged."""
    d = synth.config_inputs("tiny", 4)
    base = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                              d["residual"], d["gamma"], d["eps"], d["scale"])
    for j in (-2, 3):
        c = 2.0 ** j
        sh = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(d["shared_out"]) * np.float32(c))
        rs = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(d["residual"]) * np.float32(c))
        out = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], sh, rs, d["gamma"],
                                 d["eps"] * c * c, d["scale"] * c)
        assert np.array_equal(exact.bf16_values(out["residual_out"]),
                              exact.bf16_values(base["residual_out"]) * c), j
        assert np.array_equal(out["normed_out"], base["normed_out"]), j


def pin_unit_rms(o):
    """gamma = 1: the RMS of each token's normed output is sqrt(ms / (ms + eps))."""
    d = synth.config_inputs("decode", 4)
    ones = synth.f32_to_bf16_bits(np.ones(d["H"], dtype=np.float32))
    out = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                             d["residual"], ones, d["eps"], d["scale"])
    ms = np.mean(out["s"] ** 2, axis=1)
    want = np.sqrt(ms / (ms + d["eps"]))
    got = np.sqrt(np.mean(out["normed_exact"] ** 2, axis=1))
    assert np.all(np.abs(got - want) <= 1e-13 * want)
    got_r = np.sqrt(np.mean(exact.bf16_values(out["normed_out"]) ** 2, axis=1))
    assert np.all(np.abs(got_r - want) <= 2.0 ** -8)


def pin_masked_nan_poison(o):
    """Masked slots are skipped entirely: NaN weights on masked slots and NaN in
    every row that no valid index names leave the outputs bit-identical."""
    d = synth.config_inputs("decode_masked", 64)
    base = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                              d["residual"], d["gamma"], d["eps"], d["scale"])
    E = d["expert_out"].copy()
    used = np.zeros(d["R"], dtype=bool)
    used[d["perm_idx"][d["perm_idx"] >= 0]] = True
    E[~used] = NAN_BF16
    w = d["topk_w"].copy()
    w[d["perm_idx"] < 0] = np.nan
    assert (~used).sum() > 0 and np.isnan(w).sum() > 0
    out = o.finalize_rmsnorm(E, d["perm_idx"], w, d["shared_out"], d["residual"], d["gamma"],
                             d["eps"], d["scale"])
    assert np.array_equal(out["residual_out"], base["residual_out"])
    assert np.array_equal(out["normed_out"], base["normed_out"])


def pin_weight_zero_reads_row(o):
    """A zero weight on a valid index is not a mask: the row is read, so a NaN
    in it reaches the output (0 * NaN = NaN)."""
    d = synth.generate(1, 16, 2, scale=1.0, seed=4)
    E = d["expert_out"].copy()
    w = d["topk_w"].copy()
    w[0, 1] = 0.0
    E[d["perm_idx"][0, 1], 3] = NAN_BF16
    out = o.finalize_rmsnorm(E, d["perm_idx"], w, d["shared_out"], d["residual"], d["gamma"],
                             d["eps"], d["scale"])
    assert _is_nan_bits(out["residual_out"][0, 3])
    assert np.sum(_is_nan_bits(out["residual_out"])) == 1


def pin_index_range(o):
    """An index equal to the row count is rejected; the last row is accepted."""
    import oracle as oracle_pkg
    d = synth.generate(2, 16, 2, seed=6)
    p = d["perm_idx"].copy()
    p[1, 0] = d["R"] - 1
    o.finalize_rmsnorm(d["expert_out"], p, d["topk_w"], d["shared_out"], d["residual"],
                       d["gamma"], d["eps"], d["scale"])
    p[1, 0] = d["R"]
    try:
        o.finalize_rmsnorm(d["expert_out"], p, d["topk_w"], d["shared_out"], d["residual"],
                           d["gamma"], d["eps"], d["scale"])
    except oracle_pkg.OracleIndexError:
        return
    raise AssertionError("index == R was accepted")


# --------------------------------------------------------------------------
# Dense residual add + RMSNorm (no routed part)
# --------------------------------------------------------------------------

def pin_dense_hand_case(o):
    for case in dense_hand_cases():
        for eps in case["eps_values"]:
            out = o.residual_rmsnorm(_bits(np.asarray(case["x"], dtype=np.float64)),
                                     _bits(np.asarray(case["residual"], dtype=np.float64)),
                                     _bits(np.asarray(case["gamma"], dtype=np.float64)), eps)
            want_r = _bits(np.asarray(case["residual_out"], dtype=np.float64))
            want_n = _bits(np.asarray(case["normed_out"], dtype=np.float64))
            assert np.array_equal(out["residual_out"], want_r), (case["name"], eps)
            assert np.array_equal(out["normed_out"], want_n), (case["name"], eps)


def pin_dense_bruteforce_exact(o, n_cases=40, seed=77):
    """Exact rationals on tiny dyadic inputs: s = x + residual rounded once,
    the normed value from a 60-digit square root."""
    rng = np.random.default_rng(seed)
    for ci in range(n_cases):
        T = int(rng.integers(1, 4))
        H = int(rng.choice([8, 16]))
        x = rng.integers(-32, 33, size=(T, H)) / 8.0
        r = rng.integers(-64, 65, size=(T, H)) / 16.0
        g = rng.integers(1, 17, size=H) / 8.0
        eps = float(rng.choice([0.0, 2.0 ** -10, float(np.float32(1e-6))]))
        out = o.residual_rmsnorm(_bits(x), _bits(r), _bits(g), eps)
        for t in range(T):
            s, normed = exact.exact_token([[0.0] * H], [-1], [0.0], x[t].tolist(), r[t].tolist(),
                                          g.tolist(), eps, 1.0)
            for h in range(H):
                assert out["residual_out"][t, h] == exact.fraction_to_bf16_bits(s[h]), (ci, t, h)
                if normed[h] is None:
                    assert _is_nan_bits(out["normed_out"][t, h])
                    continue
                want = exact.fraction_to_bf16_bits(normed[h])
                if out["normed_out"][t, h] != want:
                    assert _near_tie(normed[h]), (ci, t, h, "normed")


def pin_dense_rms_norm_library(o):
    """torch.nn.functional.rms_norm in float64 of x + residual."""
    d = synth.generate(16, 2048, 1, seed=12)
    x, r = d["shared_out"], d["residual"]
    out = o.residual_rmsnorm(x, r, d["gamma"], d["eps"])
    s = exact.bf16_values(x) + exact.bf16_values(r)
    assert np.array_equal(out["s"], s)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(s), (2048,),
                                       weight=torch.from_numpy(exact.bf16_values(d["gamma"])),
                                       eps=d["eps"]).numpy()
    assert np.all(np.abs(out["normed_exact"] - ref) <= 1e-12 * np.abs(ref) + 1e-300)


def pin_dense_equals_all_masked_finalize(o):
    """The dense op on x equals the fused finalize with every slot masked and
    shared = x (values equal; a zero may differ in sign only)."""
    d = synth.generate(8, 1024, 4, scale=2.5, seed=13)
    p = np.full_like(d["perm_idx"], -1)
    a = o.finalize_rmsnorm(d["expert_out"], p, d["topk_w"], d["shared_out"], d["residual"],
                           d["gamma"], d["eps"], d["scale"])
    b = o.residual_rmsnorm(d["shared_out"], d["residual"], d["gamma"], d["eps"])
    for k in ("residual_out", "normed_out"):
        assert np.array_equal(exact.bf16_values(a[k]), exact.bf16_values(b[k])), k


# --------------------------------------------------------------------------
# Dynamic per-token FP8 (E4M3) quantisation
# --------------------------------------------------------------------------

FINITE_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def _e4m3_values(codes):
    """Library decode of E4M3 codes: torch's float8_e4m3fn widening (exact)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def pin_e4m3_roundtrip(o):
    """Every finite E4M3 value rounds back to its own code."""
    vals = _e4m3_values(FINITE_E4M3)
    assert np.array_equal(o.rne_e4m3_from_f64(vals), FINITE_E4M3)
    assert [float(exact.e4m3_code_value(c)) for c in FINITE_E4M3] == vals.tolist()


def pin_e4m3_midpoints_and_saturation(o):
    lo = np.arange(0, 0x7E, dtype=np.uint8)  # neighbours lo, lo + 1 up to 448
    a, c = _e4m3_values(lo), _e4m3_values(lo + 1)
    m = (a + c) / 2.0
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(o.rne_e4m3_from_f64(m), even)
    assert np.array_equal(o.rne_e4m3_from_f64(np.nextafter(m, np.inf)), lo + 1)
    assert np.array_equal(o.rne_e4m3_from_f64(np.nextafter(m, 0.0)), lo)
    assert np.array_equal(o.rne_e4m3_from_f64(-m), even | np.uint8(0x80))
    sat = o.rne_e4m3_from_f64(np.array([448.0, 449.0, 464.0, 1e30, np.inf, -448.0, -1e30,
                                        2.0 ** -10, -2.0 ** -10, 0.0, -0.0]))
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x00, 0x80]


def pin_e4m3_vs_torch(o):
    """Library special case: inside +-448 (where torch's float8_e4m3fn
    conversion does not need to saturate) the rounding equals torch's."""
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(100_000) * np.exp2(rng.integers(-12, 9, size=100_000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.rne_e4m3_from_f64(x.astype(np.float64)), ref)


def pin_e4m3_nan(o):
    """NaN has one E4M3 encoding, all exponent and mantissa bits set
    (S.1111.111), with the sign kept. This is a library special case:
    torch's float8_e4m3fn converter gives the same codes. In a row, a NaN
    element keeps that code and takes no part in amax."""
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert ref.tolist() == [0x7F, 0xFF]
    assert np.array_equal(o.rne_e4m3_from_f64(x.astype(np.float64)), ref)
    codes, scales, _ = o.fp8_quantize_rows(np.array([[1.0, np.nan, -7.0, 0.5]]))
    assert scales.tolist() == [7.0 / 448.0]
    assert (codes[0, 1] & 0x7F) == 0x7F and codes[0, 2] == 0xFE


def pin_e4m3_vs_exact(o):
    """Doubles that are not binary32 values, against exact rational search."""
    rng = np.random.default_rng(19)
    x = (rng.random(600) + 1.0) * np.exp2(rng.integers(-11, 10, size=600)) * np.where(
        rng.random(600) < 0.5, -1.0, 1.0)
    want = np.array([exact.fraction_to_e4m3_code(Fraction(float(v))) for v in x], dtype=np.uint8)
    assert np.array_equal(o.rne_e4m3_from_f64(x), want)


def pin_fp8_hand_case(o):
    with open(GOLDEN) as f:
        cases = json.load(f)["fp8_cases"]
    for case in cases:
        codes, scales, _ = o.fp8_quantize_rows(np.asarray(case["y"], dtype=np.float64))
        assert codes.tolist() == case["codes"], case["name"]
        assert scales.tolist() == case["scale"], case["name"]


def pin_fp8_quantize_properties(o):
    """On real normed rows: scale = amax / 448; the largest element becomes
    exactly +-448; every code is the nearest E4M3 value of y / scale; powers of
    two of y leave the codes unchanged and scale the scale; an all-zero row has
    scale 1 and zero codes."""
    d = synth.config_inputs("decode", 12)
    y = o.finalize_rmsnorm(d["expert_out"], d["perm_idx"], d["topk_w"], d["shared_out"],
                           d["residual"], d["gamma"], d["eps"], d["scale"])["normed_exact"]
    codes, scales, scaled = o.fp8_quantize_rows(y)
    amax = np.abs(y).max(axis=1)
    assert np.array_equal(scales, amax / 448.0)
    arg = np.abs(y).argmax(axis=1)
    top = codes[np.arange(len(arg)), arg]
    assert np.all((top & 0x7F) == 0x7E)
    vals = _e4m3_values(codes)
    grid = _e4m3_values(FINITE_E4M3)
    best = np.abs(scaled[..., None] - grid[None, None, :]).min(axis=-1)
    assert np.all(np.abs(vals - scaled) <= best)
    for j in (-3, 5):
        c2, s2, _ = o.fp8_quantize_rows(y * 2.0 ** j)
        assert np.array_equal(c2, codes) and np.array_equal(s2, scales * 2.0 ** j)
    cz, sz, _ = o.fp8_quantize_rows(np.zeros((2, 16)))
    assert np.all(cz == 0) and np.all(sz == 1.0)


ALL_PINS = [
    pin_rne_roundtrip, pin_rne_midpoints, pin_rne_overflow_and_specials, pin_rne_vs_torch,
    pin_rne_vs_exact_random, pin_hand_cases, pin_bruteforce_exact, pin_sparse_matmul,
    pin_rms_norm_library, pin_closed_form_k1, pin_slot_permutation, pin_zero_routed,
    pin_scale_invariance, pin_unit_rms, pin_masked_nan_poison, pin_weight_zero_reads_row,
    pin_index_range, pin_dense_hand_case, pin_dense_bruteforce_exact, pin_dense_rms_norm_library,
    pin_dense_equals_all_masked_finalize, pin_e4m3_roundtrip, pin_e4m3_midpoints_and_saturation,
    pin_e4m3_vs_torch, pin_e4m3_nan, pin_e4m3_vs_exact, pin_fp8_hand_case,
    pin_fp8_quantize_properties,
]
