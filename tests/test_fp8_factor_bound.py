"""The bound behind the FP8 factor of the fused kernels (csrc/mfr_device.h,
e4m3_factor): with c = RN(1/448), u = RN(m * c), r = the hardware reciprocal
of u (within 1 ulp), and f = RN(r * (1 - 2^-21)), the product m * f stays
below 448 for any rounding of those steps, so no element scaled by f can
round above the largest E4M3 value, and f stays within 2^-20 of 448 / m.
Checked here in float32 with every one-ulp choice of each step, on seeded
m over the range the kernels use (2^-90 to 2^128) and at its binade edges;
the products are exact in float64."""
import itertools

import numpy as np

F32 = np.float32
C = F32(1.0) / F32(448.0)
SHRINK = F32(1.0) - F32(2.0**-21)


def _ulps(x):
    """x and its float32 neighbours one ulp down and up (above FLT_MAX: inf,
    which the callers skip or never reach)."""
    x = F32(x)
    with np.errstate(over="ignore"):
        return (np.nextafter(x, F32(0)), x, np.nextafter(x, F32(np.inf)))


def _factors(m):
    """Every factor the three steps can give for m, each step rounded to
    nearest or one ulp off either way (the reciprocal's 1-ulp bound covers
    the nearest value and its two neighbours)."""
    m = F32(m)
    out = []
    for u in _ulps(m * C):
        r_exact = 1.0 / float(u)
        for r in _ulps(F32(r_exact)):
            for f in _ulps(F32(float(r) * float(SHRINK))):
                out.append(f)
    return out


def _ms():
    rng = np.random.default_rng(20240607)
    e = rng.uniform(-90, 127.9, size=4000)
    m = (2.0 ** e).astype(np.float32)
    edges = [F32(2.0**k) for k in range(-90, 128, 7)]
    edges += [np.nextafter(F32(2.0**k), F32(0)) for k in range(-89, 128, 7)]
    edges += [F32(448.0), F32(1.0), np.finfo(np.float32).max]
    return list(m) + edges


def test_factor_keeps_the_row_maximum_at_or_below_448():
    for m in _ms():
        for f in _factors(m):
            assert float(m) * float(f) < 448.0, (float(m), float(f))


def test_factor_is_within_2_pow_minus_20_of_the_quotient():
    for m in _ms():
        q = 448.0 / float(m)
        for f in _factors(m):
            assert abs(float(f) - q) <= 2.0**-20 * q, (float(m), float(f))


def test_scale_product_is_within_2_pow_minus_20_of_the_quotient():
    """The per-token scale rmax * RN(1/448), with rmax within an ulp."""
    for m in _ms():
        q = float(m) / 448.0
        for rm in _ulps(m):
            s = F32(rm * C)
            if not np.isfinite(s) or s == 0:
                continue
            assert abs(float(s) - q) <= 2.0**-20 * q, (float(m), float(s))
