"""Exact-arithmetic helpers for pinning the oracle (tests only).

These do not share code with the oracle: rounding here works on Python
Fractions with the language's own round-half-to-even, and square roots go
through the decimal module at 60 significant digits.
"""
import struct
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

BF16_MAX_FINITE = Fraction(2**8 - 1, 2**7) * Fraction(2) ** 127  # (2 - 2^-7) * 2^127
OVERFLOW = Fraction(2) ** 128


def bits_to_fraction(b):
    """Exact value of a finite bf16 bit pattern."""
    f = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]
    return Fraction(f)


def fraction_to_bf16_bits(q):
    """Round an exact rational to the nearest bf16, ties to even; return the bits."""
    q = Fraction(q)
    neg = q < 0
    a = -q if neg else q
    sign = 0x8000 if neg else 0
    if a == 0:
        return sign
    # floor(log2 a), exactly
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e, -126) - 7
    quantum = Fraction(2) ** qe
    n = round(a / quantum)  # Fraction.__round__ rounds half to even
    y = n * quantum
    if y >= OVERFLOW:
        return sign | 0x7F80
    f32 = struct.unpack("<I", struct.pack("<f", float(y)))[0]
    assert f32 & 0xFFFF == 0, "rounded value is not a bf16"
    return sign | (f32 >> 16)


def decimal_of(q, prec=60):
    with localcontext() as ctx:
        ctx.prec = prec
        return Decimal(q.numerator) / Decimal(q.denominator)


def exact_token(rows, perm_idx, topk_w, shared, residual, gamma, eps, scale):
    """Exact evaluation of one token: s as Fractions, the normed value as a
    60-digit Decimal converted to Fraction. Arguments are Python floats/lists."""
    H = len(gamma)
    s = []
    for h in range(H):
        routed = Fraction(0)
        for idx, w in zip(perm_idx, topk_w):
            if idx < 0:
                continue
            routed += Fraction(w) * Fraction(rows[idx][h])
        s.append(Fraction(scale) * routed + Fraction(shared[h]) + Fraction(residual[h]))
    ms = sum((x * x for x in s), Fraction(0)) / H
    with localcontext() as ctx:
        ctx.prec = 60
        denom = decimal_of(ms + Fraction(eps)).sqrt()
        normed = []
        for h in range(H):
            if denom == 0:
                normed.append(None)
                continue
            y = decimal_of(s[h]) / denom * decimal_of(Fraction(gamma[h]))
            normed.append(Fraction(y))
    return s, normed


def bf16_values(bits):
    """float64 values of bf16 bit patterns (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


E4M3_MAX = Fraction(448)


def e4m3_code_value(code):
    """Exact value of a finite OCP E4M3 code (1 sign, 4 exponent bits with bias
    7, 3 mantissa bits; 0x7F / 0xFF are NaN and not accepted)."""
    code = int(code) & 0xFF
    sign = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    assert not (e == 0xF and m == 0x7), "NaN code"
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def fraction_to_e4m3_code(q):
    """Nearest E4M3 value to the exact rational q (ties to the even code),
    saturating to +-448; by search over the 127 non-negative finite codes."""
    q = Fraction(q)
    sign = 0x80 if q < 0 else 0
    a = -q if q < 0 else q
    if a >= E4M3_MAX:
        return sign | 0x7E
    best = None
    for code in range(0x7F):  # 0x00 .. 0x7E, increasing values
        d = abs(e4m3_code_value(code) - a)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return sign | best[1]
