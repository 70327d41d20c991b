"""Exact IEEE-754 binary16/binary32 arithmetic on rationals, for pinning the oracle.

Written from the IEEE-754 definition of round-to-nearest-even: an operation
computes the exact rational result, then rounds it once to the format
(gradual underflow through subnormals, overflow to infinity). Nothing here
uses numpy's float16/float32 casts or arithmetic, so agreement with the
oracle is evidence about numpy's rounding and about the oracle's layout.

A value is a pair (sign, magnitude) where magnitude is a Fraction or the
string "inf"; this keeps the sign of zero.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Tuple, Union

Mag = Union[Fraction, str]
Val = Tuple[int, Mag]


class Fmt:
    def __init__(self, precision: int, emin: int, emax: int, exp_bits: int):
        self.p = precision      # significand bits, hidden bit included
        self.emin = emin        # exponent of the smallest normal number
        self.emax = emax        # exponent of the largest finite number
        self.exp_bits = exp_bits


FP16 = Fmt(11, -14, 15, 5)
FP32 = Fmt(24, -126, 127, 8)


def _floor_log2(q: Fraction) -> int:
    """Largest e with 2**e <= q, for q > 0."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_to(fmt: Fmt, sign: int, mag: Mag) -> Val:
    """Round an exact magnitude to the format, nearest with ties to even."""
    if mag == "inf":
        return sign, "inf"
    if mag == 0:
        return sign, Fraction(0)
    e = max(_floor_log2(mag), fmt.emin)
    quantum = Fraction(2) ** (e - fmt.p + 1)
    n = mag / quantum
    whole = n.numerator // n.denominator
    rem = n - whole
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    r = whole * quantum
    if r >= Fraction(2) ** (fmt.emax + 1):
        return sign, "inf"
    return sign, r


def add(fmt: Fmt, a: Val, b: Val) -> Val:
    (sa, ma), (sb, mb) = a, b
    if ma == "inf" or mb == "inf":
        if ma == "inf" and mb == "inf" and sa != sb:
            raise ValueError("inf - inf")
        return (sa, "inf") if ma == "inf" else (sb, "inf")
    exact = (-ma if sa else ma) + (-mb if sb else mb)
    if exact == 0:
        # an exact zero sum is +0 under round-to-nearest unless both operands are -0
        both_neg_zero = sa == 1 and sb == 1 and ma == 0 and mb == 0
        return (1 if both_neg_zero else 0), Fraction(0)
    return round_to(fmt, 1 if exact < 0 else 0, abs(exact))


def mul(fmt: Fmt, a: Val, b: Val) -> Val:
    (sa, ma), (sb, mb) = a, b
    s = sa ^ sb
    if ma == "inf" or mb == "inf":
        if ma == 0 or mb == 0:
            raise ValueError("0 * inf")
        return s, "inf"
    return round_to(fmt, s, ma * mb)


def from_f16_bits(h: int) -> Val:
    """Value of a binary16 bit pattern (no NaNs here)."""
    s = (h >> 15) & 1
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 0x1F:
        if f:
            raise ValueError("NaN")
        return s, "inf"
    if e == 0:
        return s, Fraction(f, 1 << 24)
    return s, Fraction(1024 + f, 1 << 10) * Fraction(2) ** (e - 15)


def to_f16_bits(v: Val) -> int:
    """Bit pattern of a value that is already representable in binary16."""
    s, m = v
    if m == "inf":
        return (s << 15) | 0x7C00
    if m == 0:
        return s << 15
    e = _floor_log2(m)
    if e < -14:
        f = m * (1 << 24)
        assert f.denominator == 1 and f < 1024
        return (s << 15) | int(f)
    frac = (m / Fraction(2) ** e - 1) * 1024
    assert frac.denominator == 1 and 0 <= frac < 1024 and e <= 15
    return (s << 15) | ((e + 15) << 10) | int(frac)


def value(v: Val) -> Fraction:
    s, m = v
    if m == "inf":
        raise ValueError("infinite")
    return -m if s else m


def decode_group_bits(codeword_bits, scale_bits) -> list:
    """One decoded group under the float32-sum, float32-scale, one-round rule.

    codeword_bits: list over m of g binary16 patterns (the selected codewords);
    returns g binary16 patterns.
    """
    g = len(codeword_bits[0])
    s = from_f16_bits(scale_bits)
    out = []
    for k in range(g):
        acc = from_f16_bits(codeword_bits[0][k])      # widening to fp32 is exact
        for m in range(1, len(codeword_bits)):
            acc = add(FP32, acc, from_f16_bits(codeword_bits[m][k]))
        acc = mul(FP32, acc, s)
        out.append(to_f16_bits(round_to(FP16, acc[0], acc[1])))
    return out
