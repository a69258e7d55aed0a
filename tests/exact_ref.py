"""Independent exact reference for tiny cases, in pure-Python rationals.

Used only to pin the oracle.  Nothing here calls a float operation on the
quantities being checked: bf16 values are decoded to exact ``Fraction``s,
every binary32 rounding the method prescribes is carried out by
``round_to_f32`` on exact rationals (nearest, ties to even, with gradual
underflow), and sums of products are exact integers.
"""
from __future__ import annotations

import math
from fractions import Fraction

F32_MIN_EXP = -126  # smallest normal exponent
F32_MANT = 23  # stored mantissa bits
F32_SUB_QUANTUM = Fraction(1, 2**149)


def bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    bits &= 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    assert exp != 0xFF, "finite inputs only"
    if exp == 0:
        v = Fraction(man, 2**7) * Fraction(2) ** (1 - 127)
    else:
        v = (1 + Fraction(man, 2**7)) * Fraction(2) ** (exp - 127)
    return sign * v


def _round_half_even(q: Fraction) -> int:
    """Nearest integer to a non-negative rational, ties to even."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def round_to_f32(v: Fraction) -> Fraction:
    """Exact value of RN_binary32(v), ties to even, gradual underflow, no overflow handling."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix the float estimate of the exponent so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < F32_MIN_EXP:
        quantum = F32_SUB_QUANTUM
    else:
        quantum = Fraction(2) ** (e - F32_MANT)
    m = _round_half_even(a / quantum)
    r = m * quantum
    assert r < Fraction(2) ** 128, "overflow not expected"
    return sign * r


def bf16_round(v: Fraction) -> int:
    """bf16 bit pattern of RN_bf16(v) for a value already representable in binary32."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    if e < F32_MIN_EXP:
        quantum = Fraction(2) ** (F32_MIN_EXP - 7)
    else:
        quantum = Fraction(2) ** (e - 7)
    m = _round_half_even(a / quantum)
    r = m * quantum
    # re-encode r as bf16 bits
    if r == 0:
        return sign
    e2 = math.floor(math.log2(r.numerator) - math.log2(r.denominator))
    while Fraction(2) ** e2 > r:
        e2 -= 1
    while Fraction(2) ** (e2 + 1) <= r:
        e2 += 1
    if e2 < F32_MIN_EXP:
        man = int(r / Fraction(2) ** (F32_MIN_EXP - 7))
        return sign | man
    man = int(r / Fraction(2) ** (e2 - 7)) - 128
    assert 0 <= man < 128
    return sign | ((e2 + 127) << 7) | man


def quantize_group(xbits, mode: str = "rne", us=None):
    """(codes, scale) for one group of bf16 bit patterns, exactly as the
    definition reads: s = RN(amax/127); v = RN(x/s); RNE: round half even;
    SR: floor(RN(v + u)); clamp to [-127, 127]; all-zero group -> s = 0."""
    xs = [bf16_value(b) for b in xbits]
    amax = max(abs(v) for v in xs)
    s = round_to_f32(amax / 127)
    codes = []
    for i, x in enumerate(xs):
        if s == 0:
            codes.append(0)
            continue
        v = round_to_f32(x / s)
        if mode == "rne":
            r = _round_half_even(v) if v >= 0 else -_round_half_even(-v)
        else:
            t = round_to_f32(v + us[i])
            r = math.floor(t)
        codes.append(max(-127, min(127, r)))
    return codes, s


def epilogue_bits(acc: int, sa: Fraction, sb: Fraction) -> int:
    """bf16 bits of RN_bf16(RN32(RN32(RN32(acc) * sa) * sb))."""
    y = round_to_f32(Fraction(acc))
    y = round_to_f32(y * sa)
    y = round_to_f32(y * sb)
    return bf16_round(y)
