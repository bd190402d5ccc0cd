"""Exactness of arithmetic reformulations used inside the HIP kernels, checked
on the CPU with exact rational arithmetic (no GPU needed).

The NVFP4 block scale divides the block amax b (a bf16 value) by 6.  The
kernel replaces the IEEE division by q0 = RN(b * RN(1/6)), r = RN(b - 6 q0)
(an FMA) and q = RN(r * RN(1/6) + q0) (an FMA).  This is claimed equal to
RN(b / 6) for every finite non-negative bf16 b; here that claim is checked for
all 32640 of them, with every rounding modelled exactly (binary32, ties to
even, subnormals included).
"""
from fractions import Fraction

import pytest


def rn32(q: Fraction) -> Fraction:
    """Nearest binary32 value to the rational q >= 0 (ties to even, with
    subnormals; no overflow occurs for the values used here)."""
    assert q >= 0
    if q == 0:
        return Fraction(0)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    assert Fraction(2) ** e <= q < Fraction(2) ** (e + 1)
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = q / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * quantum


def bf16_value(h: int) -> Fraction:
    exp, man = (h >> 7) & 0xFF, h & 0x7F
    if exp == 0:
        return man * Fraction(2) ** -133
    return (128 + man) * Fraction(2) ** (exp - 134)


def test_rn32_model():
    # the model agrees with the hardware format on known values
    assert rn32(Fraction(1, 3)) == Fraction(float.fromhex("0x1.555556p-2"))
    assert rn32(Fraction(2) ** -149) == Fraction(2) ** -149
    assert rn32(Fraction(3, 2) * Fraction(2) ** -149) == Fraction(2) ** -148   # tie -> even
    assert rn32(Fraction(1, 2) * Fraction(2) ** -149) == 0                      # tie -> even (0)
    assert rn32(1 + Fraction(1, 2 ** 24)) == 1                                   # tie -> even
    assert rn32(1 + Fraction(3, 2 ** 24)) == 1 + Fraction(1, 2 ** 22)


def test_div6_fma_sequence_is_correctly_rounded():
    c = rn32(Fraction(1, 6))
    assert c == Fraction(float.fromhex("0x1.555556p-3"))   # the kernel's constant
    checked = 0
    for h in range(0x0000, 0x7F80):                           # every finite bf16 >= 0
        b = bf16_value(h)
        q0 = rn32(b * c)
        exact_r = b - 6 * q0
        r = rn32(abs(exact_r)) * (1 if exact_r >= 0 else -1)
        assert r == exact_r, f"residual not exact for bf16 {h:#06x}"
        t = r * c + q0
        q = rn32(t) if t >= 0 else -rn32(-t)
        assert q == rn32(b / 6), f"bf16 {h:#06x}"
        checked += 1
    assert checked == 32640
