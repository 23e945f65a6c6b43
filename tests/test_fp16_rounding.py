"""Pin: the oracle stores norms and decoded values by NumPy casts from fp64.
Those casts must be single round-to-nearest-even conversions (no detour through
fp32, whose double rounding differs).  Checked against exact rational rounding."""
from fractions import Fraction

import numpy as np


def _rne_fp16_exact(v: float) -> float:
    """Round a finite double to the nearest fp16 value, ties to even, by exact arithmetic."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    a = Fraction(abs(v))
    if a >= Fraction(65520):
        return sign * float("inf")
    # exponent of the fp16 spacing: normal numbers [2^e, 2^{e+1}) have spacing 2^{e-10}; subnormals 2^-24
    e = max(a.numerator.bit_length() - a.denominator.bit_length(), -14)
    while Fraction(2) ** e > a and e > -14:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    spacing = Fraction(2) ** (e - 10)
    q = a / spacing
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * spacing)


def test_direct_rounding_on_double_rounding_traps():
    # 1 + 2^-11 + 2^-40 is just above the fp16 tie between 1 and 1+2^-10; through
    # fp32 it becomes the exact tie and rounds down to 1 — direct rounding gives 1+2^-10.
    traps = [1 + 2.0 ** -11 + 2.0 ** -40, 1 + 3 * 2.0 ** -11 - 2.0 ** -40, 2.0 ** -24 * 1.5 + 2.0 ** -60,
             65519.999, 65520.0, 6.1e-5, 3.0e-8, 1024 + 0.5 + 2 ** -30]
    for v in traps:
        assert float(np.float64(v).astype(np.float16)) == _rne_fp16_exact(v), v
    assert float(np.float16(1 + 2.0 ** -11 + 2.0 ** -40)) == 1 + 2.0 ** -10


def test_random_values_round_correctly():
    rng = np.random.default_rng(3)
    v = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 20000)) * rng.choice([-1, 1], 20000)
    got = v.astype(np.float16).astype(np.float64)
    for a, g in zip(v, got):
        assert g == _rne_fp16_exact(float(a))


def test_fp32_cast_is_rne():
    v = np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 1 + 2.0 ** -24 + 2.0 ** -50])
    assert list(v.astype(np.float32).astype(np.float64)) == [1.0, 1 + 2.0 ** -22, 1 + 2.0 ** -23]
