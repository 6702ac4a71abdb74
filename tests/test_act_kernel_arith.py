"""CPU check of the activation quantizer kernel's division recipe (host
logic; no GPU).  The kernel decides each code on q1 = q0 + fma(-q0, b, a) * r
with a = x * (7/8) * pre, b = max * pre / 512, r = fl(1/b), q0 = fl(a * r)
(csrc/coat_act.hip, act_quot).  Here every FP32 step is emulated exactly
(fractions, rounded once to FP32, ties to even), and the E4M3 rounding of q1
must equal the definition's rounding of the exact quotient 448 x / max
(e4m3_exact) on random BF16 groups, on groups built from exact ties with
maxima that are not powers of two, and on tiny and huge groups."""
from fractions import Fraction

import numpy as np
import torch

from e4m3_exact import E4M3_VALUES, nearest_code


def f32(fr: Fraction) -> Fraction:
    """fr rounded once to FP32 (nearest, ties to even), as a Fraction."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # subnormals share the 2^-149 quantum
    quantum = Fraction(2) ** (e - 23)
    units = a / quantum
    lo = units.numerator // units.denominator
    rem = units - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def kernel_code(x: float, amax: float) -> int:
    """E4M3 code of x as the kernel computes it, every FP32 step exact."""
    pre = Fraction(2) ** 64 if amax < 2.0 ** -100 else Fraction(1)
    c = Fraction(7, 8) * pre
    b = f32(Fraction(amax) * pre / 512)
    r = f32(1 / b)
    a = f32(Fraction(x) * c)              # exact for BF16 x (asserted below)
    assert a == Fraction(x) * c
    q0 = f32(a * r)
    e = f32(a - q0 * b)                   # FMA: one rounding
    q1 = f32(e * r + q0)                  # FMA: one rounding
    if q1 == 0:                           # an underflow keeps the sign of a nonzero x
        return 0x80 if x < 0 else 0x00
    return nearest_code(q1)


def exact_code(x: float, amax: float) -> int:
    return nearest_code(Fraction(448) * Fraction(x) / Fraction(amax))


def _bf16(v):
    return torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double().numpy()


def test_random_bf16_groups():
    rng = np.random.default_rng(0)
    for scale in (1.0, 50.0, 3e-3, 1e-39, 2.0 ** -110, 1e30):
        x = _bf16(rng.standard_normal(2048) * scale)
        x = x.reshape(16, 128)
        for grp in x:
            amax = float(np.abs(grp).max())
            if amax == 0:
                continue
            for v in grp:
                assert kernel_code(float(v), amax) == exact_code(float(v), amax), (v, amax)


def test_exact_ties_any_max():
    for amax in (3.25, 98.0, 25.5, 12.75, 7.0, 3.0 * 2.0 ** -20, 3.0 * 2.0 ** 99, 5.0 * 2.0 ** -120):
        n = 0
        for lo, hi in zip(E4M3_VALUES, E4M3_VALUES[1:]):
            x = (lo + hi) / 2 * Fraction(amax) / 448
            xb = float(_bf16(float(x)))
            if Fraction(xb) != x:
                continue
            n += 1
            for v in (xb, -xb):
                assert kernel_code(v, amax) == exact_code(v, amax), (v, amax)
        assert n >= 4


def test_group_max_and_signed_zero():
    for amax in (3.25, 1e-39, 2.0 ** -110, 3.3e38):
        amax = float(_bf16(amax))
        assert kernel_code(amax, amax) == 0x7E
        assert kernel_code(-amax, amax) == 0xFE
        assert kernel_code(-0.0, amax) == 0x00
    # a quotient far below FP32's range still rounds to a signed zero
    assert kernel_code(-float(_bf16(1e-20)), float(_bf16(1e30))) == 0x80
