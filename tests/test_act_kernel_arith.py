"""CPU check of the activation quantizer kernel's division recipe (host
logic; no GPU).  The kernel decides each code on q1 = fma(fma(-q0, b, a), r, q0)
with a = x * (7/8) * pre, b = max * pre / 512, r = fl(1/b), q0 = fl(a * r)
(csrc/coat_common.h, group_quot).  Here every FP32 step is emulated exactly
(fractions, rounded once to FP32, ties to even, with IEEE signed zeros), and
the E4M3 rounding of q1 must equal the definition's rounding of the exact
quotient 448 x / max (e4m3_exact) on random BF16 groups, on groups built from
exact ties with maxima that are not powers of two, and on tiny and huge
groups; -0.0 must come out as +0 (code 0x00) and a negative quotient that
underflows as -0 (0x80).  The linear layer forms r with the hardware
reciprocal (within one ulp): with r one or two ulps off, exact ties of FP32
quotients must still go to the even code, and BF16 codes must not change."""
import math
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


# An FP32 value as (magnitude-carrying Fraction, sign bit); the sign bit
# matters only for zeros, which IEEE arithmetic keeps signed.
def _val(x: float):
    return (Fraction(x), math.copysign(1.0, x) < 0)


def _round(exact: Fraction, zero_neg: bool):
    """One IEEE rounding to FP32 of an exact result; zero_neg is the sign an
    exact zero takes.  A nonzero result that rounds to zero keeps its sign."""
    if exact == 0:
        return (Fraction(0), zero_neg)
    return (f32(exact), exact < 0)


def _mul(x, y):
    return _round(x[0] * y[0], x[1] != y[1])


def _fma(x, y, z):
    """x * y + z, one rounding.  An exact zero sum is -0 only when both the
    product and the addend are negative zeros (round to nearest)."""
    p = x[0] * y[0]
    p_neg = x[1] != y[1]
    both_neg_zero = p == 0 and z[0] == 0 and p_neg and z[1]
    return _round(p + z[0], both_neg_zero)


def _ulp(v: Fraction) -> Fraction:
    """Spacing of FP32 values at the normal magnitude v."""
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    return Fraction(2) ** (e - 23)


def kernel_code(x: float, amax: float, r_ulps: int = 0, exact_a: bool = True) -> int:
    """E4M3 code of x as the kernel computes it, every FP32 step exact.
    r_ulps moves the reciprocal r = fl(1/b) by that many ulps: the hardware
    reciprocal that the linear layer uses is within one ulp of 1/b."""
    pre = Fraction(2) ** 64 if amax < 2.0 ** -100 else Fraction(1)
    c = (Fraction(7, 8) * pre, False)
    b = (f32(Fraction(amax) * pre / 512), False)
    r0 = f32(1 / b[0])
    r = (r0 + r_ulps * _ulp(r0), False)
    a = _mul(_val(x), c)
    if exact_a:                           # exact for BF16 x
        assert a[0] == Fraction(x) * c[0]
    q0 = _mul(a, r)
    e = _fma((-q0[0], not q0[1]), b, a)
    q1 = _fma(e, r, q0)
    if q1[0] == 0:                        # the cvt keeps the sign of a zero
        return 0x80 if q1[1] else 0x00
    return nearest_code(q1[0])


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


def test_signed_zero_helpers_follow_ieee():
    """The emulation's zero signs against the host's IEEE doubles, on operands
    (signed zeros and ones) where every product and sum is exact."""
    vals = (0.0, -0.0, 1.0, -1.0)
    for x in vals:
        for y in vals:
            want = x * y
            got = _mul(_val(x), _val(y))
            assert got[0] == Fraction(want) and got[1] == (math.copysign(1.0, want) < 0)
            for z in vals:
                want = x * y + z
                got = _fma(_val(x), _val(y), _val(z))
                assert got[0] == Fraction(want) and got[1] == (math.copysign(1.0, want) < 0), (x, y, z)



def test_ties_stay_exact_with_an_approximate_reciprocal():
    """The refinement q1 = fma(fma(-q0, b, a), r, q0) lands exactly on a
    midpoint M whenever a / b = M, for r up to two ulps off 1/b: q0 is then a
    few ulps from M, the residual b (M - q0) is exact, and the correction's
    error is far below half an ulp.  FP32 values C with 21-24 significant
    bits over maxima that are not powers of two, ties to the even code."""
    n = 0
    # maxima 7 m 2^e with m odd and up to 16 bits make both C = M max / 448
    # and 7/8 C exact FP32 values for every midpoint M
    for amax in (3.25, 98.0 + 2.0 ** -17, 25.5 * (1 + 2.0 ** -21), 7.0 * (1 - 2.0 ** -22),
                 7.0 * 40961 * 2.0 ** -10, 7.0 * 65533 * 2.0 ** -20, 7.0 * 52429 * 2.0 ** 5,
                 7.0 * 3 * 2.0 ** -30, 7.0 * 12345 * 2.0 ** 40):
        amax = float(np.float32(amax))
        for lo, hi in zip(E4M3_VALUES, E4M3_VALUES[1:]):
            x = (lo + hi) / 2 * Fraction(amax) / 448        # a / b is exactly the midpoint
            if f32(x) != x or f32(x * Fraction(7, 8)) != x * Fraction(7, 8):
                continue
            n += 1
            for k in (-2, -1, 1, 2):
                for v in (float(x), -float(x)):
                    assert kernel_code(v, amax, k, exact_a=False) == exact_code(v, amax), (v, amax, k)
    assert n >= 40


def test_bf16_codes_keep_with_an_approximate_reciprocal():
    """For BF16 groups the codes do not depend on the reciprocal's last bits:
    a BF16 quotient that is not a midpoint lies at least 2^-12.8 (relative)
    from every midpoint."""
    rng = np.random.default_rng(5)
    for scale in (1.0, 3e-3, 2.0 ** -110):
        x = _bf16(rng.standard_normal(512) * scale).reshape(4, 128)
        for grp in x:
            amax = float(np.abs(grp).max())
            for v in grp[:64]:
                want = exact_code(float(v), amax)
                for k in (-1, 1):
                    assert kernel_code(float(v), amax, k) == want, (v, amax, k)
