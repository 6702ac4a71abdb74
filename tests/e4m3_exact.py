"""Exact rational reference for the absmax E4M3 quantizer of one group, written
from the format and the equation alone (no oracle code): COAT review, section
三 核心公式, eq. FP8量化 (S = max|X| / Δmax, X_FP8 = round(X / S)), with the
OFP8 E4M3 value set (max 448) and rounding to nearest, ties to the even code.

Everything is a fractions.Fraction, so a tie is a tie: used by the pins to
check the oracle's quantizer against the definition on small inputs."""
from fractions import Fraction

# OFP8 E4M3: exponent field e (bias 7), 3 mantissa bits f; e = 0 is subnormal
# f * 2^-9; S.1111.111 is NaN, so the largest code is 0x7E = 448.
E4M3_VALUES = []
for _code in range(0x7F):
    _e, _f = _code >> 3, _code & 7
    E4M3_VALUES.append(Fraction(_f, 512) if _e == 0 else Fraction(8 + _f, 8) * Fraction(2) ** (_e - 7))
assert E4M3_VALUES[-1] == 448


def nearest_code(q: Fraction) -> int:
    """E4M3 code of the real q (|q| <= 448): the nearest value by exact
    comparison, ties to the code with an even mantissa; sign bit from q."""
    mag = abs(q)
    assert mag <= 448
    best, best_d = 0, None
    for c, v in enumerate(E4M3_VALUES):
        d = abs(v - mag)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if q < 0 else 0)


def group_codes(xs, amax) -> list:
    """Codes of one group of floats with group max amax > 0: the code of
    x / S with S = amax / 448, computed exactly."""
    m = Fraction(float(amax))
    return [nearest_code(Fraction(448) * Fraction(float(x)) / m) for x in xs]


def is_midpoint(q: Fraction) -> bool:
    """True when |q| lies exactly half way between two neighbouring E4M3 values."""
    mag = abs(q)
    return any(mag == (a + b) / 2 for a, b in zip(E4M3_VALUES, E4M3_VALUES[1:]))
