"""Pins of the oracle's per-group (1 x G) activation quantizer (COAT review,
section 三 "混合粒度激活量化" and eq. FP8量化; transposed FP8 output of the
non-linear-layer kernels).

Pinned by: the definition itself in exact rational arithmetic (every code the
E4M3 value nearest to 448 x / max, ties to even, checked by brute force over
the format's value set), exact power-of-two groups (closed form), the format's
round-trip error bound, degenerate groups, the transpose relation, the
memory-overhead row the page prints (golden), and the direction of the
mixed-granularity claim (per-group error below per-tensor error on
activations with outliers)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from e4m3_exact import E4M3_VALUES, group_codes, is_midpoint

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "act_group_overhead.json")


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _act(rows, cols, seed, outliers=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g)
    if outliers:  # a few large channels, as in transformer activations
        ch = torch.randint(0, cols, (max(1, cols // 64),), generator=g)
        x[:, ch] *= 50.0
    return x.to(torch.bfloat16)


def _tie_values(amax, limit=24):
    """BF16 values x <= amax whose exact quotient 448 x / amax is an E4M3
    midpoint (exact ties of the rounding), for a group maximum amax."""
    out = []
    for lo, hi in zip(E4M3_VALUES, E4M3_VALUES[1:]):
        x = (lo + hi) / 2 * Fraction(float(amax)) / 448
        xb = torch.tensor(float(x), dtype=torch.float64).to(torch.bfloat16).double().item()
        if Fraction(xb) == x:
            out.append(xb)
    return out[-limit:]


def _check_exact(x, G, codes, scales):
    rows, cols = x.shape
    xf = x.float().numpy()
    for i in range(rows):
        for j in range(cols // G):
            grp = xf[i, j * G:(j + 1) * G]
            amax = np.abs(grp).max()
            if amax == 0:
                assert scales[i, j] == 0 and not codes[i, j * G:(j + 1) * G].any()
                continue
            assert scales[i, j] == np.float32(amax) / np.float32(448.0)     # S rounded once
            want = group_codes(grp, amax)
            got = codes[i, j * G:(j + 1) * G].tolist()
            assert got == want, (i, j, [(a, b, v) for a, b, v in zip(got, want, grp) if a != b][:4])


@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_matches_exact_definition(G):
    """Every code equals the E4M3 value nearest to the exact quotient
    448 x / max (ties to even), computed with fractions; every scale is
    max / 448 rounded once to FP32."""
    rows, cols = 12, 4 * G
    x = _act(rows, cols, G)
    codes, scales, codes_t = oracle.quantize_act(_bits(x), rows, cols, G)
    _check_exact(x, G, codes, scales)
    assert np.array_equal(codes_t, codes.T)


@pytest.mark.parametrize("amax", [3.25, 98.0, 25.5, 12.75, 7.0, 3.0 * 2.0 ** -20, 3.0 * 2.0 ** 99, 5.0 * 2.0 ** -120])
def test_exact_ties_with_any_group_max(amax):
    """Groups whose max is not a power of two, filled with values whose exact
    quotient is an E4M3 midpoint: each goes to the even neighbour, as the
    definition rounds it."""
    G = 32
    ties = _tie_values(amax)
    assert len(ties) >= 4
    vals = np.zeros(G, np.float64)
    vals[0] = amax
    vals[1:1 + len(ties)] = ties
    vals[1::3] *= -1
    x = torch.from_numpy(vals).reshape(1, G).to(torch.bfloat16)
    assert torch.equal(x.double(), torch.from_numpy(vals).reshape(1, G))    # exact in BF16
    codes, scales, _ = oracle.quantize_act(_bits(x), 1, G, G)
    _check_exact(x, G, codes, scales)
    q = [Fraction(448) * Fraction(v) / Fraction(float(amax)) for v in vals[1:1 + len(ties)]]
    assert all(is_midpoint(v) for v in q)
    got = codes[0, 1:1 + len(ties)] & 0x7F
    assert np.all(got % 2 == 0)                     # the even neighbour


def test_fp32_reciprocal_recipe_differs_only_at_exact_ties():
    """The obvious FP32 recipe, RNE(fl(x * fl(448 / max))), agrees with the
    definition everywhere except at exact ties whose max is not a power of
    two (its two roundings push the quotient off the midpoint).  Such ties
    are common in BF16 activations, well above 1e-4 of the codes here, so a
    kernel must decide ties exactly to match the definition."""
    G = 128
    rows, cols = 37, 4 * G
    x = _act(rows, cols, G)
    codes, _, _ = oracle.quantize_act(_bits(x), rows, cols, G, transpose=False)
    xf = x.float().reshape(rows, cols // G, G)
    amax = xf.abs().amax(-1, keepdim=True)
    r = torch.tensor(448.0, dtype=torch.float32) / amax
    fp32 = (xf * r).reshape(rows, cols).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    diff = np.argwhere(codes != fp32)
    assert diff.shape[0] / codes.size > 1e-4
    am = amax.reshape(rows, cols // G).numpy()
    for i, j in diff:
        q = Fraction(448) * Fraction(float(xf.reshape(rows, cols)[i, j])) / Fraction(float(am[i, j // G]))
        assert is_midpoint(q)
        assert abs(int(codes[i, j] & 0x7F) - int(fp32[i, j] & 0x7F)) == 1


def test_power_of_two_group_closed_form():
    G = 16
    m = 3.0 * 2.0 ** -7
    vals = np.array([m * 2.0 ** -j for j in range(G)], np.float32)
    vals[1::2] *= -1
    x = torch.from_numpy(vals).reshape(1, G).to(torch.bfloat16)
    assert np.array_equal(x.float().numpy().ravel(), vals)        # exact in BF16
    codes, scales, _ = oracle.quantize_act(_bits(x), 1, G, G)
    assert scales[0, 0] == np.float32(m / 448.0)
    want = oracle.e4m3_encode_array(448.0 * 2.0 ** -np.arange(G))
    want[1::2] |= 0x80
    assert np.array_equal(codes.ravel(), want)
    assert codes[0, 0] == 0x7E


@pytest.mark.parametrize("G", [16, 128])
def test_round_trip_error_bound_and_degenerate_groups(G):
    rows, cols = 20, 2 * G
    x = _act(rows, cols, 7 * G).float()
    x[3, :G] = 0.0                      # all-zero group
    x[4, G:] = 0.0
    x[4, G + 5] = -1.5                  # single nonzero
    xb = x.to(torch.bfloat16)
    codes, scales, _ = oracle.quantize_act(_bits(xb), rows, cols, G)
    assert scales[3, 0] == 0 and not codes[3, :G].any()
    assert codes[4, G + 5] == 0xFE and np.count_nonzero(codes[4, G:]) == 1
    back = oracle.e4m3_decode_array(codes.ravel()).reshape(rows, cols) * \
        np.repeat(scales.astype(np.float64), G, axis=1)
    xf = xb.float().numpy().astype(np.float64)
    normal = (codes & 0x7F) >= 0x08
    rel = np.abs(back[normal] - xf[normal]) / np.abs(xf[normal])
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
    assert np.array_equal(np.signbit(back[normal]), np.signbit(xf[normal]))
    sub = ((codes & 0x7F) < 0x08) & (xf != 0)
    scale_full = np.repeat(scales.astype(np.float64), G, axis=1)
    assert np.all(np.abs(back[sub] - xf[sub]) <= 2.0 ** -10 * scale_full[sub] * (1 + 1e-6))


def test_memory_overhead_row_of_group_size_table():
    rec = json.load(open(GOLDEN))
    for G, pct in zip(rec["group_size"], rec["memory_overhead_percent"]):
        rows, cols = 8, 4 * G
        x = _act(rows, cols, G)
        _, scales, _ = oracle.quantize_act(_bits(x), rows, cols, G)
        overhead = 100.0 * scales.nbytes / (x.numel() * 2)          # vs BF16 data
        assert overhead == pytest.approx(pct, rel=0.05)


def test_per_group_beats_per_tensor_on_outliers():
    rows, cols = 64, 512
    x = _act(rows, cols, 3)
    bits = _bits(x)
    xf = x.float().numpy().astype(np.float64)

    def mse(codes, scales, G):
        back = oracle.e4m3_decode_array(codes.ravel()).reshape(codes.shape) * \
            np.repeat(scales.astype(np.float64), G, axis=1)
        return np.mean((back.reshape(rows, cols) - xf) ** 2)

    c16, s16, _ = oracle.quantize_act(bits, rows, cols, 16, transpose=False)
    ct, st, _ = oracle.quantize_act(bits, 1, rows * cols, rows * cols, transpose=False)
    per_tensor = mse(ct.reshape(rows, cols), np.full((rows, 1), st[0, 0], np.float32), cols)
    assert mse(c16, s16, 16) < per_tensor


def test_rejects_ragged_group():
    with pytest.raises(oracle.OracleError):
        oracle.quantize_act(np.zeros(30, np.uint16), 1, 30, 16)


@pytest.mark.parametrize("G", [16, 128])
def test_tiny_groups_are_scale_invariant(G):
    """Groups with max |x| < 2^-100 (including BF16 subnormals, where 448/max
    overflows FP32) quantize as FP32 with an unbounded exponent would: their
    codes equal those of the same group times 2^64, a normal-range group; the
    scale is still the FP32 quotient max/448."""
    rows, cols = 12, 2 * G
    base = _act(rows, cols, 11 * G, outliers=False).float().numpy().astype(np.float64)
    factors = np.array([1e-39, 2.0 ** -110, 2.0 ** -101, 3e-38, 1e-32, 2.0 ** -126,
                        1e-40, 2.0 ** -99, 5e-31, 1e-36, 2.0 ** -120, 7e-34])
    tiny = torch.from_numpy(base * factors[:, None]).to(torch.bfloat16)
    big = (tiny.double() * 2.0 ** 64).to(torch.bfloat16)
    assert torch.equal(big.double(), tiny.double() * 2.0 ** 64)       # exact scaling
    assert (tiny.float().abs().amax(1) < 2.0 ** -100).sum() >= 8
    ct, st, _ = oracle.quantize_act(_bits(tiny), rows, cols, G)
    cb, _, _ = oracle.quantize_act(_bits(big), rows, cols, G)
    assert np.array_equal(ct, cb)
    amax = tiny.float().reshape(rows, cols // G, G).abs().amax(-1).numpy()
    assert np.array_equal(st, amax / np.float32(448.0))             # numpy FP32 division
    # subnormal BF16 groups (max below 2^-126) still spread over the code range
    sub = tiny.float().abs().amax(1).numpy() < 2.0 ** -126
    assert sub.any() and (ct[sub] & 0x7F).max() == 0x7E


def test_negative_zero_and_signed_underflow():
    """-0.0 gives code 0x00; a negative value whose quotient is below half the
    smallest E4M3 subnormal rounds to zero and keeps its sign (0x80), however
    small the quotient is."""
    G = 16
    v = np.zeros(G, np.float32)
    v[0] = 1.0
    v[1] = -0.0
    v[2] = -2.0 ** -20            # x * 448 = -4.3e-4 < 2^-10 -> E4M3 -0 (0x80)
    v[3] = 2.0 ** -20
    x = torch.from_numpy(v).reshape(1, G).to(torch.bfloat16)
    c, _, _ = oracle.quantize_act(_bits(x), 1, G, G)
    assert c[0, 0] == 0x7E and c[0, 1] == 0x00 and c[0, 2] == 0x80 and c[0, 3] == 0x00
    w = np.zeros(G, np.float32)
    w[0] = 1e30
    w[1] = -1e-20                 # quotient -4.5e-48, below FP32's range -> 0x80
    w[2] = -1e-5                  # quotient -4.5e-33 -> 0x80
    w[3] = -0.0
    y = torch.from_numpy(w).reshape(1, G).to(torch.bfloat16)
    c, _, _ = oracle.quantize_act(_bits(y), 1, G, G)
    assert c[0, 1] == 0x80 and c[0, 2] == 0x80 and c[0, 3] == 0x00


def test_ties_round_to_even():
    """A group whose max is 448 * 2^e has r = 2^-e exactly, so midpoints
    between neighbouring E4M3 values times 2^e are exact ties: they go to
    the even code (17 -> 16, 19 -> 20, 8.5 -> 8, 9.5 -> 10, 248 -> 256,
    3 * 2^-10 -> 2^-8)."""
    G = 16
    mids = [17.0, 19.0, 8.5, 9.5, 248.0, 3.0 * 2.0 ** -10]
    want = [16.0, 20.0, 8.0, 10.0, 256.0, 2.0 ** -8]
    for e in (-20, 0, 10):
        v = np.zeros(G, np.float64)
        v[0] = 448.0 * 2.0 ** e
        v[1:1 + len(mids)] = np.array(mids) * 2.0 ** e
        x = torch.from_numpy(v).reshape(1, G).to(torch.bfloat16)
        assert torch.equal(x.double(), torch.from_numpy(v).reshape(1, G))
        c, _, _ = oracle.quantize_act(_bits(x), 1, G, G)
        got = oracle.e4m3_decode_array(c.ravel()[1:1 + len(mids)])
        assert np.array_equal(got, want)
