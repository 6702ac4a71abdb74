"""Pins of the oracle's OCP E4M3 codec against things other than itself:
the OFP8 specification's printed values (golden fixture), torch's
float8_e4m3fn conversion (a library routine), and a brute-force nearest-value
search with ties to even."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_values.json")


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_spec_values():
    spec = json.load(open(GOLDEN))
    for code, val in spec["values"].items():
        got = oracle.e4m3_decode(int(code, 16))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in spec["nan_codes"]:
        assert math.isnan(oracle.e4m3_decode(int(code, 16)))


def test_decode_all_codes_matches_torch():
    ours = oracle.e4m3_decode_array(np.arange(256))
    ref = torch_decode_all()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_encode_decode_roundtrip_every_finite_code():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        back = oracle.e4m3_encode(oracle.e4m3_decode(c))
        assert back == (0x00 if c == 0x80 else c), hex(c)


def _fp32_sweep():
    # every 61st float32 bit pattern in [0, 448]: ~18.5M values
    bits = np.arange(0, 0x43E00001, 61, dtype=np.uint32)
    return bits.view(np.float32)


def test_encode_matches_torch_cast_dense_sweep():
    x = _fp32_sweep()
    ours = oracle.e4m3_encode_array(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    neg = oracle.e4m3_encode_array(-x[1:].astype(np.float64))
    refn = torch.from_numpy(-x[1:]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign on values that round to zero, as the oracle does
    assert np.array_equal(neg, refn)


def _midpoints():
    vals = np.unique(np.abs(torch_decode_all()[np.isfinite(torch_decode_all())]))
    return (vals[:-1] + vals[1:]) / 2.0, vals


def test_encode_ties_go_to_even_mantissa():
    mids, vals = _midpoints()
    for i, m in enumerate(mids):
        c = oracle.e4m3_encode(m)
        lo, hi = oracle.e4m3_encode(vals[i]), oracle.e4m3_encode(vals[i + 1])
        assert c in (lo, hi)
        assert c & 1 == 0, (m, hex(c))          # even mantissa wins the tie
        # one float32 ulp either side of the tie decides by distance
        below = np.nextafter(np.float32(m), np.float32(0))
        above = np.nextafter(np.float32(m), np.float32(1e9))
        if float(below) < m:
            assert oracle.e4m3_encode(float(below)) == lo
        if float(above) > m:
            assert oracle.e4m3_encode(float(above)) == hi


def test_encode_brute_force_nearest():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(0, 448, 20000),
                        np.exp2(rng.uniform(-12, 8.8, 20000))])
    table = oracle.e4m3_decode_array(np.arange(0x7F))   # 0x00..0x7E
    ours = oracle.e4m3_encode_array(x)
    for xi, c in zip(x, ours):
        d = np.abs(table - xi)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, (xi, c, want)


def test_encode_saturates_and_signs():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.9) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(-0.0) == 0x00
    assert oracle.e4m3_encode(-1e-9) == 0x80     # negative, rounds to zero
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00  # tie between 0 and 2^-9
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert oracle.e4m3_encode(float("nan")) == 0x7F
