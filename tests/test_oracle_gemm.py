"""Pins of the oracle's group-scaled FP8 linear layer (COAT review, section 三
"Triton优化内核" / linear-layer kernels: output reshaped into 1xG groups whose
max is taken; section 四 table, group scaling).

Pinned by: exact rational arithmetic on small cases (brute force with
fractions), closed forms (an identity-like A copies B^T), the transpose and
scale laws, the quantizer's definition in exact rational arithmetic for the
quantization step, and rejection of NaN codes and ragged groups."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from e4m3_exact import group_codes

E4M3_ONE = 0x38


def _rand_codes(rng, shape, finite_only=True):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E           # no NaN codes
    return c


def _dec(codes):
    return oracle.e4m3_decode_array(np.ascontiguousarray(codes).ravel()).reshape(codes.shape)


def test_exact_against_rational_brute_force():
    rng = np.random.default_rng(0)
    M, N, K, G = 3, 32, 9, 16
    a, b = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sa, sb = 0.375, 1.25
    _, _, c64, c32 = oracle.gemm_fp8_group_quant(a, b, sa, sb, G, want_c=True)
    fa = [[Fraction(float(v)) for v in row] for row in _dec(a)]
    fb = [[Fraction(float(v)) for v in row] for row in _dec(b)]
    for i in range(M):
        for j in range(N):
            exact = Fraction(sa) * Fraction(sb) * sum(x * y for x, y in zip(fa[i], fb[j]))
            assert c64[i, j] == float(exact)                 # exact here (few terms)
            assert c32[i, j] == np.float32(float(exact))


def test_identity_like_a_copies_b():
    rng = np.random.default_rng(1)
    N, K, G = 64, 64, 32
    a = np.zeros((K, K), np.uint8)
    a[np.arange(K), np.arange(K)] = E4M3_ONE                # A = I (as E4M3 ones)
    b = _rand_codes(rng, (N, K))
    _, _, c64, _ = oracle.gemm_fp8_group_quant(a, b, 2.0, 0.5, G, want_c=True)
    assert np.array_equal(c64, _dec(b).T)                    # C = A B^T = B^T


def test_transpose_and_scale_laws():
    rng = np.random.default_rng(2)
    M, N, K, G = 16, 48, 40, 16
    a, b = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    codes, scales, c64, _ = oracle.gemm_fp8_group_quant(a, b, 1.0, 1.0, G, want_c=True)
    _, _, c64t, _ = oracle.gemm_fp8_group_quant(b, a, 1.0, 1.0, G, want_c=True)
    assert np.array_equal(c64, c64t.T)
    codes8, scales8, c64s, _ = oracle.gemm_fp8_group_quant(a, b, 8.0, 0.25, G, want_c=True)
    assert np.array_equal(c64s, 2.0 * c64)                   # power-of-two scales are exact
    assert np.array_equal(codes8, codes)                     # codes are scale invariant
    assert np.array_equal(scales8, 2.0 * scales)


@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_quantization_matches_exact_definition(G):
    """Each 1xG group of the FP32 output C goes through eq. FP8量化 as the
    page defines it: the E4M3 value nearest to the exact quotient
    448 C / max|C| (ties to even, brute force over the format's values with
    fractions), and S = max / 448 rounded once to FP32."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 2 * G, 96
    a, b = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    codes, scales, _, c32 = oracle.gemm_fp8_group_quant(a, b, 0.01, 0.02, G, want_c=True)
    for i in range(M):
        for j in range(N // G):
            grp = c32[i, j * G:(j + 1) * G]
            amax = np.abs(grp).max()
            assert scales[i, j] == np.float32(amax) / np.float32(448.0)
            assert codes[i, j * G:(j + 1) * G].tolist() == group_codes(grp, amax)


def test_matches_float64_matmul_of_decoded_values():
    rng = np.random.default_rng(4)
    M, N, K, G = 20, 64, 256, 64
    a, b = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    _, _, c64, _ = oracle.gemm_fp8_group_quant(a, b, 1.0, 1.0, G, want_c=True)
    ref = _dec(a) @ _dec(b).T
    assert np.allclose(c64, ref, rtol=1e-12, atol=1e-9)


def test_zero_rows_nan_codes_and_ragged_groups():
    rng = np.random.default_rng(5)
    a = _rand_codes(rng, (4, 32))
    a[2] = 0
    b = _rand_codes(rng, (32, 32))
    codes, scales = oracle.gemm_fp8_group_quant(a, b, 1.0, 1.0, 16)
    assert not codes[2].any() and not scales[2].any()
    bad = a.copy()
    bad[0, 0] = 0x7F
    with pytest.raises(oracle.OracleError):
        oracle.gemm_fp8_group_quant(bad, b, 1.0, 1.0, 16)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_fp8_group_quant(a, b[:24], 1.0, 1.0, 16)     # N = 24 not a multiple of G


@pytest.mark.parametrize("G", [16, 128])
def test_negative_scale_flips_signs_and_codes_zero_as_plus(G):
    """The quantizer is odd: with the scale product negated, every nonzero
    output's code is its positive-product code with the sign bit flipped
    (round to nearest even is symmetric), the scales are unchanged, and an
    exact zero output, now -0, still codes 0x00."""
    rng = np.random.default_rng(6)
    M, N, K = 6, 2 * G, 64
    a, b = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    a[0, 1:] = 0                                   # row 0: a[0, 0] * b[j, 0] only
    b[::2, 0] = 0                                  # ... which is zero for every other j
    pc, ps, _, pc32 = oracle.gemm_fp8_group_quant(a, b, 0.5, 2.0, G, want_c=True)
    nc, ns, _, nc32 = oracle.gemm_fp8_group_quant(a, b, -0.5, 2.0, G, want_c=True)
    assert np.array_equal(ps.view(np.uint32), ns.view(np.uint32))
    zero = pc32 == 0
    assert zero.sum() >= N // 2 and np.all(np.signbit(nc32[zero]))
    assert np.all(nc[zero] == 0x00) and np.all(pc[zero] == 0x00)
    nz = ~zero & (pc != 0x00)
    assert np.array_equal(nc[nz], pc[nz] ^ 0x80)
    # values that round to zero keep their sign: code 0x80 under the negative product
    under = ~zero & (pc == 0x00)
    assert np.all(nc[under] == 0x80)
