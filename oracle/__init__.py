"""Python access to the CPU oracle of COAT's FP8 AdamW step.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline call this; the product path never does.  Arrays are numpy arrays on
the host; every function copies nothing it does not have to and works in place
where the C function does.  The arithmetic lives in ``coat_oracle.c``; this
module only marshals arguments.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.coat_oracle_e4m3_decode.restype = ctypes.c_double
        lib.coat_oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.coat_oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.coat_oracle_e4m3_encode.argtypes = [ctypes.c_double]
        _f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
        lib.coat_oracle_e4m3_encode_array.restype = None
        lib.coat_oracle_e4m3_encode_array.argtypes = [_f64p, ctypes.c_int64, _u8p]
        lib.coat_oracle_e4m3_decode_array.restype = None
        lib.coat_oracle_e4m3_decode_array.argtypes = [_u8p, ctypes.c_int64, _f64p]
        lib.coat_oracle_expand_quantize.restype = ctypes.c_int
        lib.coat_oracle_expand_quantize.argtypes = [
            _f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            _u8p, _f32p, _f32p, _vp]
        lib.coat_oracle_dequantize_expand.restype = ctypes.c_int
        lib.coat_oracle_dequantize_expand.argtypes = [
            _u8p, _f32p, _f32p, ctypes.c_int64, ctypes.c_int32, _f32p]
        lib.coat_oracle_adamw_step_fp32.restype = ctypes.c_int
        lib.coat_oracle_adamw_step_fp32.argtypes = [
            _f32p, _u16p, _f32p, _f32p, ctypes.c_int64,
            ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
            ctypes.c_float, ctypes.c_int64]
        lib.coat_oracle_adamw_fp8_step.restype = ctypes.c_int
        lib.coat_oracle_adamw_fp8_step.argtypes = [
            _f32p, _u16p, _u8p, _f32p, _f32p, _u8p, _f32p, _f32p,
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
            ctypes.c_float, ctypes.c_int64, _vp, _vp, _vp, _vp]
        lib.coat_oracle_quantize_act.restype = ctypes.c_int
        lib.coat_oracle_quantize_act.argtypes = [
            _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _u8p, _f32p, _vp]
        lib.coat_oracle_gemm_fp8_group_quant.restype = ctypes.c_int
        lib.coat_oracle_gemm_fp8_group_quant.argtypes = [
            _u8p, _u8p, ctypes.c_float, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int32, _u8p, _f32p, _vp, _vp]
        _LIB = lib
    return _LIB


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_groups(n, group_size):
    return (n + group_size - 1) // group_size


def e4m3_decode(code):
    return _lib().coat_oracle_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(x):
    return _lib().coat_oracle_e4m3_encode(float(x))


def e4m3_decode_array(codes):
    codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    out = np.zeros(codes.size, np.float64)
    _lib().coat_oracle_e4m3_decode_array(codes, codes.size, out)
    return out


def e4m3_encode_array(x):
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    out = np.zeros(x.size, np.uint8)
    _lib().coat_oracle_e4m3_encode_array(x, x.size, out)
    return out


class QuantizedState:
    """One FP8 moment: codes[n] (uint8), scale[ng] and k[ng] (float32)."""

    def __init__(self, codes, scale, k):
        self.codes = codes
        self.scale = scale
        self.k = k

    @classmethod
    def zeros(cls, n, group_size):
        ng = num_groups(n, group_size)
        return cls(np.zeros(n, np.uint8), np.zeros(ng, np.float32),
                   np.zeros(ng, np.float32))

    def copy(self):
        return QuantizedState(self.codes.copy(), self.scale.copy(), self.k.copy())


def expand_quantize(x, group_size, dre=True, want_q=False):
    """Per-group expansion + E4M3 quantization of an FP32 vector."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    st = QuantizedState.zeros(x.size, group_size)
    q = np.zeros(x.size, np.float64) if want_q else None
    _check(_lib().coat_oracle_expand_quantize(
        x, x.size, group_size, int(bool(dre)), st.codes, st.scale, st.k, _ptr(q)),
        "expand_quantize")
    return (st, q) if want_q else st


def dequantize_expand(state, group_size):
    n = state.codes.size
    x = np.zeros(n, np.float32)
    _check(_lib().coat_oracle_dequantize_expand(
        state.codes, state.scale, state.k, n, group_size, x), "dequantize_expand")
    return x


def adamw_step_fp32(w, g_bf16, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """In place on w, m, v (float32 arrays); g_bf16 is uint16 bit patterns."""
    _check(_lib().coat_oracle_adamw_step_fp32(
        w, g_bf16, m, v, w.size, lr, beta1, beta2, eps, weight_decay, step),
        "adamw_step_fp32")


def adamw_fp8_step(w, g_bf16, m, v, group_size, lr, beta1, beta2, eps,
                   weight_decay, step, dre=True, want_moments=False, want_q=False):
    """Fused FP8 step, in place on w (float32) and the two QuantizedStates.

    Returns a dict with the optional diagnostics: the FP32 moments before
    re-quantization ("m_t", "v_t") and the unrounded code magnitudes
    ("q_m", "q_v")."""
    n = w.size
    assert g_bf16.size == n and m.codes.size == n and v.codes.size == n
    out = {}
    if want_moments:
        out["m_t"] = np.zeros(n, np.float32)
        out["v_t"] = np.zeros(n, np.float32)
    if want_q:
        out["q_m"] = np.zeros(n, np.float64)
        out["q_v"] = np.zeros(n, np.float64)
    _check(_lib().coat_oracle_adamw_fp8_step(
        w, g_bf16, m.codes, m.scale, m.k, v.codes, v.scale, v.k, n, group_size,
        int(bool(dre)), lr, beta1, beta2, eps, weight_decay, step,
        _ptr(out.get("m_t")), _ptr(out.get("v_t")),
        _ptr(out.get("q_m")), _ptr(out.get("q_v"))), "adamw_fp8_step")
    return out


def quantize_act(x_bf16_bits, rows, cols, group_size, transpose=True):
    """Per-group (1 x group_size) E4M3 quantization of a row-major BF16 matrix
    given as uint16 bit patterns.  Returns (codes[rows, cols],
    scales[rows, cols // group_size], codes_t[cols, rows] or None)."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16).ravel()
    assert x.size == rows * cols
    codes = np.zeros(rows * cols, np.uint8)
    scales = np.zeros(rows * (cols // group_size), np.float32)
    codes_t = np.zeros(rows * cols, np.uint8) if transpose else None
    _check(_lib().coat_oracle_quantize_act(x, rows, cols, group_size, codes, scales,
                                           _ptr(codes_t)), "quantize_act")
    return (codes.reshape(rows, cols), scales.reshape(rows, cols // group_size),
            None if codes_t is None else codes_t.reshape(cols, rows))


def gemm_fp8_group_quant(a_codes, b_codes, a_scale, b_scale, group_size, want_c=False):
    """Group-scaled FP8 linear layer: C = a_scale * b_scale * A B^T with A
    (M x K) and B (N x K) given as E4M3 codes, quantized per 1 x group_size
    group of each row of C.  Returns (codes[M, N], scales[M, N // G]) and,
    with want_c, also (c_exact float64[M, N], c_f32 float32[M, N])."""
    a = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b = np.ascontiguousarray(b_codes, dtype=np.uint8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    codes = np.zeros((M, N), np.uint8)
    scales = np.zeros((M, N // group_size if group_size else 0), np.float32)
    c64 = np.zeros((M, N), np.float64) if want_c else None
    c32 = np.zeros((M, N), np.float32) if want_c else None
    _check(_lib().coat_oracle_gemm_fp8_group_quant(
        a, b, a_scale, b_scale, M, N, K, group_size, codes, scales, _ptr(c64), _ptr(c32)),
        "gemm_fp8_group_quant")
    if want_c:
        return codes, scales, c64, c32
    return codes, scales
