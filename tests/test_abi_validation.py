"""Validation paths of every C-ABI entry point, on the CPU: each rejected
argument returns its status before any HIP call, so these run without a GPU.
The pointers passed are never dereferenced (validation fails first); host
structs (tensor list, hyperparameters) are real."""
import ctypes

import pytest

from test_abi_exports import _ensure_built

OK, NULLP, INVAL, GSIZE, MISAL = 0, 1, 2, 3, 4
A16 = 0x10000          # fake, 16-byte aligned device addresses (never touched)
B16 = 0x20000


@pytest.fixture(scope="module")
def lib():
    from adamw_coat_fp8_amd import coat
    return coat


def _hp(coat, **kw):
    d = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1, group_size=128)
    d.update(kw)
    return coat.AdamWHParams(d["lr"], d["beta1"], d["beta2"], d["eps"], d["weight_decay"],
                             d["step"], d["group_size"])


def _tensor(coat, n=4096, **kw):
    f = dict(w=A16, g=A16 + 0x1000, mc=A16 + 0x2000, ms=A16 + 0x3000, mk=A16 + 0x4000,
             vc=A16 + 0x5000, vs=A16 + 0x6000, vk=A16 + 0x7000)
    f.update(kw)
    return coat.AdamWTensor(f["w"], f["g"], coat.FP8State(f["mc"], f["ms"], f["mk"]),
                            coat.FP8State(f["vc"], f["vs"], f["vk"]), n)


def _step(coat, tensors, hp, num=None):
    arr = (coat.AdamWTensor * max(1, len(tensors)))(*tensors)
    return coat.lib.coat_adamw_fp8_step(ctypes.addressof(arr),
                                        len(tensors) if num is None else num,
                                        ctypes.byref(hp) if hp is not None else None, None)


def test_step_rejections(lib):
    coat = lib
    nan = float("nan")
    cases = [
        ([_tensor(coat)], None, NULLP),
        ([_tensor(coat)], _hp(coat, group_size=48), GSIZE),
        ([_tensor(coat)], _hp(coat, step=0), INVAL),
        ([_tensor(coat)], _hp(coat, beta1=1.0), INVAL),
        ([_tensor(coat)], _hp(coat, beta2=-0.1), INVAL),
        ([_tensor(coat)], _hp(coat, lr=nan), INVAL),
        ([_tensor(coat)], _hp(coat, eps=float("inf")), INVAL),
        ([_tensor(coat)], _hp(coat, weight_decay=nan), INVAL),
        ([_tensor(coat, n=-1)], _hp(coat), INVAL),
        ([_tensor(coat, w=0)], _hp(coat), NULLP),
        ([_tensor(coat, vk=0)], _hp(coat), NULLP),
        ([_tensor(coat, w=A16 + 4)], _hp(coat), MISAL),
        ([_tensor(coat, mc=A16 + 0x2001)], _hp(coat), MISAL),
        ([_tensor(coat, ms=A16 + 0x3002)], _hp(coat), MISAL),
        # the bad tensor is last: nothing may be launched for the good ones
        ([_tensor(coat), _tensor(coat, g=A16 + 2)], _hp(coat), MISAL),
    ]
    for tensors, hp, want in cases:
        assert _step(coat, tensors, hp) == want
    assert _step(coat, [_tensor(coat)], _hp(coat), num=-1) == INVAL
    assert coat.lib.coat_adamw_fp8_step(None, 3, ctypes.byref(_hp(coat)), None) == NULLP
    # empty list, or only empty tensors: success without a launch
    assert _step(coat, [], _hp(coat), num=0) == OK
    assert _step(coat, [_tensor(coat, n=0, w=0, g=0, mc=0, ms=0, mk=0, vc=0, vs=0, vk=0)],
                 _hp(coat)) == OK


def test_codec_rejections(lib):
    coat = lib
    L = coat.lib
    st = coat.FP8State(A16, B16, B16 + 0x100)
    assert L.coat_fp8_expand_quantize(A16, -1, 128, st, None) == INVAL
    assert L.coat_fp8_expand_quantize(A16, 100, 100, st, None) == GSIZE
    assert L.coat_fp8_expand_quantize(A16, 0, 128, coat.FP8State(0, 0, 0), None) == OK
    assert L.coat_fp8_expand_quantize(None, 100, 128, st, None) == NULLP
    assert L.coat_fp8_expand_quantize(A16, 100, 128, coat.FP8State(A16, 0, B16), None) == NULLP
    assert L.coat_fp8_expand_quantize(A16 + 8, 100, 128, st, None) == MISAL
    assert L.coat_fp8_expand_quantize(A16, 100, 128, coat.FP8State(A16 + 1, B16, B16), None) == MISAL
    assert L.coat_fp8_dequantize_expand(A16, B16, B16, -5, 64, A16, None) == INVAL
    assert L.coat_fp8_dequantize_expand(A16, B16, B16, 5, 8, A16, None) == GSIZE
    assert L.coat_fp8_dequantize_expand(None, B16, B16, 5, 64, A16, None) == NULLP
    assert L.coat_fp8_dequantize_expand(A16, B16, B16, 5, 64, A16 + 4, None) == MISAL
    assert L.coat_fp8_dequantize_expand(A16, B16 + 2, B16, 5, 64, A16, None) == MISAL
    assert L.coat_e4m3_encode(A16, -1, A16, None) == INVAL
    assert L.coat_e4m3_encode(None, 4, A16, None) == NULLP
    assert L.coat_e4m3_encode(A16, 4, A16 + 3, None) == MISAL
    assert L.coat_e4m3_decode(A16, 0, None, None) == OK
    assert L.coat_e4m3_decode(A16 + 1, 4, A16, None) == MISAL


def test_act_rejections(lib):
    L = lib.lib
    q = L.coat_fp8_quantize_act
    assert q(A16, -1, 128, 128, A16, B16, A16, None) == INVAL
    assert q(A16, 4, 100, 16, A16, B16, A16, None) == INVAL        # cols % G
    assert q(A16, 4, 128, 12, A16, B16, A16, None) == GSIZE
    assert q(None, 0, 128, 16, None, None, None, None) == OK
    assert q(A16, 4, 128, 16, None, B16, A16, None) == NULLP
    assert q(A16, 4, 128, 16, A16, None, A16, None) == NULLP
    assert q(A16 + 2, 4, 128, 16, A16, B16, A16, None) == MISAL
    assert q(A16, 4, 128, 16, A16, B16 + 1, A16, None) == MISAL
    assert q(A16, 4, 128, 16, A16, B16, A16 + 8, None) == MISAL
    assert q(A16, 1 << 40, 1 << 24, 16, A16, B16, A16, None) == INVAL   # grid too large


def test_status_strings(lib):
    for s in range(6):
        assert lib.status_string(s).startswith("COAT_")
    assert "unknown" in lib.status_string(99)
    assert lib.lib.coat_last_hip_error() is not None
