"""Boundary behaviour of the C ABI on the GPU: every validation error is
returned before anything is enqueued (buffers compared before/after), n = 0 is
a no-op, and the error strings exist.  No call here makes a kernel fault: the
invalid cases are all rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

from adamw_coat_fp8_amd import inputs
from gpu_util import DEV, lib, require_gpu

pytestmark = pytest.mark.gpu


def setup_module():
    require_gpu()


def _slot(n, G):
    coat = lib()
    w = inputs.weights(n, 0, DEV)
    g = inputs.gradient(n, 1e-3, 1, 0, DEV)
    return coat.ParamSlot(w, g, coat.QuantState.zeros(n, G, DEV), coat.QuantState.zeros(n, G, DEV))


def _snapshot(s):
    return [t.clone() for t in (s.w, s.m.codes, s.m.scale, s.m.k, s.v.codes, s.v.scale, s.v.k)]


def _same(s, snap):
    now = (s.w, s.m.codes, s.m.scale, s.m.k, s.v.codes, s.v.scale, s.v.k)
    return all(torch.equal(a, b) for a, b in zip(now, snap))


def _call(arr, num, hp):
    coat = lib()
    ptr = ctypes.addressof(arr) if arr is not None else None
    st = coat.adamw_fp8_step_raw(ptr, num, hp)
    torch.cuda.synchronize()
    return st


def test_validation_errors_touch_nothing():
    coat = lib()
    G = 128
    s = _slot(4096, G)
    snap = _snapshot(s)
    good = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1,
                group_size=G)

    def hp(**kw):
        d = dict(good)
        d.update(kw)
        return coat.AdamWHParams(d["lr"], d["beta1"], d["beta2"], d["eps"],
                                 d["weight_decay"], d["step"], d["group_size"])

    arr = (coat.AdamWTensor * 1)(s.as_c())
    cases = [
        (dict(group_size=100), coat.COAT_ERR_GROUP_SIZE),
        (dict(group_size=256), coat.COAT_ERR_GROUP_SIZE),
        (dict(step=0), coat.COAT_ERR_INVALID_VALUE),
        (dict(beta1=1.0), coat.COAT_ERR_INVALID_VALUE),
        (dict(beta2=-0.5), coat.COAT_ERR_INVALID_VALUE),
        (dict(lr=float("nan")), coat.COAT_ERR_INVALID_VALUE),
        (dict(eps=float("inf")), coat.COAT_ERR_INVALID_VALUE),
    ]
    for kw, want in cases:
        assert _call(arr, 1, hp(**kw)) == want, kw
    assert _call(arr, -1, hp()) == coat.COAT_ERR_INVALID_VALUE
    assert _call(None, 1, hp()) == coat.COAT_ERR_NULL_POINTER
    assert coat.lib.coat_adamw_fp8_step(ctypes.addressof(arr), 1, None,
                                        torch.cuda.current_stream().cuda_stream) == \
        coat.COAT_ERR_NULL_POINTER
    # per-tensor problems; a good tensor first, so a partial launch would show
    good_c = s.as_c()
    for field, val, want in [("n", -5, coat.COAT_ERR_INVALID_VALUE),
                             ("w", None, coat.COAT_ERR_NULL_POINTER),
                             ("grad", None, coat.COAT_ERR_NULL_POINTER),
                             ("w", s.w.data_ptr() + 4, coat.COAT_ERR_MISALIGNED),
                             ("grad", s.grad.data_ptr() + 2, coat.COAT_ERR_MISALIGNED)]:
        bad = s.as_c()
        setattr(bad, field, val)
        arr2 = (coat.AdamWTensor * 2)(good_c, bad)
        assert _call(arr2, 2, hp()) == want, field
    for st_name in ("m", "v"):
        for f, val, want in [("codes", None, coat.COAT_ERR_NULL_POINTER),
                             ("scale", None, coat.COAT_ERR_NULL_POINTER),
                             ("codes", s.m.codes.data_ptr() + 1, coat.COAT_ERR_MISALIGNED),
                             ("k", s.m.k.data_ptr() + 2, coat.COAT_ERR_MISALIGNED)]:
            bad = s.as_c()
            setattr(getattr(bad, st_name), f, val)
            arr2 = (coat.AdamWTensor * 2)(good_c, bad)
            assert _call(arr2, 2, hp()) == want, (st_name, f)
    assert _same(s, snap)
    # n = 0 tensors (with NULL pointers) and an empty list are no-ops
    empty = coat.AdamWTensor(None, None, coat.FP8State(), coat.FP8State(), 0)
    arr3 = (coat.AdamWTensor * 1)(empty)
    assert _call(arr3, 1, hp()) == coat.COAT_OK
    assert _call(None, 0, hp()) == coat.COAT_OK
    assert _same(s, snap)
    # and a valid call does change the state
    assert _call(arr, 1, hp()) == coat.COAT_OK
    assert not _same(s, snap)


def test_codec_entry_points_validate():
    coat = lib()
    x = torch.zeros(64, device=DEV)
    st = coat.QuantState.zeros(64, 16, DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert coat.lib.coat_fp8_expand_quantize(x.data_ptr(), 64, 48, st.as_c(), s) == \
        coat.COAT_ERR_GROUP_SIZE
    assert coat.lib.coat_fp8_expand_quantize(x.data_ptr(), -1, 16, st.as_c(), s) == \
        coat.COAT_ERR_INVALID_VALUE
    assert coat.lib.coat_fp8_expand_quantize(None, 64, 16, st.as_c(), s) == \
        coat.COAT_ERR_NULL_POINTER
    assert coat.lib.coat_fp8_expand_quantize(x.data_ptr() + 4, 60, 16, st.as_c(), s) == \
        coat.COAT_ERR_MISALIGNED
    assert coat.lib.coat_fp8_dequantize_expand(st.codes.data_ptr(), st.scale.data_ptr(),
                                               None, 64, 16, x.data_ptr(), s) == \
        coat.COAT_ERR_NULL_POINTER
    assert coat.lib.coat_fp8_dequantize_expand(None, None, None, 0, 16, None, s) == coat.COAT_OK
    assert coat.lib.coat_e4m3_encode(x.data_ptr(), -3, st.codes.data_ptr(), s) == \
        coat.COAT_ERR_INVALID_VALUE
    assert coat.lib.coat_e4m3_decode(st.codes.data_ptr() + 1, 8, x.data_ptr(), s) == \
        coat.COAT_ERR_MISALIGNED
    torch.cuda.synchronize()
    assert not st.codes.any() and not x.any()
