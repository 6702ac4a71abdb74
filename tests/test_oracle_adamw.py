"""Pins of the oracle's AdamW arithmetic (COAT review, section 三 核心公式,
equation "AdamW优化器更新规则") and of the fused FP8 step built on it.

* FP32-state mode against torch.optim.AdamW (a library routine), 10 steps.
* Closed form of the first step from zero moments.
* v >= 0 on every step, including stress gradients.
* The fused step is exactly dequantize -> AdamW -> quantize, group by group.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from adamw_coat_fp8_amd import inputs

HP = inputs.DEFAULT_HPARAMS


def _bits(g_bf16):
    return inputs.bf16_bits(g_bf16).numpy().view(np.uint16)


def _grad(n, std, step, ti=0, kind="gaussian", G=128):
    return inputs.gradient(n, std, step, ti, "cpu", kind=kind, group_size=G)


def test_fp32_mode_matches_torch_adamw():
    """Each of 10 steps starts the oracle from torch's own state (w, m, v), so
    the comparison sees one step's arithmetic; tolerances are relative to the
    operands of each update, which can cancel to near zero."""
    n = 4096
    w0 = inputs.weights(n, 0, "cpu")
    p = torch.nn.Parameter(w0.clone())
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]),
                            eps=HP["eps"], weight_decay=HP["weight_decay"],
                            foreach=False, fused=False)
    m_prev = np.zeros(n, np.float32)
    v_prev = np.zeros(n, np.float32)
    for t in range(1, 11):
        g = _grad(n, 1e-3, t)
        w_prev = p.detach().numpy().copy()
        w, m, v = w_prev.copy(), m_prev.copy(), v_prev.copy()
        p.grad = g.float()
        opt.step()
        oracle.adamw_step_fp32(w, _bits(g), m, v, HP["lr"], HP["beta1"],
                               HP["beta2"], HP["eps"], HP["weight_decay"], t)
        ref = p.detach().numpy()
        st = opt.state[p]
        m_ref, v_ref = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
        # torch forms m by lerp, m + (1-b1)(g-m): both forms can cancel, so
        # m is compared relative to its operands b1*m and (1-b1)*g, and w
        # relative to |w| plus the update built from those operands
        gf = g.float().numpy().astype(np.float64)
        mscale = HP["beta1"] * np.abs(m_prev) + (1 - HP["beta1"]) * np.abs(gf)
        assert np.all(np.abs(m - m_ref) <= 1e-6 * mscale)
        bc1 = 1 - HP["beta1"] ** t
        bc2 = 1 - HP["beta2"] ** t
        uscale = HP["lr"] * (mscale / bc1 / (np.sqrt(v_ref / bc2) + HP["eps"])
                             + HP["weight_decay"] * np.abs(w_prev))
        wscale = np.abs(w_prev) + uscale
        assert np.all(np.abs(w - ref) <= 1e-6 * wscale)
        np.testing.assert_allclose(v, v_ref, rtol=1e-6, atol=0)
        m_prev, v_prev = m_ref.copy(), v_ref.copy()


@pytest.mark.parametrize("fused", [False, True])
def test_first_step_closed_form(fused):
    """From zero moments: m1 = (1-b1) g, v1 = (1-b2) g^2, mhat = g, vhat = g^2,
    so w1 = w0 - lr (g / (|g| + eps) + wd w0)."""
    n = 3000
    w0 = inputs.weights(n, 1, "cpu").numpy()
    g = _grad(n, 1e-3, 1).float().numpy()
    g[::7] = 0.0
    gb = torch.from_numpy(g).to(torch.bfloat16)
    g = gb.float().numpy().astype(np.float64)
    w = w0.copy()
    if fused:
        m = oracle.QuantizedState.zeros(n, 128)
        v = oracle.QuantizedState.zeros(n, 128)
        out = oracle.adamw_fp8_step(w, _bits(gb), m, v, 128, **HP, step=1,
                                    want_moments=True)
        mt, vt = out["m_t"], out["v_t"]
    else:
        mt = np.zeros(n, np.float32)
        vt = np.zeros(n, np.float32)
        oracle.adamw_step_fp32(w, _bits(gb), mt, vt, **HP, step=1)
    b1, b2 = np.float32(HP["beta1"]), np.float32(HP["beta2"])
    assert np.array_equal(mt, (np.float32(1) - b1) * g.astype(np.float32))
    assert np.array_equal(vt, (np.float32(1) - b2) * (g * g).astype(np.float32))
    lr, eps, wd = HP["lr"], HP["eps"], HP["weight_decay"]
    w0d = w0.astype(np.float64)
    u = g / (np.abs(g) + eps) + wd * w0d
    expect = w0d - lr * u
    # FP32 rounding, relative to the operands |w0| and lr*|u|
    assert np.all(np.abs(w - expect) <= 2e-6 * (np.abs(w0d) + lr * np.abs(u)))
    z = g == 0
    np.testing.assert_allclose(w[z], w0d[z] * (1 - lr * wd), rtol=1e-6)


@pytest.mark.parametrize("G", [16, 128])
def test_v_nonnegative_and_fused_composition(G):
    """Fused step == (dequantize, FP32 AdamW, quantize) and v codes never carry
    a sign, on stress gradients over several steps, with a ragged tail."""
    n = 5 * G * 7 + 37
    w = inputs.weights(n, 2, "cpu").numpy().copy()
    m = oracle.QuantizedState.zeros(n, G)
    v = oracle.QuantizedState.zeros(n, G)
    for t in range(1, 6):
        gb = _grad(n, 1e-3, t, kind="stress", G=G)
        # composition from the same pre-step state
        w2 = w.copy()
        mx = oracle.dequantize_expand(m, G)
        vx = oracle.dequantize_expand(v, G)
        oracle.adamw_step_fp32(w2, _bits(gb), mx, vx, **HP, step=t)
        mq = oracle.expand_quantize(mx, G)
        vq = oracle.expand_quantize(vx, G)
        oracle.adamw_fp8_step(w, _bits(gb), m, v, G, **HP, step=t)
        assert np.array_equal(w, w2)
        for a, b in ((m, mq), (v, vq)):
            assert np.array_equal(a.codes, b.codes)
            assert np.array_equal(a.scale, b.scale)
            assert np.array_equal(a.k, b.k)
        assert not np.any(v.codes & 0x80)
        assert np.all(v.scale >= 0) and np.all(m.scale >= 0)
        assert np.all((m.k > 0) & (m.k <= 16)) and np.all((v.k > 0) & (v.k <= 16))


def test_fused_tracks_fp32_adamw():
    """Quantized moments move the weights almost as FP32 moments do: after 10
    steps the difference stays a small fraction of the total update."""
    n, G = 128 * 64, 128
    w0 = inputs.weights(n, 3, "cpu").numpy()
    wq, wf = w0.copy(), w0.copy()
    m = oracle.QuantizedState.zeros(n, G)
    v = oracle.QuantizedState.zeros(n, G)
    mf = np.zeros(n, np.float32)
    vf = np.zeros(n, np.float32)
    for t in range(1, 11):
        gb = _bits(_grad(n, 1e-3, t))
        oracle.adamw_fp8_step(wq, gb, m, v, G, **HP, step=t)
        oracle.adamw_step_fp32(wf, gb, mf, vf, **HP, step=t)
    upd = np.abs(wf - w0)
    assert np.median(np.abs(wq - wf) / upd) < 0.05


def test_invalid_arguments_rejected():
    n = 16
    w = np.zeros(n, np.float32)
    g = np.zeros(n, np.uint16)
    m = oracle.QuantizedState.zeros(n, 16)
    v = oracle.QuantizedState.zeros(n, 16)
    for bad in (dict(step=0), dict(beta1=1.0), dict(beta2=-0.1), dict(lr=math.inf)):
        hp = dict(HP, step=1)
        hp.update(bad)
        with pytest.raises(oracle.OracleError):
            oracle.adamw_fp8_step(w, g, m, v, 16, **hp)
    m.scale[0] = 1.0
    m.k[0] = 0.0                       # nonempty group with k = 0: bad state
    with pytest.raises(oracle.OracleError):
        oracle.adamw_fp8_step(w, g, m, v, 16, **HP, step=1)
