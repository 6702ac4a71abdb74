"""GPU-vs-oracle comparison for the fused FP8 AdamW step.

Both sides start from the same pre-step state (the oracle's own state, never a
GPU output) and the same gradient.  The only place where the two can differ
before rounding is the dequantization of the stored moments: the oracle
evaluates s * (|c|/448)^(1/k) in double and rounds once; the GPU evaluates it
with FP32 log2/exp2 and is within a few FP32 ulps (bounded per element below,
measured by the dequantize tests).  Everything downstream is judged against
that bound:

* moments: the GPU's dequantized x is within dequant_bound() relative of the
  oracle's (FP32 carries the exponent log2(|c|/448)/k with an absolute error
  proportional to its size);
  m_t = b1*x + (1-b1)*g may cancel, so each m_t (and v_t) is known to lie
  within dq*b*|x| + 2^-22*(b*|x| + (1-b)*|g|) of the oracle's value;
* scale and k: the group max and min-nonzero are bounded by intervals over
  those perturbations; GPU scale and k must lie in the resulting interval,
  widened by REL_TOL (1e-5 relative);
* codes: the GPU code must be the E4M3 rounding of some q in the interval that
  448 (|m_t|/s)^k spans over the box, widened by TIE_TOL for FP32 log/exp
  rounding; and at least 99.99% of codes must be identical (gated when a state
  has >= 10^4 codes); every other code one ordinal away, except where the
  moment itself cancels;
* w: |dw| <= REL_TOL * (|w| + lr*|operands of the update|).

The report also carries the plain numbers (identical-code fraction, max
relative differences) for logging.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_TOL = 1e-5          # spec relative tolerance for scale, k, w
DEQ_A = 3e-7            # GPU dequantization error bound, see dequant_bound()
DEQ_B = 1.5 * np.log(2.0) * 2.0 ** -24
ARITH_REL = 2.0 ** -22  # FP32 rounding of the moment update, relative to operands
TIE_TOL = 1e-4          # relative slack on q for FP32 log2/exp2 near ties
MIN_IDENTICAL = 0.9999  # identical-code fraction, per state per step
RATE_GATE_N = 10_000

L_E = 12.0 + np.log2(7.0)
K_MAX = 16.0

_DEC = None


def _dec_table():
    global _DEC
    if _DEC is None:
        _DEC = oracle.e4m3_decode_array(np.arange(256))
    return _DEC


def canon(codes):
    c = np.asarray(codes, np.uint8)
    return np.where(c == 0x80, 0, c).astype(np.uint8)


def signed_ordinal(codes):
    c = canon(codes).astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def _encode_mag(q):
    """E4M3 magnitude ordinal of q >= 0 (oracle encoder, saturating)."""
    return (oracle.e4m3_encode_array(np.clip(q, 0, 448.0)) & 0x7F).astype(np.int32)


def _group_reduce(a, starts, fn):
    return fn.reduceat(a, starts)


def _k_of(s, mu):
    with np.errstate(divide="ignore", invalid="ignore"):
        lx = np.log2(s / mu)
        k = np.where(lx > 0, np.minimum(K_MAX, L_E / np.where(lx > 0, lx, 1.0)), K_MAX)
    return k


class ParityFailure(AssertionError):
    pass


def dequant_bound(state, G):
    """Relative error bound of the GPU's FP32 dequantization per element.

    The GPU forms x = s * 2^(L(c) * (1/k) + c0) with L(c) = log2(|c|/448)
    correctly rounded to FP32 (a table), 1/k to about half an ulp, one FMA, the
    hardware exp2 and one multiply; c0 = 64 only for groups with k < 0.15
    (compensated in s).  The exponent then carries an absolute error of about
    3 * 2^-24 * |L|/k (table, 1/k, product) plus 2^-24 * |exponent| (FMA
    rounding), which 2^(.) turns into ln2 times that, relative; exp2 and the
    multiply add a few 2^-24.  The bound takes that sum with a 1.5x margin."""
    dec = np.abs(_dec_table()[state.codes])
    grp = np.arange(state.codes.size) // G
    k = state.k[grp].astype(np.float64)
    live = (dec > 0) & (state.scale[grp] > 0) & (k > 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        l = np.abs(np.log2(np.where(live, dec, 448.0) / 448.0))
        rk = np.where(live, 1.0 / np.where(live, k, 1.0), 0.0)
    c0 = np.where(rk > 6.7, 64.0, 0.0)
    a = l * rk
    return DEQ_A + DEQ_B * (3.0 * a + np.abs(c0 - a))


def oracle_reference(w, g_bits, m_state, v_state, G, hp, step):
    """Run the oracle on copies of the pre-step state; returns everything the
    comparison needs (all host numpy arrays)."""
    x_m = oracle.dequantize_expand(m_state, G)
    x_v = oracle.dequantize_expand(v_state, G)
    w_ref = w.copy()
    m_ref, v_ref = m_state.copy(), v_state.copy()
    out = oracle.adamw_fp8_step(w_ref, g_bits, m_ref, v_ref, G, **hp, step=step,
                                want_moments=True, want_q=True)
    return dict(w_prev=w, x_m=x_m, x_v=x_v, g=(g_bits.astype(np.uint32) << 16).view(np.float32),
                dq_m=dequant_bound(m_state, G), dq_v=dequant_bound(v_state, G),
                w=w_ref, m=m_ref, v=v_ref, **out)


def _check_state(name, gpu_codes, gpu_scale, gpu_k, ref_state, mt, oper, delta, G, report,
                 signed):
    n = mt.size
    starts = np.arange(0, n, G)
    amt = np.abs(mt.astype(np.float64))
    lo = np.maximum(0.0, amt - delta)
    hi = amt + delta
    nz = mt != 0
    s_lo = _group_reduce(np.where(nz, lo, 0.0), starts, np.maximum)
    s_hi = _group_reduce(np.where(nz, hi, 0.0), starts, np.maximum)
    big = np.inf
    mu_lo = _group_reduce(np.where(nz, lo, big), starts, np.minimum)
    mu_hi = _group_reduce(np.where(nz, hi, big), starts, np.minimum)
    empty = s_hi == 0

    ref_scale = ref_state.scale.astype(np.float64)
    ref_k = ref_state.k.astype(np.float64)
    gs = gpu_scale.astype(np.float64)
    gk = gpu_k.astype(np.float64)

    # empty groups must match exactly
    bad_empty = empty & ((gs != 0) | (gk != 1))
    bad_nonempty = (~empty) & (gs == 0)
    if bad_empty.any() or bad_nonempty.any():
        raise ParityFailure(f"{name}: empty-group mismatch at groups "
                            f"{np.flatnonzero(bad_empty | bad_nonempty)[:8]}")
    ne = ~empty
    s_ok = (gs >= s_lo * (1 - REL_TOL)) & (gs <= s_hi * (1 + REL_TOL))
    if not s_ok[ne].all():
        i = np.flatnonzero(ne & ~s_ok)[:5]
        raise ParityFailure(f"{name}: scale outside interval at groups {i}: gpu {gs[i]} "
                            f"ref {ref_scale[i]} lo {s_lo[i]} hi {s_hi[i]}")
    mu_lo_pos = np.where(mu_lo > 0, mu_lo, np.minimum(mu_hi, 1e-300))
    k_min = _k_of(s_hi, mu_lo_pos)
    k_max = _k_of(s_lo, mu_hi)
    k_ok = (gk >= k_min * (1 - REL_TOL)) & (gk <= k_max * (1 + REL_TOL))
    if not k_ok[ne].all():
        i = np.flatnonzero(ne & ~k_ok)[:5]
        raise ParityFailure(f"{name}: k outside interval at groups {i}: gpu {gk[i]} "
                            f"ref {ref_k[i]} [{k_min[i]}, {k_max[i]}]")

    # codes
    o_gpu = signed_ordinal(gpu_codes)
    o_ref = signed_ordinal(ref_state.codes)
    diff = o_gpu != o_ref
    grp = np.arange(n) // G
    # the GPU encodes with its own scale and k, which lie inside the interval:
    # bound q over element box x (group scale and k boxes)
    with np.errstate(divide="ignore", invalid="ignore"):
        qa = 448.0 * (lo / s_hi[grp]) ** k_max[grp]
        qb = 448.0 * np.minimum(1.0, hi / np.maximum(s_lo[grp], 1e-300)) ** k_min[grp]
    q_min = np.minimum(qa, qb) * (1 - TIE_TOL)
    q_max = np.minimum(448.0, np.maximum(qa, qb) * (1 + TIE_TOL))
    q_min = np.where(empty[grp], 0.0, q_min)
    q_max = np.where(empty[grp], 0.0, q_max)
    idx = np.flatnonzero(diff)
    mag_gpu = np.abs(o_gpu[idx])
    lo_ord = _encode_mag(q_min[idx])
    hi_ord = _encode_mag(q_max[idx])
    in_box = (mag_gpu >= lo_ord) & (mag_gpu <= hi_ord)
    sign_free = (lo[idx] == 0) | (mag_gpu == 0) | (np.abs(o_ref[idx]) == 0)
    sign_ok = sign_free | (np.sign(o_gpu[idx]) == np.sign(o_ref[idx]))
    if not signed:
        sign_ok &= o_gpu[idx] >= 0
    ok = in_box & sign_ok
    if not ok.all():
        j = idx[~ok][:5]
        raise ParityFailure(
            f"{name}: codes outside their rounding interval at {j}: gpu "
            f"{o_gpu[j]} ref {o_ref[j]} q [{q_min[j]}, {q_max[j]}] m_t {mt[j]}")
    cancel = amt[idx] < 1e-3 * oper[idx]
    far = np.abs(o_gpu[idx] - o_ref[idx]) > 1
    if (far & ~cancel).any():
        j = idx[far & ~cancel][:5]
        raise ParityFailure(f"{name}: codes more than one ordinal apart at {j}")
    ident = 1.0 - idx.size / max(1, n)
    if n >= RATE_GATE_N and ident < MIN_IDENTICAL:
        raise ParityFailure(f"{name}: only {ident:.6f} of codes identical")
    with np.errstate(divide="ignore", invalid="ignore"):
        rs = np.abs(gs - ref_scale) / np.where(ref_scale > 0, ref_scale, 1)
        rk = np.abs(gk - ref_k) / ref_k
    report[name] = dict(n=n, identical=ident, mismatches=int(idx.size),
                        far=int(far.sum()),
                        max_rel_scale=float(rs.max(initial=0)),
                        max_rel_k=float(rk.max(initial=0)),
                        k_groups_within_1e5=float(np.mean(rk <= REL_TOL)) if rk.size else 1.0)


def compare_step(gpu, ref, G, hp, step, report=None):
    """gpu: dict of host arrays w, m_codes, m_scale, m_k, v_codes, v_scale,
    v_k.  ref: output of oracle_reference.  Raises ParityFailure."""
    report = {} if report is None else report
    b1, b2 = hp["beta1"], hp["beta2"]
    g = ref["g"].astype(np.float64)
    xm = b1 * np.abs(ref["x_m"].astype(np.float64))
    xv = b2 * np.abs(ref["x_v"].astype(np.float64))
    oper_m = xm + (1 - b1) * np.abs(g)
    oper_v = xv + (1 - b2) * g * g
    delta_m = ref["dq_m"] * xm + ARITH_REL * oper_m
    delta_v = ref["dq_v"] * xv + ARITH_REL * oper_v
    _check_state("m", gpu["m_codes"], gpu["m_scale"], gpu["m_k"], ref["m"], ref["m_t"],
                 oper_m, delta_m, G, report, signed=True)
    _check_state("v", gpu["v_codes"], gpu["v_scale"], gpu["v_k"], ref["v"], ref["v_t"],
                 oper_v, delta_v, G, report, signed=False)
    # weights
    lr, eps, wd = hp["lr"], hp["eps"], hp["weight_decay"]
    bc1 = 1 - b1 ** step
    bc2 = 1 - b2 ** step
    vt = ref["v_t"].astype(np.float64)
    w_prev = ref["w_prev"].astype(np.float64)
    uscale = abs(lr) * ((oper_m + delta_m / REL_TOL) / bc1 / (np.sqrt(vt / bc2) + eps)
                        + abs(wd) * np.abs(w_prev))
    wtol = REL_TOL * (np.abs(w_prev) + uscale)
    dw = np.abs(gpu["w"].astype(np.float64) - ref["w"].astype(np.float64))
    if not (dw <= wtol).all():
        j = np.flatnonzero(dw > wtol)[:5]
        raise ParityFailure(f"w outside tolerance at {j}: gpu {gpu['w'][j]} ref "
                            f"{ref['w'][j]} tol {wtol[j]}")
    with np.errstate(divide="ignore", invalid="ignore"):
        rw = dw / np.abs(ref["w"].astype(np.float64))
    report["w"] = dict(max_abs=float(dw.max(initial=0)),
                       frac_rel_1e5=float(np.mean(rw <= REL_TOL)) if rw.size else 1.0)
    return report
