"""GPU-vs-oracle comparison for the fused FP8 AdamW step.

Both sides start from the same pre-step state (the oracle's own state, never a
GPU output) and the same gradient.  The gates are the stated tolerances of the
method, applied per state (m, v) and per step:

* codes: after folding 0x80 onto 0x00, at least 99.99% of the codes of a
  state are identical to the oracle's (gated over every code of one library
  call: gate_identical); every other code is exactly one ordinal away in the
  signed ordering (same sign, or one side zero);
* scale: |scale_gpu - scale_ref| <= 1e-5 scale_ref in every group, and an
  empty group (scale 0) must be empty on both sides;
* k: |k_gpu - k_ref| <= 1e-5 k_ref in every group;
* w: |w_gpu - w_ref| <= 1e-5 |w_ref| + 1e-5 lr (|b1 m| + |(1-b1) g|) / bc1 /
  (sqrt(vh) + eps): one part in 1e5 of the new weight, with an absolute floor
  of one part in 1e5 of the gradient step formed from the magnitudes of the
  first moment's two terms (reading: where the decayed weight and the step
  cancel, or b1 m and (1-b1) g cancel inside the step, a relative error of the
  result is ill-conditioned, and the bound falls back to 1e-5 relative to the
  operands of the update).

The interval model of the GPU's FP32 dequantization (dequant_bound and the
boxes it induces on m_t, v_t, the group statistics and q) is kept as a
printed diagnostic: it says whether a difference is explained by the FP32
evaluation of s * (|c|/448)^(1/k), but it gates nothing.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_TOL = 1e-5          # stated relative tolerance for scale, k and w
MIN_IDENTICAL = 0.9999  # identical-code fraction, per state per step
DEQ_A = 3e-7            # GPU dequantization error bound, see dequant_bound()
DEQ_B = 1.5 * np.log(2.0) * 2.0 ** -24
ARITH_REL = 2.0 ** -22  # FP32 rounding of the moment update, relative to operands
TIE_TOL = 1e-4          # relative slack on q for FP32 log2/exp2 near ties (diagnostic)

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


def _k_of(s, mu):
    with np.errstate(divide="ignore", invalid="ignore"):
        lx = np.log2(s / mu)
        k = np.where(lx > 0, np.minimum(K_MAX, L_E / np.where(lx > 0, lx, 1.0)), K_MAX)
    return k


class ParityFailure(AssertionError):
    pass


def dequant_bound(state, G):
    """Relative error bound of the GPU's FP32 dequantization per element
    (diagnostic model, and the gate of the stand-alone dequantize tests).

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


def _interval_diagnostic(gs, gk, gpu_codes, mt, delta, G):
    """Count groups and codes that the FP32-dequantization box does not
    explain (printed, not gated)."""
    n = mt.size
    starts = np.arange(0, n, G)
    amt = np.abs(mt.astype(np.float64))
    lo = np.maximum(0.0, amt - delta)
    hi = amt + delta
    nz = mt != 0
    s_lo = np.maximum.reduceat(np.where(nz, lo, 0.0), starts)
    s_hi = np.maximum.reduceat(np.where(nz, hi, 0.0), starts)
    mu_lo = np.minimum.reduceat(np.where(nz, lo, np.inf), starts)
    mu_hi = np.minimum.reduceat(np.where(nz, hi, np.inf), starts)
    ne = s_hi > 0
    k_min = _k_of(s_hi, np.where(mu_lo > 0, mu_lo, np.minimum(mu_hi, 1e-300)))
    k_max = _k_of(s_lo, mu_hi)
    s_out = ne & ((gs < s_lo * (1 - REL_TOL)) | (gs > s_hi * (1 + REL_TOL)))
    k_out = ne & ((gk < k_min * (1 - REL_TOL)) | (gk > k_max * (1 + REL_TOL)))
    grp = np.arange(n) // G
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        qa = 448.0 * (lo / s_hi[grp]) ** k_max[grp]
        qb = 448.0 * np.minimum(1.0, hi / np.maximum(s_lo[grp], 1e-300)) ** k_min[grp]
    q_min = np.where(ne[grp], np.minimum(qa, qb) * (1 - TIE_TOL), 0.0)
    q_max = np.where(ne[grp], np.minimum(448.0, np.maximum(qa, qb) * (1 + TIE_TOL)), 0.0)
    mag = np.abs(signed_ordinal(gpu_codes))
    c_out = (mag < _encode_mag(q_min)) | (mag > _encode_mag(q_max))
    return int(s_out.sum()), int(k_out.sum()), int(c_out.sum())


def _check_state(name, gpu_codes, gpu_scale, gpu_k, ref_state, mt, delta, G, report, signed):
    n = mt.size
    ref_scale = ref_state.scale.astype(np.float64)
    ref_k = ref_state.k.astype(np.float64)
    gs = gpu_scale.astype(np.float64)
    gk = gpu_k.astype(np.float64)

    # scale: empty groups on both sides at once, 1e-5 relative elsewhere
    empty = ref_scale == 0
    bad_empty = (empty != (gs == 0)) | (empty & (gk != 1.0))
    if bad_empty.any():
        i = np.flatnonzero(bad_empty)[:8]
        raise ParityFailure(f"{name}: empty-group mismatch at groups {i}: gpu scale {gs[i]} "
                            f"k {gk[i]}, oracle scale {ref_scale[i]} k {ref_k[i]}")
    ne = ~empty
    with np.errstate(divide="ignore", invalid="ignore"):
        rs = np.where(ne, np.abs(gs - ref_scale) / np.where(ne, ref_scale, 1.0), 0.0)
        rk = np.abs(gk - ref_k) / ref_k
    if (rs > REL_TOL).any():
        i = np.flatnonzero(rs > REL_TOL)[:5]
        raise ParityFailure(f"{name}: scale off by more than {REL_TOL} relative at groups {i}: "
                            f"gpu {gs[i]} oracle {ref_scale[i]}")
    if not (rk <= REL_TOL).all():
        i = np.flatnonzero(~(rk <= REL_TOL))[:5]
        raise ParityFailure(f"{name}: k off by more than {REL_TOL} relative at groups {i}: "
                            f"gpu {gk[i]} oracle {ref_k[i]}")

    # codes: identical, or exactly one ordinal away in the signed ordering
    o_gpu = signed_ordinal(gpu_codes)
    o_ref = signed_ordinal(ref_state.codes)
    idx = np.flatnonzero(o_gpu != o_ref)
    step = np.abs(o_gpu[idx] - o_ref[idx])
    if (step > 1).any():
        j = idx[step > 1][:5]
        raise ParityFailure(f"{name}: codes more than one ordinal apart at {j}: gpu "
                            f"{gpu_codes[j]} oracle {ref_state.codes[j]} m_t {mt[j]}")
    if not signed and (o_gpu < 0).any():
        raise ParityFailure(f"{name}: signed code in a non-negative state at "
                            f"{np.flatnonzero(o_gpu < 0)[:5]}")

    s_out, k_out, c_out = _interval_diagnostic(gs, gk, gpu_codes, mt, delta, G)
    report[name] = dict(n=n, identical=1.0 - idx.size / max(1, n), mismatches=int(idx.size),
                        max_rel_scale=float(rs.max(initial=0)),
                        max_rel_k=float(rk.max(initial=0)),
                        groups=int(ref_scale.size),
                        outside_fp32_model=dict(scale=s_out, k=k_out, codes=c_out))


def compare_step(gpu, ref, G, hp, step, report=None):
    """gpu: dict of host arrays w, m_codes, m_scale, m_k, v_codes, v_scale,
    v_k.  ref: output of oracle_reference.  Raises ParityFailure on any
    per-group or per-element gate; the identical-code fraction is gated over a
    whole call by gate_identical()."""
    report = {} if report is None else report
    b1, b2 = hp["beta1"], hp["beta2"]
    g = ref["g"].astype(np.float64)
    xm = b1 * np.abs(ref["x_m"].astype(np.float64))
    xv = b2 * np.abs(ref["x_v"].astype(np.float64))
    delta_m = ref["dq_m"] * xm + ARITH_REL * (xm + (1 - b1) * np.abs(g))
    delta_v = ref["dq_v"] * xv + ARITH_REL * (xv + (1 - b2) * g * g)
    _check_state("m", gpu["m_codes"], gpu["m_scale"], gpu["m_k"], ref["m"], ref["m_t"],
                 delta_m, G, report, signed=True)
    _check_state("v", gpu["v_codes"], gpu["v_scale"], gpu["v_k"], ref["v"], ref["v_t"],
                 delta_v, G, report, signed=False)
    # weights
    lr, eps = hp["lr"], hp["eps"]
    bc1 = 1 - b1 ** step
    bc2 = 1 - b2 ** step
    mt = ref["m_t"].astype(np.float64)
    vt = ref["v_t"].astype(np.float64)
    den = np.sqrt(vt / bc2) + eps
    grad_step = abs(lr) * np.abs(mt / bc1) / den
    step_operands = abs(lr) * (xm + (1 - b1) * np.abs(g)) / bc1 / den
    w_ref = ref["w"].astype(np.float64)
    dw = np.abs(gpu["w"].astype(np.float64) - w_ref)
    wtol = REL_TOL * (np.abs(w_ref) + step_operands)
    if not (dw <= wtol).all():
        j = np.flatnonzero(~(dw <= wtol))[:5]
        raise ParityFailure(f"w outside tolerance at {j}: gpu {gpu['w'][j]} oracle "
                            f"{ref['w'][j]} tol {wtol[j]} (w before {ref['w_prev'][j]})")
    with np.errstate(divide="ignore", invalid="ignore"):
        rw = dw / np.abs(w_ref)
    # diagnostic: a floor of two FP32 ulps of the larger operand of the final
    # subtraction instead of 1e-5 of the step
    big = np.maximum(np.abs(ref["w_prev"].astype(np.float64)), grad_step).astype(np.float32)
    ulp_floor = 2.0 * np.spacing(big).astype(np.float64)
    report["w"] = dict(n=int(dw.size), max_abs=float(dw.max(initial=0)),
                       frac_rel_1e5=float(np.mean(rw <= REL_TOL)) if rw.size else 1.0,
                       floor_used=int(np.sum(rw > REL_TOL)),
                       outside_ulp_floor=int(np.sum(dw > REL_TOL * np.abs(w_ref) + ulp_floor)))
    return report


def gate_identical(reports, tag="", states=("m", "v")):
    """The identical-code gate over every code of one call (all tensors, or
    all sampled groups): at least MIN_IDENTICAL of each state's codes.
    Returns {state: (identical fraction, codes)}."""
    out = {}
    for s in states:
        n = sum(r[s]["n"] for r in reports)
        mism = sum(r[s]["mismatches"] for r in reports)
        ident = 1.0 - mism / max(1, n)
        if n and ident < MIN_IDENTICAL:
            raise ParityFailure(f"{tag} {s}: only {ident:.6f} of {n} codes identical "
                                f"({mism} differ by one ordinal)")
        out[s] = (ident, n)
    return out


def summary(reports, tag=""):
    """One printable line of the plain figures over a call's reports."""
    ident = gate_identical(reports, tag)
    rs = max(max(r["m"]["max_rel_scale"], r["v"]["max_rel_scale"]) for r in reports)
    rk = max(max(r["m"]["max_rel_k"], r["v"]["max_rel_k"]) for r in reports)
    nw = sum(r["w"]["n"] for r in reports)
    floor = sum(r["w"]["floor_used"] for r in reports)
    ulp = sum(r["w"]["outside_ulp_floor"] for r in reports)
    dwmax = max(r["w"]["max_abs"] for r in reports)
    diag = {s: {k: sum(r[s]["outside_fp32_model"][k] for r in reports)
                for k in ("scale", "k", "codes")} for s in ("m", "v")}
    return (f"{tag}: identical codes m {ident['m'][0]:.6f} v {ident['v'][0]:.6f} "
            f"(of {ident['m'][1]}); max rel scale {rs:.2e}, max rel k {rk:.2e}; "
            f"w max |dw| {dwmax:.2e}, {floor} of {nw} weights inside the step floor only "
            f"({ulp} outside a two-ulp floor); outside the FP32-dequantization model {diag}")
