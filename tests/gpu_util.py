"""Helpers shared by the GPU tests: host<->device copies of states and the
per-step "oracle-forced" check (the GPU starts each step from the oracle's
state; no oracle input ever comes from the GPU).  The identical-code gate
applies over every code of the call, per state."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from parity import compare_step, gate_identical, oracle_reference

DEV = "cuda"


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def lib():
    from adamw_coat_fp8_amd import coat
    return coat


def to_dev_state(st: "oracle.QuantizedState"):
    coat = lib()
    return coat.QuantState(torch.from_numpy(st.codes.copy()).to(DEV),
                           torch.from_numpy(st.scale.copy()).to(DEV),
                           torch.from_numpy(st.k.copy()).to(DEV))


def to_host_state(st) -> "oracle.QuantizedState":
    return oracle.QuantizedState(st.codes.cpu().numpy().copy(), st.scale.cpu().numpy().copy(),
                                 st.k.cpu().numpy().copy())


def bits_np(g_bf16: torch.Tensor) -> np.ndarray:
    return g_bf16.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def forced_step_check(tensors, hp, step, G, reports=None):
    """tensors: list of dicts with host arrays w, g (uint16 bits) and oracle
    states m, v (pre-step).  Runs ONE GPU call over all tensors from those
    states, the oracle per tensor, compares, and returns the oracle's post-step
    states (for the next step) plus the per-tensor reports."""
    coat = lib()
    slots = []
    for t in tensors:
        w = torch.from_numpy(t["w"].copy()).to(DEV)
        g = torch.from_numpy(t["g"].view(np.int16).copy()).to(DEV).view(torch.bfloat16)
        slots.append(coat.ParamSlot(w, g, to_dev_state(t["m"]), to_dev_state(t["v"])))
    coat.adamw_fp8_step(slots, **hp, step=step, group_size=G)
    torch.cuda.synchronize()
    out = []
    reps = [] if reports is None else reports
    for t, s in zip(tensors, slots):
        ref = oracle_reference(t["w"], t["g"], t["m"], t["v"], G, hp, step)
        gpu = dict(w=s.w.cpu().numpy(), m_codes=s.m.codes.cpu().numpy(),
                   m_scale=s.m.scale.cpu().numpy(), m_k=s.m.k.cpu().numpy(),
                   v_codes=s.v.codes.cpu().numpy(), v_scale=s.v.scale.cpu().numpy(),
                   v_k=s.v.k.cpu().numpy())
        reps.append(compare_step(gpu, ref, G, hp, step))
        out.append(dict(w=ref["w"], m=ref["m"], v=ref["v"]))
    gate_identical(reps, f"step {step}")
    return out, reps
