"""Parity at the full workload sizes, in the launch configuration the
benchmark times (the whole shard, one library call per balanced run of at most
40 tensors), on sampled groups the oracle computes one by one.

The GPU runs the warm-up steps over the whole model.  The oracle runs the same
steps on the sampled groups alone, from the same seeded inputs (groups are
independent).  Before the checked step the oracle's state of the sampled
groups is written into the GPU buffers, so the checked step starts both sides
from the oracle's state; every other group keeps the GPU's own history.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from adamw_coat_fp8_amd import inputs
from gpu_util import DEV, lib, require_gpu
from parity import compare_step, oracle_reference, summary

pytestmark = pytest.mark.gpu

HP = inputs.DEFAULT_HPARAMS


def setup_module():
    require_gpu()


def teardown_function(_):
    gc.collect()
    torch.cuda.empty_cache()


def _pick_groups(shard, per_tensor, rng):
    """Flat element and group indices of the sampled groups: the first and last
    group of every tensor plus `per_tensor` random ones."""
    G = shard.group_size
    elem_idx, grp_idx, sizes = [], [], []
    for i, n in enumerate(shard.numels):
        ng = (n + G - 1) // G
        pick = {0, ng - 1} | set(int(x) for x in rng.integers(0, ng, per_tensor))
        e0, g0 = shard.offsets[i], shard.goffsets[i]
        for j in sorted(pick):
            L = min(G, n - j * G)
            elem_idx.append(np.arange(e0 + j * G, e0 + j * G + L))
            grp_idx.append(g0 + j)
            sizes.append(L)
    return elem_idx, np.array(grp_idx), sizes


def _run(workload, G, kind, warm, per_tensor, extra_tail=False):
    from adamw_coat_fp8_amd.shard import FP8AdamWShard
    specs = inputs.workload_specs(workload)
    numels = [s.numel for s in specs] + ([1000] if extra_tail else [])
    stds = inputs.grad_stds(len(numels))
    print(f"[fullsize] {workload} G={G} {kind}: {len(numels)} tensors, {sum(numels)} params",
          flush=True)
    shard = FP8AdamWShard(numels, group_size=G, device=DEV)
    inputs.fill_weights(shard)
    rng = np.random.default_rng(123)
    elem_list, gidx, sizes = _pick_groups(shard, per_tensor, rng)
    # full groups travel as one concatenated oracle tensor; short (tail)
    # groups as their own tensors
    full = [k for k, L in enumerate(sizes) if L == G]
    tails = [k for k, L in enumerate(sizes) if L != G]
    pieces = [full] + [[k] for k in tails]
    eidx = [torch.from_numpy(np.concatenate([elem_list[k] for k in p])).to(DEV) for p in pieces]
    gsel = [torch.from_numpy(gidx[p]).to(DEV) for p in pieces]
    st = []
    for e in eidx:
        n = e.numel()
        st.append(dict(w=shard.w[e].cpu().numpy(), m=oracle.QuantizedState.zeros(n, G),
                       v=oracle.QuantizedState.zeros(n, G)))
    for t in range(1, warm + 1):
        inputs.fill_gradients(shard, t, stds, kind)
        shard.step(t, **HP)
        for s, e in zip(st, eidx):
            g = shard.grad[e].view(torch.int16).cpu().numpy().view(np.uint16)
            oracle.adamw_fp8_step(s["w"], g, s["m"], s["v"], G, **HP, step=t)
        if t % 20 == 0 or t == warm:
            print(f"[fullsize] warm-up step {t} done", flush=True)
    torch.cuda.synchronize()
    # oracle state of the sampled groups into the GPU buffers
    for s, e, gs in zip(st, eidx, gsel):
        shard.w[e] = torch.from_numpy(s["w"]).to(DEV)
        shard.m_codes[e] = torch.from_numpy(s["m"].codes).to(DEV)
        shard.v_codes[e] = torch.from_numpy(s["v"].codes).to(DEV)
        shard.m_scale[gs] = torch.from_numpy(s["m"].scale).to(DEV)
        shard.m_k[gs] = torch.from_numpy(s["m"].k).to(DEV)
        shard.v_scale[gs] = torch.from_numpy(s["v"].scale).to(DEV)
        shard.v_k[gs] = torch.from_numpy(s["v"].k).to(DEV)
    t = warm + 1
    inputs.fill_gradients(shard, t, stds, kind)
    shard.step(t, **HP)
    torch.cuda.synchronize()
    reps = []
    for s, e, gs in zip(st, eidx, gsel):
        g = shard.grad[e].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle_reference(s["w"], g, s["m"], s["v"], G, HP, t)
        gpu = dict(w=shard.w[e].cpu().numpy(), m_codes=shard.m_codes[e].cpu().numpy(),
                   m_scale=shard.m_scale[gs].cpu().numpy(), m_k=shard.m_k[gs].cpu().numpy(),
                   v_codes=shard.v_codes[e].cpu().numpy(), v_scale=shard.v_scale[gs].cpu().numpy(),
                   v_k=shard.v_k[gs].cpu().numpy())
        reps.append(compare_step(gpu, ref, G, HP, t))
    print(f"[fullsize] {summary(reps, f'{workload} G={G} step {t}, {sum(sizes)} sampled params in {len(sizes)} groups')}",
          flush=True)
    del shard
    return reps


def test_olmo_1b_after_100_steps():
    _run("olmo_1b", 128, "gaussian", warm=100, per_tensor=6)


def test_llama2_7b():
    _run("llama2_7b", 128, "gaussian", warm=5, per_tensor=4)


def test_llama2_13b():
    _run("llama2_13b", 128, "gaussian", warm=5, per_tensor=3)


@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_llama2_7b_stress(G):
    _run("llama2_7b", G, "stress", warm=3, per_tensor=4, extra_tail=True)
