"""Sizes past 2^31 elements, where 32-bit index arithmetic would overflow:
one optimizer tensor of 2^31 + 12345 elements (its last groups, the short
tail group included, lie beyond 2^31), a 65536 x 40960 activation matrix and
a linear layer whose 65536 x 33024 output has 2.16e9 elements.  The oracle
checks sampled groups or rows; properties that hold everywhere are checked
on the device."""
import gc

import numpy as np
import pytest
import torch

import oracle
from adamw_coat_fp8_amd import inputs
from gpu_util import DEV, bits_np, lib, require_gpu
from parity import compare_step, oracle_reference, summary
from test_gpu_gemm import assert_codes_near_ties

pytestmark = pytest.mark.gpu

HP = inputs.DEFAULT_HPARAMS


def setup_module():
    require_gpu()


def teardown_function(_):
    gc.collect()
    torch.cuda.empty_cache()


def test_step_tensor_past_2_31_elements():
    """One tensor of 2^31 + 12345 elements, G = 128.  Sampled groups (the
    first, the one holding element 2^31, the last full one and the 57-element
    tail, plus random ones) get an oracle state from two oracle steps; the GPU
    then steps the whole tensor and the sampled groups are compared with the
    oracle's step from that state."""
    from adamw_coat_fp8_amd.shard import FP8AdamWShard
    n, G = (1 << 31) + 12345, 128
    ng = (n + G - 1) // G
    print(f"[maxsize] step tensor of {n} elements", flush=True)
    shard = FP8AdamWShard([n], group_size=G, device=DEV)
    er = shard.element_range(0)                    # the buffers are padded past n
    shard.w[er] = inputs.weights(n, 0, DEV)
    rng = np.random.default_rng(9)
    pick = sorted({0, (1 << 31) // G, ng - 2, ng - 1} | set(int(x) for x in rng.integers(0, ng, 100)))
    full = [j for j in pick if j < ng - 1]
    pieces = [full, [ng - 1]]                      # full groups together; the tail alone
    eidx, gsel, st = [], [], []
    for p in pieces:
        e = np.concatenate([np.arange(j * G, min(n, (j + 1) * G)) for j in p])
        eidx.append(torch.from_numpy(e).to(DEV))
        gsel.append(torch.from_numpy(np.array(p)).to(DEV))
        w = shard.w[eidx[-1]].cpu().numpy()
        m, v = oracle.QuantizedState.zeros(e.size, G), oracle.QuantizedState.zeros(e.size, G)
        for t in (1, 2):                           # warm oracle state, seeded gradients
            g = bits_np(inputs.gradient(e.size, 1e-3, t, 7, "cpu"))
            oracle.adamw_fp8_step(w, g, m, v, G, **HP, step=t)
        st.append(dict(w=w, m=m, v=v))
        shard.w[eidx[-1]] = torch.from_numpy(w).to(DEV)
        shard.m_codes[eidx[-1]] = torch.from_numpy(m.codes).to(DEV)
        shard.v_codes[eidx[-1]] = torch.from_numpy(v.codes).to(DEV)
        shard.m_scale[gsel[-1]] = torch.from_numpy(m.scale).to(DEV)
        shard.m_k[gsel[-1]] = torch.from_numpy(m.k).to(DEV)
        shard.v_scale[gsel[-1]] = torch.from_numpy(v.scale).to(DEV)
        shard.v_k[gsel[-1]] = torch.from_numpy(v.k).to(DEV)
    shard.grad[er] = inputs.gradient(n, 1e-3, 3, 0, DEV)
    shard.step(3, **HP)
    torch.cuda.synchronize()
    reps = []
    for s, e, gs in zip(st, eidx, gsel):
        g = shard.grad[e].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle_reference(s["w"], g, s["m"], s["v"], G, HP, 3)
        gpu = dict(w=shard.w[e].cpu().numpy(), m_codes=shard.m_codes[e].cpu().numpy(),
                   m_scale=shard.m_scale[gs].cpu().numpy(), m_k=shard.m_k[gs].cpu().numpy(),
                   v_codes=shard.v_codes[e].cpu().numpy(), v_scale=shard.v_scale[gs].cpu().numpy(),
                   v_k=shard.v_k[gs].cpu().numpy())
        reps.append(compare_step(gpu, ref, G, HP, 3))
    print(f"[maxsize] {summary(reps, 'step past 2^31')}", flush=True)
    del shard


def test_act_quantizer_past_2_31_elements():
    coat = lib()
    rows, cols, G = 65536, 40960, 128
    print(f"[maxsize] activation {rows}x{cols}", flush=True)
    x = inputs.activation(rows, cols, 5, DEV, "llm", G)
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, cols // G), dtype=torch.float32, device=DEV)
    codes_t = torch.empty((cols, rows), dtype=torch.uint8, device=DEV)
    coat.quantize_act(x, codes, scales, codes_t, group_size=G)
    torch.cuda.synchronize()
    assert torch.equal(codes_t, codes.t().contiguous())
    sel = np.array([0, 1, 32767, 32768, 52429, rows - 1])
    sub = x[torch.from_numpy(sel).to(DEV)]
    rc, rs, _ = oracle.quantize_act(bits_np(sub).reshape(len(sel), cols), len(sel), cols, G,
                                    transpose=False)
    assert np.array_equal(codes[torch.from_numpy(sel).to(DEV)].cpu().numpy(), rc)
    got_s = scales[torch.from_numpy(sel).to(DEV)].cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), rs.view(np.uint32))


def test_gemm_output_past_2_31_elements():
    coat = lib()
    M, N, K, G = 65536, 33024, 128, 128
    print(f"[maxsize] linear layer {M}x{N}x{K}", flush=True)
    a, b, sa, sb = inputs.fp8_operands(M, N, K, 8, DEV, "exact")
    codes = torch.empty((M, N), dtype=torch.uint8, device=DEV)
    scales = torch.empty((M, N // G), dtype=torch.float32, device=DEV)
    coat.gemm_group_quant(a, b, sa, sb, codes, scales, group_size=G)
    torch.cuda.synchronize()
    sel = np.array([0, 16383, 32768, 65024, M - 1])
    rc, rs, _, c32 = oracle.gemm_fp8_group_quant(a.cpu().numpy()[sel], b.cpu().numpy(), sa, sb, G,
                                                 want_c=True)
    assert_codes_near_ties("past 2^31", codes[torch.from_numpy(sel).to(DEV)].cpu().numpy(), rc,
                           c32.astype(np.float64), G)
    got_s = scales[torch.from_numpy(sel).to(DEV)].cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), rs.view(np.uint32))
