"""Host-side logic that runs without a GPU: workload shapes, the flat shard
layout, the split of a tensor list into library calls, the benchmark's byte
accounting and its refusal of multi-GPU runs, and the stress input recipe."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from adamw_coat_fp8_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,tensors,params", [
    ("single_1m", 1, 1_048_576),
    ("olmo_1b", 146, 1_176_832_000),
    ("llama2_7b", 291, 6_738_415_616),
    ("llama2_13b", 363, 13_015_864_320),
])
def test_workload_shapes(name, tensors, params):
    specs = inputs.workload_specs(name)
    assert len(specs) == tensors
    assert inputs.total_params(specs) == params
    # every tensor of these shapes is a whole number of 128-element groups
    assert all(s.numel % 128 == 0 for s in specs)


def test_balanced_calls_cover_list_within_launch_capacity():
    from adamw_coat_fp8_amd.shard import MAX_TENSORS_PER_CALL, balanced_calls
    for name in ("olmo_1b", "llama2_7b", "llama2_13b"):
        numels = [s.numel for s in inputs.workload_specs(name)]
        calls = balanced_calls(numels)
        flat = [i for c in calls for i in c]
        assert flat == list(range(len(numels)))          # contiguous, in order
        assert all(1 <= len(c) <= MAX_TENSORS_PER_CALL for c in calls)
        sizes = [sum(numels[i] for i in c) for c in calls]
        assert max(sizes) <= 1.3 * sum(numels) / len(calls)
    rng = np.random.default_rng(0)
    numels = [int(x) for x in rng.integers(1, 10_000, 500)]
    calls = balanced_calls(numels)
    assert [i for c in calls for i in c] == list(range(500))
    assert all(len(c) <= MAX_TENSORS_PER_CALL for c in calls)


def test_flat_shard_layout_alignment():
    from adamw_coat_fp8_amd.shard import FP8AdamWShard
    numels = [1000, 1, 17, 4096, 4101, 128 * 3]
    for G in (16, 32, 64, 128):
        sh = FP8AdamWShard(numels, group_size=G, device="cpu")
        for i, n in enumerate(numels):
            slot = sh.slots[i]
            assert slot.w.numel() == n and slot.grad.numel() == n
            assert slot.m.codes.numel() == n and slot.v.codes.numel() == n
            assert slot.m.scale.numel() == -(-n // G) == slot.v.k.numel()
            for t in (slot.w, slot.grad, slot.m.codes, slot.v.codes):
                assert t.data_ptr() % 16 == 0
            for t in (slot.m.scale, slot.m.k, slot.v.scale, slot.v.k):
                assert t.data_ptr() % 4 == 0
        # views do not overlap
        ends = [(sh.offsets[i], sh.offsets[i] + n) for i, n in enumerate(numels)]
        assert all(a[1] <= b[0] for a, b in zip(ends, ends[1:]))
        assert sh.state_bytes() == 2 * sh.total_elems + 16 * sh.total_groups


def test_bench_byte_accounting():
    sys.path.insert(0, ROOT)
    import bench
    numels = [s.numel for s in inputs.workload_specs("llama2_7b")]
    total = sum(bench.algorithmic_bytes(n, 128) for n in numels)
    # 14 B per parameter and 32 B per 128-element group
    assert total == 14 * 6_738_415_616 + 32 * 52_643_872 == 96_022_422_528


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stress_recipe_features():
    n, G = 128 * 400 + 77, 128
    g = inputs.gradient(n, 1e-3, 1, 0, "cpu", kind="stress", group_size=G).float().numpy()
    g2 = inputs.gradient(n, 1e-3, 2, 0, "cpu", kind="stress", group_size=G).float().numpy()
    zero1, zero2 = g == 0, g2 == 0
    assert 0.05 < zero1.mean() < 0.15               # 5% mask plus zeroed groups
    zero3 = inputs.gradient(n, 1e-3, 3, 0, "cpu", kind="stress", group_size=G).float().numpy() == 0
    # the exact-zero mask is the same on every step (plus the all-zero groups)
    assert (zero1 & zero2 & zero3).mean() > 0.05
    assert np.array_equal(zero1 & zero2, zero1 & zero2 & zero3)
    groups = np.split(g, np.arange(G, n, G))
    nnz = np.array([np.count_nonzero(x) for x in groups])
    assert (nnz == 1).any() and (nnz == 0).any()     # single-nonzero and all-zero groups
    assert np.any(np.isclose(np.abs(g), 4.5e-15, rtol=0.01))   # tiny magnitudes
    assert inputs.gradient(n, 1e-3, 1, 0, "cpu", kind="stress", group_size=G).dtype == torch.bfloat16


def test_bench_act_byte_accounting():
    sys.path.insert(0, ROOT)
    import bench
    # read BF16 2 B, write codes 1 B + transposed codes 1 B, FP32 scale per group
    assert bench.act_bytes(8192, 11008, 128) == 8192 * 11008 * 4 + 4 * 8192 * 86 == 363_528_192
    assert bench.act_bytes(8192, 11008, 16, transpose=False) == 8192 * 11008 * 3 + 4 * 8192 * 688


def test_activation_recipe_features():
    rows, cols = 256, 1024
    x = inputs.activation(rows, cols, 0, "cpu", "llm", 128)
    assert x.dtype == torch.bfloat16 and x.shape == (rows, cols)
    ch = x.float().abs().amax(0)
    assert 3 <= int((ch > 20).sum()) <= 40                      # ~1% outlier channels
    assert torch.equal(x, inputs.activation(rows, cols, 0, "cpu", "llm", 128))
    for G in (16, 128):
        s = inputs.activation(rows, cols, 3, "cpu", "stress", G).float()
        grp = s.reshape(rows, cols // G, G)
        amax = grp.abs().amax(-1)
        nnz = (grp != 0).sum(-1)
        assert (amax == 0).any() and (nnz == 1).any()           # zero and single-nonzero
        assert ((amax > 0) & (amax < 2.0 ** -126)).any()        # subnormal groups
        assert ((amax >= 2.0 ** -126) & (amax < 2.0 ** -100)).any()
        assert (amax > 1e29).any()
        assert (torch.signbit(s) & (s == 0)).any()              # -0.0 entries
        tie = (amax / 448.0).log2()
        assert ((tie == tie.round()) & (amax > 0)).any()        # max = 448 * 2^e
    with pytest.raises(ValueError):
        inputs.activation(4, 100, 0, "cpu", "llm", 16)


def test_bench_codec_byte_accounting():
    """Codec traffic: 4 B of FP32 and 1 B of code per element, scale and k
    (8 B) per group, in either direction."""
    import bench
    assert bench.codec_bytes(128 * 1024, 128) == 5 * 128 * 1024 + 8 * 1024
    assert bench.codec_bytes(1000, 16) == 5 * 1000 + 8 * 63


def test_shard_over_another_shards_storage():
    """A shard for another group size built over an existing shard's buffers
    shares its memory, starts from fresh (zero) state, and rejects storage
    whose per-group arrays are too short."""
    from adamw_coat_fp8_amd.shard import FP8AdamWShard
    numels = [1000, 4096 + 5, 3 * 128, 17]
    base = FP8AdamWShard(numels, group_size=16, device="cpu")
    base.m_codes.fill_(7)
    base.v_scale.fill_(1.5)
    sh = FP8AdamWShard(numels, group_size=128, device="cpu", storage=base)
    assert sh.w.data_ptr() == base.w.data_ptr() and sh.m_k.data_ptr() == base.m_k.data_ptr()
    assert not sh.m_codes.any() and not sh.v_scale.any()
    assert sh.total_groups == sum(-(-n // 128) for n in numels)
    for i, n in enumerate(numels):
        assert sh.slot(i).w.numel() == n
    with pytest.raises(ValueError):
        FP8AdamWShard(numels, group_size=16, device="cpu", storage=sh)


def test_bench_separate_streams_bound():
    """The no-mixing bound of the step's traffic: equal read and write rates
    give that rate; otherwise the byte-weighted harmonic mean of the two, with
    8 + 16/G bytes read and 6 + 16/G written per parameter."""
    sys.path.insert(0, ROOT)
    import bench
    assert bench.separate_streams_gbps(128, 5000.0, 5000.0) == pytest.approx(5000.0)
    rd, wr = 8.125, 6.125
    want = (rd + wr) / (rd / 6500.0 + wr / 5900.0)
    assert bench.separate_streams_gbps(128, 6500.0, 5900.0) == pytest.approx(want)
    assert 5900.0 < want < 6500.0
    # smaller groups move more per-group bytes both ways
    assert bench.separate_streams_gbps(16, 6500.0, 5900.0) != pytest.approx(want)
