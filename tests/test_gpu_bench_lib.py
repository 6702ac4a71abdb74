"""The benchmark's math-free copy of the step's traffic (libcoat_bench.so,
coat_bench_mix_ceiling): it runs on the benchmark's real shard, so it must
leave every byte of every stream as it was, touch every full tile, and reject
bad arguments without launching."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV, require_gpu

pytestmark = pytest.mark.gpu


def setup_module():
    require_gpu()


def _lib():
    from adamw_coat_fp8_amd import build
    lib = ctypes.CDLL(build.BENCH_LIB)
    vp = ctypes.c_void_p
    lib.coat_bench_mix_ceiling.restype = ctypes.c_int
    lib.coat_bench_mix_ceiling.argtypes = [vp] * 8 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                      ctypes.c_uint32, vp]
    return lib


@pytest.mark.parametrize("G", [16, 32, 64, 128])
def test_mix_ceiling_leaves_the_shard_unchanged(G):
    from adamw_coat_fp8_amd.shard import FP8AdamWShard
    numels = [1024 * 37 + 128, 4096, 1024 * 3]
    sh = FP8AdamWShard(numels, group_size=G, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(G)
    streams = [sh.w, sh.grad, sh.m_codes, sh.v_codes, sh.m_scale, sh.m_k, sh.v_scale, sh.v_k]
    for t in streams:
        t.view(torch.uint8).copy_(torch.randint(0, 256, (t.numel() * t.element_size(),),
                                                generator=gen, device=DEV, dtype=torch.uint8))
    before = [t.view(torch.uint8).clone() for t in streams]
    lib = _lib()
    n = sh.total_elems // 1024 * 1024
    rc = lib.coat_bench_mix_ceiling(*[t.data_ptr() for t in streams], n, sh.total_groups, G, 0,
                                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    for a, b in zip(before, streams):
        assert torch.equal(a, b.view(torch.uint8))
    # a nonzero mask changes every full tile's w words (so every tile is visited)
    rc = lib.coat_bench_mix_ceiling(*[t.data_ptr() for t in streams], n, sh.total_groups, G,
                                    0xFFFFFFFF, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    w0 = before[0].view(torch.int32).cpu().numpy()
    w1 = sh.w.view(torch.int32).cpu().numpy()
    changed = (w0[:n] != w1[:n]).reshape(-1, 1024).mean(axis=1)
    assert changed.min() > 0.5                     # every full tile was visited
    assert np.array_equal(w0[n:], w1[n:])          # nothing past the full tiles


def test_mix_ceiling_rejects_bad_arguments():
    lib = _lib()
    buf = torch.zeros(4096, dtype=torch.float32, device=DEV)
    p = buf.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    assert lib.coat_bench_mix_ceiling(None, p, p, p, p, p, p, p, 2048, 16, 128, 0, s) == 1
    assert lib.coat_bench_mix_ceiling(p, p, p, p, p, p, p, p, 1000, 16, 128, 0, s) == 1
    assert lib.coat_bench_mix_ceiling(p, p, p, p, p, p, p, p, 2048, 16, 48, 0, s) == 1
    assert lib.coat_bench_mix_ceiling(p + 4, p, p, p, p, p, p, p, 2048, 16, 128, 0, s) == 1
