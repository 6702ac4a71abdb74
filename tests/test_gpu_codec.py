"""GPU parity of the codec entry points against the oracle: the element-wise
E4M3 cast (bit-exact), stand-alone dequantize-expand (relative error bound)
and expand-quantize (scale exact, k within 1e-5, at least 99.99% of codes
identical and the rest one ordinal away)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, lib, require_gpu, to_dev_state
from parity import REL_TOL, _check_state, dequant_bound, gate_identical

pytestmark = pytest.mark.gpu


def setup_module():
    require_gpu()


def test_decode_all_codes_bit_exact():
    coat = lib()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(DEV)
    x = torch.empty(256, dtype=torch.float32, device=DEV)
    coat.e4m3_decode(codes, x)
    got = x.cpu().numpy().astype(np.float64)
    ref = oracle.e4m3_decode_array(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _encode_gpu(x_np):
    coat = lib()
    x = torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).to(DEV)
    c = torch.empty(x.numel(), dtype=torch.uint8, device=DEV)
    coat.e4m3_encode(x, c)
    return c.cpu().numpy()


def test_encode_dense_sweep_bit_exact():
    # every 7th FP32 bit pattern in [0, 448] (~163M values) and their negatives
    # would be slow on the host; take every 997th plus all near-tie values
    bits = np.arange(0, 0x43E00001, 997, dtype=np.uint32)
    x = bits.view(np.float32)
    table = np.unique(np.abs(oracle.e4m3_decode_array(np.arange(0x7F))))
    mids = (table[:-1] + table[1:]) / 2
    near = []
    for m in mids.astype(np.float32):
        v = m
        for _ in range(4):
            v = np.nextafter(v, np.float32(0))
        for _ in range(9):
            near.append(v)
            v = np.nextafter(v, np.float32(1e9))
    x = np.concatenate([x, np.array(near, np.float32), table.astype(np.float32),
                        np.array([448.0, 460.0, 463.99, 1e6, 3e38], np.float32)])
    for sgn in (1.0, -1.0):
        xs = (sgn * x).astype(np.float32)
        got = _encode_gpu(xs)
        ref = oracle.e4m3_encode_array(xs.astype(np.float64))
        # signed zero: the oracle gives 0x00 for -0.0
        zero = xs == 0
        assert np.array_equal(got[~zero], ref[~zero])
        assert np.all((got[zero] & 0x7F) == 0)


def test_encode_exhaustive_fp32_range():
    """Every FP32 bit pattern in [-448, 448] (2.28e9 values) through the GPU
    cast equals the oracle's RNE encoder; -0.0 may give 0x80 or 0x00."""
    import concurrent.futures as cf
    coat = lib()
    end = 0x43E00001                      # bits of 448.0, inclusive
    chunk = 1 << 26
    codes = torch.empty(chunk, dtype=torch.uint8, device=DEV)
    pool = cf.ThreadPoolExecutor(8)

    def host_ref(bits_np):
        parts = np.array_split(bits_np, 8)
        return np.concatenate(list(pool.map(
            lambda b: oracle.e4m3_encode_array(b.view(np.float32).astype(np.float64)), parts)))

    for sign in (0, 1):
        for start in range(0, end, chunk):
            stop = min(end, start + chunk)
            bits = torch.arange(start, stop, dtype=torch.int32, device=DEV)
            if sign:
                bits = bits + torch.iinfo(torch.int32).min       # set bit 31
            c = codes[:stop - start]
            coat.e4m3_encode(bits.view(torch.float32), c)
            got = c.cpu().numpy()
            hb = np.arange(start, stop, dtype=np.uint32) | np.uint32(sign << 31)
            ref = host_ref(hb)
            if start == 0:                                    # +-0.0
                assert (got[0] & 0x7F) == 0 and ref[0] == 0
                got, ref = got[1:], ref[1:]
            bad = np.flatnonzero(got != ref)
            assert bad.size == 0, (sign, start, bad[:4], got[bad[:4]], ref[bad[:4]])
    pool.shutdown()
    print("[codec] exhaustive FP32 [-448, 448] sweep bit-exact", flush=True)


def _random_groups(rng, n, G, spreads):
    x = np.empty(n, np.float32)
    for g0 in range(0, n, G):
        sp = spreads[(g0 // G) % len(spreads)]
        L = min(G, n - g0)
        mag = np.exp2(rng.uniform(-sp / 2, sp / 2, L) + rng.uniform(-30, 5))
        x[g0:g0 + L] = mag * np.where(rng.random(L) < 0.5, -1, 1)
    x[rng.random(n) < 0.05] = 0.0
    return x


@pytest.mark.parametrize("G", [16, 32, 64, 128])
@pytest.mark.parametrize("n", [1, 1000, 4096, 70000 + 3])
def test_dequantize_matches_oracle(G, n):
    coat = lib()
    rng = np.random.default_rng(G * 7 + n)
    x = _random_groups(rng, n, G, [0.5, 4, 10, 20, 40, 100])
    st = oracle.expand_quantize(x, G)
    ref = oracle.dequantize_expand(st, G).astype(np.float64)
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    coat.dequantize_expand(to_dev_state(st), out, G)
    got = out.cpu().numpy().astype(np.float64)
    zero = ref == 0
    assert np.array_equal(got[zero], ref[zero])
    rel = np.abs(got[~zero] - ref[~zero]) / np.abs(ref[~zero])
    bound = dequant_bound(st, G)[~zero]
    print(f"[dequant] G={G} n={n}: max rel err {rel.max(initial=0):.2e}, "
          f"max rel err / bound {np.max(rel / bound, initial=0):.2f}", flush=True)
    assert np.all(rel <= bound)
    assert rel.max(initial=0) <= REL_TOL
    assert np.array_equal(np.signbit(got[~zero]), np.signbit(ref[~zero]))


@pytest.mark.parametrize("G", [16, 32, 64, 128])
@pytest.mark.parametrize("n", [1, 17, 1000, 65536, 70000 + 3])
def test_expand_quantize_matches_oracle(G, n):
    coat = lib()
    rng = np.random.default_rng(G * 13 + n)
    x = _random_groups(rng, n, G, [0.0, 0.5, 4, 10, 14.8, 20, 40, 100])
    if n > 100:
        x[:G] = 0.0                       # an all-zero group
        x[G:2 * G] = 0.0
        x[G + 3] = -2.5e-9                 # a single-nonzero group
    ref = oracle.expand_quantize(x, G)
    out = coat.QuantState.zeros(n, G, DEV)
    coat.expand_quantize(torch.from_numpy(x).to(DEV), out, G)
    torch.cuda.synchronize()
    gs, gk = out.scale.cpu().numpy(), out.k.cpu().numpy()
    assert np.array_equal(gs, ref.scale)          # max|x| is exact
    rep = {}
    # inputs are exact on both sides: zero-width box, only near-tie slack
    _check_state("x", out.codes.cpu().numpy(), gs, gk, ref, x, np.zeros(n), G, rep, signed=True)
    gate_identical([rep], f"expand_quantize G={G} n={n}", states=("x",))
    nz = ref.scale > 0
    assert np.all(np.abs(gk[nz] - ref.k[nz]) <= 1e-5 * ref.k[nz])
    assert np.all(gk[~nz] == 1.0)


@pytest.mark.parametrize("G", [128, 32])
def test_full_size_codec_sampled_groups(G):
    """Both codec entry points at the benchmark's launch: one call each over a
    Llama-2-7B-sized FP32 first moment (6,738,415,616 values, the benchmark's
    input recipe, at G = 128 and at G = 32, the other group size measured).  On 1,500 sampled groups (the first, the one
    holding element 2^31, the last, and random ones): expand-quantize against
    the oracle's (scale exact, k within 1e-5, codes by the parity rules), and
    dequantize-expand of the GPU's own state against the oracle's
    dequantization of it (within the relative error bound)."""
    from adamw_coat_fp8_amd import inputs
    coat = lib()
    numels = [s.numel for s in inputs.workload_specs("llama2_7b")]
    n = sum(numels)
    ng = n // G
    print(f"[codec] full size: {n} values, G={G}", flush=True)
    x = inputs.fill_moment_like(torch.empty(n, dtype=torch.float32, device=DEV), numels,
                                inputs.grad_stds(len(numels)))
    st = coat.QuantState.zeros(n, G, DEV)
    coat.expand_quantize(x, st, G)
    y = torch.empty_like(x)
    coat.dequantize_expand(st, y, G)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    pick = np.array(sorted({0, (1 << 31) // G, ng - 1} | set(int(v) for v in rng.integers(0, ng, 1497))))
    e = torch.from_numpy((pick[:, None] * G + np.arange(G)[None, :]).ravel()).to(DEV)
    gsel = torch.from_numpy(pick).to(DEV)
    xs = x[e].cpu().numpy()
    ref = oracle.expand_quantize(xs, G)
    gs, gk = st.scale[gsel].cpu().numpy(), st.k[gsel].cpu().numpy()
    assert np.array_equal(gs, ref.scale)
    rep = {}
    _check_state("x", st.codes[e].cpu().numpy(), gs, gk, ref, xs, np.zeros(xs.size), G, rep,
                 signed=True)
    gate_identical([rep], "expand_quantize full size", states=("x",))
    nz = ref.scale > 0
    assert np.all(np.abs(gk[nz] - ref.k[nz]) <= 1e-5 * ref.k[nz])
    # dequantize-expand of the GPU's own state on the same groups
    gst = oracle.QuantizedState(st.codes[e].cpu().numpy(), gs.copy(), gk.copy())
    dref = oracle.dequantize_expand(gst, G).astype(np.float64)
    got = y[e].cpu().numpy().astype(np.float64)
    zero = dref == 0
    assert np.array_equal(got[zero], dref[zero])
    rel = np.abs(got[~zero] - dref[~zero]) / np.abs(dref[~zero])
    assert np.all(rel <= dequant_bound(gst, G)[~zero])
    print(f"[codec] full size: {rep['x']['identical']:.6f} codes identical, dequant max rel err "
          f"{rel.max(initial=0):.2e}", flush=True)
    del x, y, st
    torch.cuda.empty_cache()


def test_graph_capture_replays_match_eager():
    """Expand-quantize and then dequantize-expand of the same state (n with
    a partial last group), captured in one HIP graph and replayed three times
    with the outputs reset and eager work between replays: every replay's
    codes, scale, k and FP32 output equal an eager call's bit for bit."""
    coat = lib()
    G, n = 32, 70000 + 3
    rng = np.random.default_rng(404)
    x = torch.from_numpy(_random_groups(rng, n, G, [0.0, 0.5, 4, 10, 20, 40])).to(DEV)
    st_e = coat.QuantState.zeros(n, G, DEV)
    y_e = torch.empty(n, dtype=torch.float32, device=DEV)
    coat.expand_quantize(x, st_e, G)
    coat.dequantize_expand(st_e, y_e, G)
    st_g = coat.QuantState.zeros(n, G, DEV)
    y_g = torch.empty(n, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        coat.expand_quantize(x, st_g, G)
        coat.dequantize_expand(st_g, y_g, G)
    torch.cuda.synchronize()
    for replay in range(3):
        st_g.codes.fill_(0xA5)
        st_g.scale.fill_(float("nan"))
        st_g.k.fill_(float("nan"))
        y_g.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device=DEV).sum()      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st_g.codes, st_e.codes), f"replay {replay}: codes"
        assert torch.equal(st_g.scale.view(torch.int32), st_e.scale.view(torch.int32)), \
            f"replay {replay}: scale"
        assert torch.equal(st_g.k.view(torch.int32), st_e.k.view(torch.int32)), f"replay {replay}: k"
        assert torch.equal(y_g.view(torch.int32), y_e.view(torch.int32)), f"replay {replay}: output"
        del scratch
