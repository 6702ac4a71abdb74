"""GPU parity of the per-group activation quantizer (coat_fp8_quantize_act)
against the oracle: bit-exact codes, scales and transposed codes.  The oracle
codes the exact quotient 448 x / max and stores max / 448 rounded once to
FP32; the kernel's FP32 quotient is exact at midpoints, and for BF16 inputs
the exact quotient is either a midpoint or far (relative 2^-13 and more) from
every midpoint, so no tolerance applies.  Cases: every group size over tile-aligned and ragged
shapes (rows not a multiple of 64 or 16, cols not a multiple of 128), the
stress recipe (zero, single-nonzero, subnormal, tiny, huge, tie, -0.0 and
wide-range groups), the variant without the transpose, the full 8192 x 11008
shape on sampled rows plus the transpose property over every element, and
host-side rejection of bad arguments."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from adamw_coat_fp8_amd import inputs
from gpu_util import DEV, bits_np, lib, require_gpu

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5          # output bytes the kernel must overwrite


def setup_module():
    require_gpu()


def _outputs(rows, cols, G, transpose=True):
    codes = torch.full((rows, cols), SENTINEL, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, cols // G), float("nan"), dtype=torch.float32, device=DEV)
    codes_t = (torch.full((cols, rows), SENTINEL, dtype=torch.uint8, device=DEV)
               if transpose else None)
    return codes, scales, codes_t


def _gpu(x, G, transpose=True):
    coat = lib()
    rows, cols = x.shape
    codes, scales, codes_t = _outputs(rows, cols, G, transpose)
    coat.quantize_act(x, codes, scales, codes_t, group_size=G)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), scales.cpu().numpy(),
            None if codes_t is None else codes_t.cpu().numpy())


def _oracle(x, G):
    rows, cols = x.shape
    return oracle.quantize_act(bits_np(x).reshape(rows, cols), rows, cols, G, transpose=True)


def _assert_same(tag, gpu, ref):
    gc, gs, gt = gpu
    rc, rs, rt = ref
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, f"{tag}: {len(bad)} codes differ, first at {bad[:4].tolist()}: " \
                          f"gpu {gc[tuple(bad[0])]:#04x} oracle {rc[tuple(bad[0])]:#04x}"
    sbad = np.argwhere(gs.view(np.uint32) != rs.view(np.uint32))
    assert sbad.size == 0, f"{tag}: {len(sbad)} scales differ, first at {sbad[:4].tolist()}"
    if gt is not None:
        tbad = np.argwhere(gt != rt)
        assert tbad.size == 0, f"{tag}: {len(tbad)} transposed codes differ, first at " \
                               f"{tbad[:4].tolist()}"


# rows % 16, 8, 4 select 16-, 8- and 4-byte stores into the transpose (40, 72: 8; 36, 100: 4)
SHAPES = [(1, 128), (3, 256), (64, 128), (65, 384), (130, 1024), (256, 640), (48, 4096),
          (17, 1152), (40, 1024), (72, 384), (36, 128), (100, 640)]


@pytest.mark.parametrize("G", [16, 32, 64, 128])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{r}x{c}" for r, c in SHAPES])
def test_llm_shapes_bit_exact(G, shape):
    rows, cols = shape
    x = inputs.activation(rows, cols, 1, DEV, "llm", G)
    print(f"[act] llm {rows}x{cols} G={G}", flush=True)
    _assert_same(f"llm {rows}x{cols} G={G}", _gpu(x, G), _oracle(x, G))


@pytest.mark.parametrize("shape,G", [((37, 48), 16), ((70, 96), 32), ((129, 192), 64),
                                     ((5, 16), 16), ((200, 32), 32)])
def test_partial_column_tiles(shape, G):
    rows, cols = shape
    x = inputs.activation(rows, cols, 2, DEV, "llm", G)
    print(f"[act] partial {rows}x{cols} G={G}", flush=True)
    _assert_same(f"partial {rows}x{cols} G={G}", _gpu(x, G), _oracle(x, G))


@pytest.mark.parametrize("G", [16, 32, 64, 128])
@pytest.mark.parametrize("shape", [(200, 1024), (77, 640), (64, 2048)])
def test_stress_bit_exact(G, shape):
    rows, cols = shape
    x = inputs.activation(rows, cols, 3, DEV, "stress", G)
    print(f"[act] stress {rows}x{cols} G={G}", flush=True)
    ref = _oracle(x, G)
    # the recipe reaches the cases it is meant to: zero groups, signed zero codes
    assert (ref[1] == 0).any() and (ref[0] == 0x80).any()
    _assert_same(f"stress {rows}x{cols} G={G}", _gpu(x, G), ref)


@pytest.mark.parametrize("G,shape", [(16, (96, 512)), (128, (96, 512)), (64, (4100, 2048))])
def test_without_transpose_same_codes(G, shape):
    """The variant without the transposed copy writes the same codes and
    scales, with 64-row tiles (96 x 512) and 128-row tiles (4100 x 2048)."""
    x = inputs.activation(*shape, 4, DEV, "stress", G)
    a = _gpu(x, G, transpose=True)
    b = _gpu(x, G, transpose=False)
    assert b[2] is None
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32),
                                                          b[1].view(np.uint32))


# Either side of the tile-height switch (128-row tiles at most two per CU on 256 CUs: 64-row
# tiles), with ragged row counts: 2040 rows (64-row tiles, 8-byte transposed stores), 2180 and
# 4100 rows (128-row tiles, 4-byte stores), 2179 rows (128-row tiles, byte stores).
SWITCH_SHAPES = [(2040, 4096), (2180, 4096), (4100, 2048), (2179, 4096)]


@pytest.mark.parametrize("shape", SWITCH_SHAPES, ids=[f"{r}x{c}" for r, c in SWITCH_SHAPES])
def test_tile_height_switch_bit_exact(shape):
    rows, cols = shape
    G = 128
    x = inputs.activation(rows, cols, 5, DEV, "llm", G)
    print(f"[act] tile switch {rows}x{cols}", flush=True)
    _assert_same(f"tile switch {rows}x{cols}", _gpu(x, G), _oracle(x, G))


@pytest.mark.parametrize("G", [128, 64, 32, 16])
def test_full_size_sampled_rows(G):
    """8192 x 11008 (4 sequences of 2048 tokens, FFN width 11008) at each
    group size, in the launch the benchmark times.  Oracle on 48 sampled rows
    (each row is independent), and codes_t == codes^T checked over every
    element on the device."""
    coat = lib()
    rows, cols = 8192, 11008
    print(f"[act] full size G={G}", flush=True)
    x = inputs.activation(rows, cols, 0, DEV, "llm", G)
    codes, scales, codes_t = _outputs(rows, cols, G)
    coat.quantize_act(x, codes, scales, codes_t, group_size=G)
    torch.cuda.synchronize()
    assert torch.equal(codes_t, codes.t().contiguous())
    sel = np.sort(np.random.default_rng(0).choice(rows, 48, replace=False))
    sel[0], sel[-1] = 0, rows - 1
    sub = x[torch.from_numpy(sel).to(DEV)]
    rc, rs, _ = _oracle(sub, G)
    gc = codes.cpu().numpy()[sel]
    gs = scales.cpu().numpy()[sel]
    assert np.array_equal(gc, rc)
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))


def test_empty_is_noop_and_bad_arguments_rejected():
    coat = lib()
    vp = ctypes.c_void_p
    x = inputs.activation(32, 256, 5, DEV, "llm", 128)
    codes, scales, codes_t = _outputs(32, 256, 16)
    snap = [t.clone() for t in (codes, scales, codes_t)]
    raw = coat.lib.coat_fp8_quantize_act
    s = torch.cuda.current_stream().cuda_stream
    xp, cp, sp, tp = x.data_ptr(), codes.data_ptr(), scales.data_ptr(), codes_t.data_ptr()
    cases = [
        ((xp, 0, 256, 16, cp, sp, tp), coat.COAT_OK),            # empty: nothing written
        ((xp, 32, 0, 16, cp, sp, tp), coat.COAT_OK),
        ((None, 0, 0, 16, None, None, None), coat.COAT_OK),
        ((xp, -1, 256, 16, cp, sp, tp), coat.COAT_ERR_INVALID_VALUE),
        ((xp, 32, 250, 16, cp, sp, tp), coat.COAT_ERR_INVALID_VALUE),   # cols % G
        ((xp, 32, 256, 24, cp, sp, tp), coat.COAT_ERR_GROUP_SIZE),
        ((None, 32, 256, 16, cp, sp, tp), coat.COAT_ERR_NULL_POINTER),
        ((xp, 32, 256, 16, None, sp, tp), coat.COAT_ERR_NULL_POINTER),
        ((xp, 32, 256, 16, cp, None, tp), coat.COAT_ERR_NULL_POINTER),
        ((xp + 2, 32, 128, 16, cp, sp, tp), coat.COAT_ERR_MISALIGNED),
        ((xp, 32, 256, 16, cp + 8, sp, tp), coat.COAT_ERR_MISALIGNED),
        ((xp, 32, 256, 16, cp, sp + 2, tp), coat.COAT_ERR_MISALIGNED),
        ((xp, 32, 256, 16, cp, sp, tp + 4), coat.COAT_ERR_MISALIGNED),
    ]
    for args, want in cases:
        got = raw(*[vp(a) if a is not None else None for a in args[:1]], args[1], args[2],
                  args[3], *[vp(a) if a is not None else None for a in args[4:]], vp(s))
        assert got == want, (args, got, want)
    torch.cuda.synchronize()
    # bit patterns: the scale sentinel is NaN
    assert torch.equal(codes, snap[0]) and torch.equal(codes_t, snap[2])
    assert torch.equal(scales.view(torch.int32), snap[1].view(torch.int32))
    with pytest.raises(coat.CoatError):
        coat.quantize_act(x, codes, scales, codes_t, group_size=24)


def _random_shapes(count=12, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        G = int(rng.choice([16, 32, 64, 128]))
        rows = int(rng.integers(1, 2500))
        cols = G * int(rng.integers(1, 3072 // G + 1))
        out.append((rows, cols, G, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _random_shapes(), ids=lambda c: "x".join(map(str, c)))
def test_random_shapes_bit_exact(case):
    """Seeded random rows (1-2499), column counts (any multiple of G up to
    3072) and G, with and without the transpose: codes, scales and transposed
    codes bit for bit against the oracle."""
    rows, cols, G, transpose = case
    x = inputs.activation(rows, cols, 9, DEV, "llm", G)
    print(f"[act] random {rows}x{cols} G={G} transpose={transpose}", flush=True)
    gpu = _gpu(x, G, transpose)
    ref = _oracle(x, G)
    if not transpose:
        ref = (ref[0], ref[1], None)
    _assert_same(f"random {case}", gpu, ref)


def test_graph_capture_replays_match_eager():
    """Three quantizer calls captured in one HIP graph: a ragged matrix on
    64-row tiles with and without the transpose, and a 4096 x 4096 matrix on
    128-row tiles.  The graph is replayed three times, with the outputs reset
    and eager work between replays; every replay's codes, scales and
    transposed codes equal an eager call's bit for bit."""
    coat = lib()
    cases = [(300, 1152, 64, True), (300, 1152, 64, False), (4096, 4096, 128, True)]
    xs = [inputs.activation(r, c, 31 + i, DEV, "llm", G) for i, (r, c, G, _) in enumerate(cases)]
    eager, captured = [], []
    for x, (r, c, G, tr) in zip(xs, cases):
        e = _outputs(r, c, G, tr)
        coat.quantize_act(x, *e, group_size=G)
        eager.append(e)
        captured.append(_outputs(r, c, G, tr))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x, (r, c, G, tr), o in zip(xs, cases, captured):
            coat.quantize_act(x, *o, group_size=G)
    torch.cuda.synchronize()
    for replay in range(3):
        for codes, scales, codes_t in captured:
            codes.fill_(SENTINEL)
            scales.fill_(float("nan"))
            if codes_t is not None:
                codes_t.fill_(SENTINEL)
        scratch = torch.randn(1 << 16, device=DEV).sum()      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for case, e, g in zip(cases, eager, captured):
            assert torch.equal(g[0], e[0]), f"replay {replay} {case}: codes"
            assert torch.equal(g[1].view(torch.int32), e[1].view(torch.int32)), \
                f"replay {replay} {case}: scales"
            if e[2] is not None:
                assert torch.equal(g[2], e[2]), f"replay {replay} {case}: transposed codes"
        del scratch
