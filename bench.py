#!/usr/bin/env python3
"""Benchmark of the fused FP8 AdamW step (COAT, dynamic range expansion) on one
MI355X.

A step is one call of the whole hot path over the whole workload: dequantize
m and v, AdamW on FP32 master weights from BF16 gradients, per-group
max/min-nonzero, k and scale, re-quantize to E4M3 -- for every tensor.

Workload (default): the Llama-2-7B-shaped parameter list on one GPU
(291 tensors, 6,738,415,616 parameters, G = 128), all buffers resident in HBM,
synthetic seeded data (w ~ N(0, 0.02); per-tensor gradient std log-uniform in
[1e-5, 1e-2]; BF16 gradients).  Warm-up steps draw a fresh gradient each step
(state history), the timed steps reuse the last gradient (its values do not
change the work or the traffic).

Prints ONE JSON line: Gparam/s over the timed steps, plus the step kernel's
roofline position (algorithmic bytes per launch / average launch duration,
HIP events on the launch stream), the rate of a math-free kernel that moves
exactly the step's traffic with its lane layout (libcoat_bench.so: the
streaming ceiling of this read/write mix, timed on the same shard), plain
read-only and write-only streams on the same shard (after the steps; the
write stream overwrites the gradient buffer), the
stress recipe at G = 128, 64, 32 and 16 (one shard each, alternating timed
rounds in this process), and the CPU oracle timed on bounded samples on the
host cores (all threads, and one thread on the single 1024 x 1024 tensor and
on 64M-parameter slices of the OLMo-1B and Llama-2-7B shapes).

``--path act_quant`` measures the per-group activation quantizer instead: one
step quantizes a (tokens x channels) BF16 matrix (default 8192 x 11008: four
2048-token sequences at the Llama-2-7B FFN width) into E4M3 codes, per-group
scales and the transposed codes; it reports Gelem/s and the same roofline and
CPU-oracle objects.  ``--path gemm_group_quant`` measures the group-scaled FP8
linear layer (TFLOP/s against the matrix cores' FP8 peak), and ``--path codec``
the stand-alone expand-quantize / dequantize-expand entry points on a
Llama-2-7B-sized FP32 moment.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
# The activation quantizer's calls last tens of microseconds, and an event
# pair around every call adds about 2.5 us to each (the event packets between
# two launches hold the next one back), so its launches are timed in batches
# of this many back-to-back calls per event pair.
ACT_CALLS_PER_EVENT = 10
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_adamw_fp8_step_llama2_7b.txt")
PMC_SUMMARY_ACT = os.path.join(ROOT, "profiles", "pmc_quantize_act_8192x11008.txt")
PMC_SUMMARY_GEMM = os.path.join(ROOT, "profiles", "pmc_gemm_group_quant_8192x11008x4096.txt")
PMC_SUMMARY_CODEC = os.path.join(ROOT, "profiles", "pmc_codec_llama2_7b.txt")
_CSRC = os.path.join(ROOT, "adamw_coat_fp8_amd", "csrc")
# the sources each profiled kernel is built from
STEP_SOURCES = [os.path.join(_CSRC, f) for f in ("coat_fp8.hip", "coat_common.h")]
ACT_SOURCES = [os.path.join(_CSRC, f) for f in ("coat_act.hip", "coat_common.h")]
GEMM_SOURCES = [os.path.join(_CSRC, f) for f in ("coat_gemm.hip", "coat_common.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--path", choices=("adamw_step", "act_quant", "gemm_group_quant", "codec"),
                    default="adamw_step")
    ap.add_argument("--gemm-shape", default="8192x11008x4096",
                    help="M x N x K of the FP8 linear layer (gemm_group_quant)")
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 for act_quant)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default 5; 20 for act_quant)")
    ap.add_argument("--act-shape", default="8192x11008",
                    help="rows x cols of the activation matrix (act_quant)")
    ap.add_argument("--no-transpose", action="store_true",
                    help="act_quant without the transposed copy")
    ap.add_argument("--workload", default="llama2_7b")
    ap.add_argument("--group-size", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=128 * 1024 * 1024,
                    help="parameters in the oracle's timing sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (PMC calibration)")
    ap.add_argument("--no-g-sweep", action="store_true",
                    help="adamw_step without the stress-recipe group-size sweep")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="adamw_step without the OLMo-1B and Llama-2-13B shapes")
    ap.add_argument("--g-sweep-only", action="store_true",
                    help="adamw_step: only the group-size sweep (for profiling it)")
    ap.add_argument("--allocations", type=int, default=1,
                    help="adamw_step: time the step on this many successive allocations of "
                         "the shard in one process (the shard is freed and allocated again)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="adamw_step: only the math-free copy of the step's traffic")
    args = ap.parse_args()
    act = args.path == "act_quant"
    gemm = args.path == "gemm_group_quant"
    codec = args.path == "codec"
    if args.steps is None:
        args.steps = 200 if act else (100 if gemm else (10 if codec else 20))
    if args.warmup is None:
        args.warmup = 20 if act else (30 if gemm else (2 if codec else 5))
    return args


def algorithmic_bytes(n: int, G: int) -> int:
    """Per tensor: read w 4 + g 2 + m 1 + v 1, write w 4 + m 1 + v 1 bytes per
    element; per group read and write scale and k of both moments (32 B)."""
    return 14 * n + 32 * ((n + G - 1) // G)


def kernel_source_sha(sources=STEP_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def act_bytes(rows: int, cols: int, G: int, transpose: bool = True) -> int:
    """Read x (2 B per element); write codes (1 B), the transposed codes (1 B)
    and one FP32 scale per group."""
    return rows * cols * (3 + (1 if transpose else 0)) + 4 * rows * (cols // G)


def traffic_from_profile(nbytes_per_launch, path=PMC_SUMMARY, sources=STEP_SOURCES,
                         key="hbm_bytes_per_launch"):
    """HBM traffic per launch (the summary's `key`) from the committed
    rocprofv3 PMC summary, if it was taken on the current kernel source; else
    None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha(sources):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_slice(specs, G, stds, budget, seed_steps=(1, 2)):
    """Host copies of the first elements of each tensor of a workload (up to
    2M per tensor) until `budget` parameters: w, the gradients of steps 1 and
    2 and zero states, for the oracle."""
    import numpy as np
    import oracle
    from adamw_coat_fp8_amd import inputs

    work, left = [], budget
    for i, s in enumerate(specs):
        if left <= 0:
            break
        n = min(s.numel, 2 * 1024 * 1024, left)
        n -= n % G if n >= G else 0
        w = inputs.weights(n, i, "cpu").numpy().copy()
        gs = [inputs.bf16_bits(inputs.gradient(n, stds[i], t, i, "cpu")).numpy().view(np.uint16).copy()
              for t in seed_steps]
        work.append([w, gs, oracle.QuantizedState.zeros(n, G), oracle.QuantizedState.zeros(n, G)])
        left -= n
    return work


def _oracle_step(item, step, G, hp):
    import oracle
    w, gs, m, v = item
    oracle.adamw_fp8_step(w, gs[min(step, len(gs)) - 1], m, v, G, **hp, step=step)


def cpu_baseline(specs, G, hp, sample_params, min_seconds=8.0):
    """The oracle, as it stands, timed on bounded samples on the host cores.

    value: all threads (up to 16) over a `sample_params` sample of the
    workload -- the first elements of each tensor (up to 2M per tensor),
    warm state from one untimed oracle step, then whole timed steps (the
    gradient of step 2 is reused, which leaves the work unchanged) until
    `min_seconds`; threads split the sample by tensor slices (the oracle is
    single-threaded C; ctypes releases the GIL).

    single_core: the same oracle on one thread over the single 1024 x 1024
    tensor, all 10 steps from zero state, and over 64M-parameter slices of the
    OLMo-1B and Llama-2-7B shapes, one step each from a warm state (made by
    one untimed step on all threads)."""
    import numpy as np
    import oracle
    from adamw_coat_fp8_amd import inputs

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    stds = inputs.grad_stds(len(specs))
    work = _oracle_slice(specs, G, stds, sample_params)
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda it: _oracle_step(it, 1, G, hp), work))
        steps = 0
        t0 = time.perf_counter()
        while True:
            list(ex.map(lambda it: _oracle_step(it, 2 + steps, G, hp), work))
            steps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    n_total = sum(it[0].size for it in work)
    del work

    single = {}
    # single 1024 x 1024 tensor, 10 steps from zero state, one thread
    n1 = 1024 * 1024
    w = inputs.weights(n1, 0, "cpu").numpy().copy()
    grads = [inputs.bf16_bits(inputs.gradient(n1, 1e-3, t, 0, "cpu")).numpy().view(np.uint16).copy()
             for t in range(1, 11)]
    m, v = oracle.QuantizedState.zeros(n1, G), oracle.QuantizedState.zeros(n1, G)
    t0 = time.perf_counter()
    for t in range(1, 11):
        oracle.adamw_fp8_step(w, grads[t - 1], m, v, G, **hp, step=t)
    dt1 = time.perf_counter() - t0
    single["single_1m"] = {"value": round(10 * n1 / dt1 / 1e6, 3), "unit": "Mparam/s",
                           "sample": f"1024x1024 tensor, steps 1-10 from zero state, "
                                     f"{dt1:.2f} s wall"}
    for name in ("olmo_1b", "llama2_7b"):
        wspecs = inputs.workload_specs(name)
        wstds = inputs.grad_stds(len(wspecs))
        sl = _oracle_slice(wspecs, G, wstds, 64 * 1024 * 1024)
        with cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda it: _oracle_step(it, 1, G, hp), sl))    # warm state
        ns = sum(it[0].size for it in sl)
        t0 = time.perf_counter()
        for it in sl:
            _oracle_step(it, 2, G, hp)
        dts = time.perf_counter() - t0
        n_full = sum(sp.numel for sp in wspecs)
        single[name] = {"value": round(ns / dts / 1e6, 3), "unit": "Mparam/s",
                        "sample": f"{ns} params (first <=2M elements of the first {len(sl)} "
                                  f"tensors), step 2 after an untimed step 1, {dts:.2f} s wall",
                        "full_step_s_extrapolated": round(n_full * dts / ns, 1)}
        del sl
    rate = steps * n_total / dt
    return {"value": rate / 1e9, "unit": "Gparam/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n_total} params: first <=2M elements of the first tensors, "
                      f"{steps} whole steps after one untimed step, {dt:.2f} s wall",
            "full_step_s_extrapolated": round(sum(sp.numel for sp in specs) / rate, 1),
            "single_core": dict(single, cores=1)}


def cpu_baseline_act(rows, cols, G, transpose, min_seconds=10.0):
    """The oracle's activation quantizer timed on the same matrix, split over
    host threads by row blocks (rows are independent), repeated over whole
    passes until at least `min_seconds` of wall time."""
    import numpy as np
    import oracle
    from adamw_coat_fp8_amd import inputs

    x = inputs.activation(rows, cols, 0, "cpu", "llm", G)
    bits = inputs.bf16_bits(x).numpy().view(np.uint16)
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    blocks = np.array_split(np.arange(rows), threads)

    def run(rs):
        if len(rs):
            oracle.quantize_act(bits[rs[0]:rs[-1] + 1], len(rs), cols, G, transpose=transpose)

    passes = 0
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, blocks))                      # untimed pass
        t0 = time.perf_counter()
        while True:
            list(ex.map(run, blocks))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    return {"value": passes * rows * cols / dt / 1e9, "unit": "Gelem/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"the whole {rows}x{cols} matrix, {passes} passes after an untimed one, "
                      f"{dt:.2f} s wall"}


def copy_ceiling_gbps(reps: int = 5) -> float:
    """Median rate of a plain 4 GiB device-to-device copy (read + write bytes
    over time): the streaming ceiling of this GPU, for context."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    dst.copy_(src)
    rates = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        rates.append(2 * src.numel() * 4 / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    torch.cuda.synchronize()
    return sorted(rates)[len(rates) // 2]


def batched_launch_ms(call, calls: int, stream) -> list:
    """Enqueues `calls` calls of call(k) on `stream`, ACT_CALLS_PER_EVENT
    back to back between the two events of a pair, and returns the mean
    time of one launch in each batch (ms), from the HIP events."""
    import torch
    nb = -(-calls // ACT_CALLS_PER_EVENT)
    events = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
              for _ in range(nb)]
    sizes = []
    k = 0
    for e0, e1 in events:
        n = min(ACT_CALLS_PER_EVENT, calls - k)
        e0.record(stream)
        for _ in range(n):
            call(k)
            k += 1
        e1.record(stream)
        sizes.append(n)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / n for (a, b), n in zip(events, sizes)]


def same_shape_copy_gbps(sets, calls: int) -> float:
    """Rate of torch's copy of each buffer set's BF16 input into a BF16
    matrix of the same shape (read + write bytes per launch over the mean
    HIP-event time of a launch), timed exactly as the quantizer is: buffer
    sets in turn, batches of back-to-back calls per event pair.  It moves
    the quantizer's bytes at its shape with no arithmetic, so it is the
    streaming ceiling of that shape, launch and ramp included."""
    import torch
    stream = torch.cuda.current_stream()
    dsts = [torch.empty_like(s[0]) for s in sets]

    def call(k):
        dsts[k % len(sets)].copy_(sets[k % len(sets)][0])

    for k in range(2 * len(sets)):
        call(k)
    torch.cuda.synchronize()
    per = batched_launch_ms(call, calls, stream)
    ms = sum(per) / len(per)
    nbytes = 2 * sets[0][0].numel() * sets[0][0].element_size()
    del dsts
    torch.cuda.synchronize()
    return nbytes / (ms * 1e-3) / 1e9


def cast_ceilings_gbps(x, y, calls: int):
    """Torch's plain casts with the codec's per-element traffic and no group
    statistics: FP32 -> E4M3 (read 4 B, write 1 B) over the same FP32 state,
    and E4M3 -> FP32 back into `y`, each timed with an event pair per call.
    Returns GB/s of 5 B per element for each direction."""
    import torch
    f8 = torch.empty(x.numel(), dtype=torch.float8_e4m3fn, device=x.device)
    f8.copy_(x)
    y.copy_(f8)
    torch.cuda.synchronize()

    def timed(fn):
        ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
              for _ in range(calls)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / calls

    nbytes = 5 * x.numel()
    q = nbytes / (timed(lambda: f8.copy_(x)) * 1e-3) / 1e9
    d = nbytes / (timed(lambda: y.copy_(f8)) * 1e-3) / 1e9
    del f8
    torch.cuda.synchronize()
    return q, d


def copy_probe():
    """Three 4 GiB device-to-device copies: a kernel of known traffic against
    which the profiler's FETCH_SIZE / WRITE_SIZE counters are scaled."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("[bench] copy probe: 3 x 4 GiB device copies done", file=sys.stderr, flush=True)
    del src, dst


def bench_act(args):
    import torch
    from adamw_coat_fp8_amd import coat, inputs

    G = args.group_size
    rows, cols = (int(v) for v in args.act_shape.lower().split("x"))
    transpose = not args.no_transpose
    # Several independent buffer sets, used in turn, so that no call finds its
    # input in the 256 MB last-level cache: at least 2 GiB in all.
    nset = max(2, -(-(2 << 30) // (4 * rows * cols)))
    print(f"[bench] act_quant {rows}x{cols} G={G} transpose={transpose}, {nset} buffer sets",
          file=sys.stderr, flush=True)
    torch.cuda.init()
    sets = []
    for i in range(nset):
        sets.append((inputs.activation(rows, cols, i, "cuda", "llm", G),
                     torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
                     torch.empty((rows, cols // G), dtype=torch.float32, device="cuda"),
                     torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
                     if transpose else None))
    stream = torch.cuda.current_stream()

    def call(k):
        x, codes, scales, codes_t = sets[k % nset]
        coat.quantize_act(x, codes, scales, codes_t, group_size=G, stream=stream)

    for k in range(args.warmup):
        call(k)
    torch.cuda.synchronize()
    print(f"[bench] {args.warmup} warm-up calls done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per_batch = batched_launch_ms(call, args.steps, stream)
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    avg_launch_ms = sum(per_batch) / len(per_batch)
    launch_sorted = sorted(per_batch)
    nbytes = act_bytes(rows, cols, G, transpose)
    achieved = nbytes / (avg_launch_ms * 1e-3) / 1e9
    same_copy = same_shape_copy_gbps(sets, args.steps)
    ceiling = copy_ceiling_gbps()
    if args.copy_probe:
        copy_probe()
    print(f"[bench] {args.steps} timed calls: {ms_per_step * 1e3:.1f} us/call wall, "
          f"avg launch {avg_launch_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    traffic = traffic_from_profile(nbytes, PMC_SUMMARY_ACT, ACT_SOURCES) if transpose else None
    rec = {
        "metric": "Gelem/s per per-group E4M3 activation quantization (codes + transposed "
                  "codes) + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(rows * cols / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"activation {rows}x{cols} BF16 (tokens x channels), 1x{G} groups, "
                        f"E4M3 codes{' + transposed codes' if transpose else ''} + FP32 scales",
            "buffer_sets": nset,
            "group_size": G,
            "algorithmic_bytes_per_step": nbytes,
            "calls_per_event_pair": ACT_CALLS_PER_EVENT,
            "launch_ms_median": round(launch_sorted[len(launch_sorted) // 2], 5),
            "launch_ms_min": round(launch_sorted[0], 5),
            "copy_ceiling_GBps": round(ceiling, 1),
            "kernel_frac_of_copy_ceiling": round(achieved / ceiling, 4),
            "same_shape_copy_GBps": round(same_copy, 1),
            "kernel_frac_of_same_shape_copy": round(achieved / same_copy, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": f"quantize_act_kernel<{G}, {'true' if transpose else 'false'}>",
            "bytes_per_launch": nbytes,
            "avg_launch_ms": round(avg_launch_ms, 5),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_act(rows, cols, G, transpose)
    print(json.dumps(rec), flush=True)


MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 matrix-core peak


def cpu_baseline_gemm(a, b, sa, sb, G, min_seconds=10.0):
    """The oracle's group-scaled linear layer timed on whole rows of the same
    operands (rows are independent), split over host threads, repeated until
    at least `min_seconds` of wall time."""
    import numpy as np
    import oracle

    an, bn = a.cpu().numpy(), b.cpu().numpy()
    M, K = an.shape
    N = bn.shape[0]
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    rows_per_pass = 2 * threads
    sel = [an[i:i + 2] for i in range(0, rows_per_pass * 1, 2)][:threads]

    def run(x):
        oracle.gemm_fp8_group_quant(x, bn, sa, sb, G)

    passes = 0
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, sel))                      # untimed pass
        t0 = time.perf_counter()
        while True:
            list(ex.map(run, sel))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    flops = passes * 2.0 * sum(x.shape[0] for x in sel) * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{sum(x.shape[0] for x in sel)} of {M} rows x {N} x {K} (exact int64 "
                      f"sums), {passes} passes after an untimed one, {dt:.2f} s wall"}


def gemm_tiling(M, N):
    """The library's tile plan for an M x N output: 256 x 256 tiles (the last
    tile column 128 wide when N is an odd multiple of 128), with the tiles of
    a last round that would leave over half the CUs idle run as 128 x 256
    halves, the last blocks of the same launch."""
    import torch
    tiles = -(-M // 256) * -(-N // 256)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rem = tiles % cus
    if rem == 0 or 2 * rem > cus:
        return f"256x256 ({tiles} tiles)"
    return f"256x256 ({tiles - rem} tiles) + 128x256 halves of the last {rem} tiles (same launch)"


def bench_gemm(args):
    import torch
    from adamw_coat_fp8_amd import coat, inputs

    G = args.group_size
    M, N, K = (int(v) for v in args.gemm_shape.lower().split("x"))
    print(f"[bench] gemm_group_quant {M}x{N}x{K} G={G}", file=sys.stderr, flush=True)
    torch.cuda.init()
    a, b, sa, sb = inputs.fp8_operands(M, N, K, 0, "cuda", "llm")
    codes = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    scales = torch.empty((M, N // G), dtype=torch.float32, device="cuda")
    c16 = torch.empty((M, N), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    flops = 2.0 * M * N * K

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
              for _ in range(steps)]
        t0 = time.perf_counter()
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        launch = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        return wall * 1e3, sum(launch) / len(launch), launch[len(launch) // 2]

    fused = lambda: coat.gemm_group_quant(a, b, sa, sb, codes, scales, group_size=G, stream=stream)
    plain = lambda: coat.gemm_bf16(a, b, sa, sb, c16, stream=stream)
    for _ in range(args.warmup):          # both kernels warm (clocks, caches) before either is timed
        plain()
    ms_wall, ms_launch, ms_med = timed(fused, args.steps, args.warmup)
    print(f"[bench] fused: {ms_launch * 1e3:.1f} us per launch", file=sys.stderr, flush=True)
    _, ms_plain, _ = timed(plain, args.steps, args.warmup)
    # the unfused alternative: the plain GEMM, then the activation quantizer on its BF16 output
    codes2 = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    scales2 = torch.empty((M, N // G), dtype=torch.float32, device="cuda")
    c16b = c16.view(torch.bfloat16)
    unfused = lambda: (plain(), coat.quantize_act(c16b, codes2, scales2, None, group_size=G,
                                                  stream=stream))
    _, ms_unfused, _ = timed(unfused, args.steps, args.warmup)
    context = {"plain_bf16_epilogue_ms": round(ms_plain, 5),
               "group_epilogue_overhead": round(ms_launch / ms_plain - 1.0, 4),
               "unfused_bf16_gemm_then_quantizer_ms": round(ms_unfused, 5),
               "fused_saving_vs_unfused": round(1.0 - ms_launch / ms_unfused, 4),
               "tile": gemm_tiling(M, N)}
    # a library FP8 GEMM (hipBLASLt through torch) for context, where torch provides one
    try:
        af = a.view(torch.float8_e4m3fn)
        bf = b.view(torch.float8_e4m3fn)
        one = torch.tensor(1.0, device="cuda")
        lib_mm = lambda: torch._scaled_mm(af, bf.t(), scale_a=one, scale_b=one,
                                          out_dtype=torch.bfloat16)
        lib_mm()
        _, ms_lib, _ = timed(lib_mm, args.steps, args.warmup)
        context["library_fp8_gemm_bf16_ms"] = round(ms_lib, 5)
        context["library_fp8_gemm_bf16_TFLOPs"] = round(flops / (ms_lib * 1e-3) / 1e12, 1)
    except Exception as e:                      # noqa: BLE001 - context only
        context["library_fp8_gemm_bf16"] = f"unavailable: {type(e).__name__}"
    achieved = flops / (ms_launch * 1e-3) / 1e12
    if args.copy_probe:
        copy_probe()
    # minimum HBM bytes: read A and B once, write codes and scales once
    min_bytes = M * K + N * K + M * N + 4 * M * (N // G)
    traffic = (traffic_from_profile(min_bytes, PMC_SUMMARY_GEMM, GEMM_SOURCES)
               if (M, N, K, G) == (8192, 11008, 4096, 128) else None)
    context["min_hbm_bytes"] = min_bytes
    rec = {
        "metric": "TFLOP/s per group-scaled FP8 linear layer (FP8 GEMM + fused 1xG group "
                  "quantization of its output), 1 GPU",
        "value": round(flops / (ms_wall * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {
            "workload": f"linear layer {M}x{N}x{K}: E4M3 activations (per-tensor) x E4M3 "
                        f"weights (per-tensor), output 1x{G} group-quantized E4M3 + FP32 scales",
            "group_size": G,
            "launch_ms_median": round(ms_med, 5),
            **context,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": MFMA_FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": f"gemm_fp8_kernel<{G}, group quant> (one launch per call)",
            "flops_per_launch": flops,
            "avg_launch_ms": round(ms_launch, 5),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_gemm(a, b, sa, sb, G)
    print(json.dumps(rec), flush=True)


def codec_bytes(n: int, G: int) -> int:
    """Either direction: FP32 values (4 B) one way, E4M3 codes (1 B) the
    other, and the group's FP32 scale and k (8 B per group)."""
    return 5 * n + 8 * ((n + G - 1) // G)


def cpu_baseline_codec(G, sample, min_seconds=10.0):
    """The oracle's expand-quantize and dequantize-expand round trip on a
    bounded sample, split over host threads in group-aligned slices."""
    import numpy as np
    import oracle
    import torch

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    gen = torch.Generator().manual_seed(7)
    x = (torch.randn(sample, generator=gen) * 1e-3).numpy()
    per = -(-sample // threads)
    per += (-per) % G
    slices = [x[i:i + per] for i in range(0, sample, per)]

    def run(xs):
        oracle.dequantize_expand(oracle.expand_quantize(xs, G), G)

    passes = 0
    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(run, slices))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    return {"value": passes * sample / dt / 1e9, "unit": "Gelem/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{sample} N(0, 1e-3) FP32 values, {passes} round trips "
                      f"(expand-quantize, then dequantize-expand), {dt:.2f} s wall"}


def bench_codec(args):
    """The stand-alone codec entry points on a Llama-2-7B-sized first moment:
    expand-quantize of the whole FP32 state into E4M3 codes + scale + k
    (converting an FP32 optimizer checkpoint), then dequantize-expand back to
    FP32.  One call each over the flat buffer: every tensor of the workload is
    a multiple of G elements, so its groups are the per-tensor groups."""
    import torch
    from adamw_coat_fp8_amd import coat, inputs

    G = args.group_size
    specs = inputs.workload_specs(args.workload)
    numels = [s.numel for s in specs]
    n = sum(numels)
    if any(x % G for x in numels):
        raise SystemExit("codec bench: every tensor must be a multiple of G")
    print(f"[bench] codec {args.workload}: {n} elements, G={G}", file=sys.stderr, flush=True)
    torch.cuda.init()
    x = inputs.fill_moment_like(torch.empty(n, dtype=torch.float32, device="cuda"), numels,
                                inputs.grad_stds(len(specs)))
    state = coat.QuantState.zeros(n, G, "cuda")
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        coat.expand_quantize(x, state, group_size=G, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        coat.dequantize_expand(state, y, group_size=G, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {args.warmup} warm-up round trips done", file=sys.stderr, flush=True)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    q_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    d_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    nbytes = codec_bytes(n, G)
    q_gbs = nbytes / (q_ms * 1e-3) / 1e9
    d_gbs = nbytes / (d_ms * 1e-3) / 1e9
    print(f"[bench] {args.steps} timed round trips: {ms_per_step:.3f} ms wall; expand-quantize "
          f"{q_ms:.3f} ms ({q_gbs:.0f} GB/s), dequantize-expand {d_ms:.3f} ms ({d_gbs:.0f} GB/s)",
          file=sys.stderr, flush=True)
    if args.copy_probe:
        copy_probe()
    cast_q, cast_d = cast_ceilings_gbps(x, y, args.steps)
    ceiling = copy_ceiling_gbps()
    rec = {
        "metric": "Gelem/s per expand-quantize + dequantize-expand round trip of an FP32 "
                  "optimizer state + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(n / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload} first moment: {n} FP32 values (per-tensor N(0, 0.1 sigma_i)) "
                        f"<-> E4M3 codes + per-group FP32 scale and k",
            "group_size": G,
            "algorithmic_bytes_per_launch": nbytes,
            "dequantize_expand": {
                "avg_launch_ms": round(d_ms, 4),
                "achieved_GBps": round(d_gbs, 1),
                "frac": round(d_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(nbytes, PMC_SUMMARY_CODEC, STEP_SOURCES,
                                                "dequantize_hbm_bytes_per_launch"),
            },
            "copy_ceiling_GBps": round(ceiling, 1),
            "torch_cast_fp32_to_e4m3_GBps": round(cast_q, 1),
            "quantize_frac_of_cast": round(q_gbs / cast_q, 4),
            "torch_cast_e4m3_to_fp32_GBps": round(cast_d, 1),
            "dequantize_frac_of_cast": round(d_gbs / cast_d, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(q_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(q_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(nbytes, PMC_SUMMARY_CODEC, STEP_SOURCES,
                                            "quantize_hbm_bytes_per_launch"),
            "kernel": f"codec_kernel<{G}, quantize>",
            "bytes_per_launch": nbytes,
            "avg_launch_ms": round(q_ms, 4),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline_codec(G, 1 << 26)
    print(json.dumps(rec), flush=True)


BENCH_LIB = os.path.join(ROOT, "adamw_coat_fp8_amd", "libcoat_bench.so")
G_SWEEP = (128, 64, 32, 16)


def mix_ceiling(shard, reps: int = 10):
    """The math-free copy of the step's traffic (libcoat_bench.so) over the
    whole flat shard, in place and value-preserving: average GB/s of
    algorithmic bytes per launch over `reps` launches (HIP events on the
    launch stream), after two untimed launches."""
    import ctypes
    import torch

    lib = ctypes.CDLL(BENCH_LIB)
    vp = ctypes.c_void_p
    lib.coat_bench_mix_ceiling.restype = ctypes.c_int
    lib.coat_bench_mix_ceiling.argtypes = [vp] * 8 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                      ctypes.c_uint32, vp]
    stream = torch.cuda.current_stream()
    G = shard.group_size
    n = shard.total_elems // 1024 * 1024
    args = [shard.w.data_ptr(), shard.grad.data_ptr(), shard.m_codes.data_ptr(),
            shard.v_codes.data_ptr(), shard.m_scale.data_ptr(), shard.m_k.data_ptr(),
            shard.v_scale.data_ptr(), shard.v_k.data_ptr(), n, shard.total_groups, G, 0,
            stream.cuda_stream]

    def launch():
        rc = lib.coat_bench_mix_ceiling(*args)
        if rc != 0:
            raise RuntimeError(f"coat_bench_mix_ceiling returned {rc}")

    launch()
    launch()
    ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / reps
    nbytes = 14 * n + 32 * (n // G)
    return nbytes / (ms * 1e-3) / 1e9, ms, nbytes


def separate_streams_gbps(G: int, read_gbps: float, write_gbps: float) -> float:
    """Rate of the step's traffic (8 + 16/G bytes read and 6 + 16/G written
    per parameter) if the reads moved at `read_gbps` and the writes at
    `write_gbps` one after the other, with no read/write mixing."""
    rd, wr = 8 + 16 / G, 6 + 16 / G
    return (rd + wr) / (rd / read_gbps + wr / write_gbps)


def stream_ceilings(shard, reps: int = 10):
    """Plain read-only and write-only streams (libcoat_bench.so) on the same
    shard: the read stream over its FP32 weights, the write stream over its
    BF16 gradient buffer, which it overwrites with zeros (call it only once
    the gradients are no longer needed).  Returns GB/s for each: bytes per
    launch over the average launch time of `reps` launches (HIP events on
    the launch stream), after two untimed launches."""
    import ctypes
    import torch

    lib = ctypes.CDLL(BENCH_LIB)
    vp = ctypes.c_void_p
    lib.coat_bench_read_stream.restype = ctypes.c_int
    lib.coat_bench_read_stream.argtypes = [vp, ctypes.c_int64, ctypes.c_uint32, vp, vp]
    lib.coat_bench_write_stream.restype = ctypes.c_int
    lib.coat_bench_write_stream.argtypes = [vp, ctypes.c_int64, ctypes.c_uint32, vp]
    stream = torch.cuda.current_stream()
    sink = torch.zeros(256, dtype=torch.int32, device=shard.w.device)
    rbytes = shard.w.numel() * 4 // 16 * 16
    wbytes = shard.grad.numel() * 2 // 16 * 16

    def read():
        rc = lib.coat_bench_read_stream(shard.w.data_ptr(), rbytes, 0x9E3779B9,
                                        sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"coat_bench_read_stream returned {rc}")

    def write():
        rc = lib.coat_bench_write_stream(shard.grad.data_ptr(), wbytes, 0, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"coat_bench_write_stream returned {rc}")

    def rate(fn, nbytes):
        fn()
        fn()
        ev = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / reps
        return nbytes / (ms * 1e-3) / 1e9

    out = rate(read, rbytes), rate(write, wbytes)
    del sink
    return out


def time_shard_steps(shard, t, hp, stream, steps, per_launch=False):
    """`steps` timed steps of a warm shard (HIP events around each step, or
    around each launch): returns (per-step ms list, per-launch ms list)."""
    import torch
    n_calls = len(shard.calls)
    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(n_calls)] for _ in range(steps)]
    for k in range(steps):
        shard.step(t + 1 + k, **hp, stream=stream, events=events[k])
    torch.cuda.synchronize()
    step_ms = [events[k][0][0].elapsed_time(events[k][-1][1]) for k in range(steps)]
    launch_ms = [events[k][j][0].elapsed_time(events[k][j][1])
                 for k in range(steps) for j in range(n_calls)]
    return step_ms, launch_ms


def g_sweep(numels, hp, stream, rounds=3, steps=5):
    """The stress recipe at every group size over the same device buffers
    (one allocation sized for the smallest G, so that the physical pages
    behind the shard are the same for every G), in alternating rounds: per
    round and G, fresh state and weights, 3 untimed steps from zero state,
    one more untimed step, then `steps` timed steps."""
    import torch
    from adamw_coat_fp8_amd import inputs
    from adamw_coat_fp8_amd.shard import FP8AdamWShard

    stds = inputs.grad_stds(len(numels))
    base = FP8AdamWShard(numels, group_size=min(G_SWEEP), device="cuda")
    per = {G: [] for G in G_SWEEP}
    for r in range(rounds):
        for G in G_SWEEP:
            sh = FP8AdamWShard(numels, group_size=G, device="cuda", storage=base)
            inputs.fill_weights(sh)
            for t in (1, 2, 3):
                inputs.fill_gradients(sh, t, stds, "stress")
                sh.step(t, **hp, stream=stream)
            sh.step(4, **hp, stream=stream)
            ms, _ = time_shard_steps(sh, 4, hp, stream, steps)
            per[G].extend(ms)
        print(f"[bench] G sweep round {r} done", file=sys.stderr, flush=True)
    n = sum(numels)
    out = {}
    for G in G_SWEEP:
        med = sorted(per[G])[len(per[G]) // 2]
        nbytes = sum(algorithmic_bytes(x, G) for x in numels)
        out[str(G)] = {"Gparam_s": round(n / (med * 1e-3) / 1e9, 1),
                       "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "step_ms_median": round(med, 4), "steps_timed": len(per[G])}
    del base, sh
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


OTHER_WORKLOADS = (("olmo_1b", 100, 10), ("llama2_13b", 5, 10))   # (shape, warm-up, timed)


def time_workload(name, G, hp, stream, warm, steps):
    """One shape of the default gradient recipe on its own shard: `warm`
    untimed steps of state history (a fresh gradient each), then `steps`
    timed steps (HIP events around each step); median step time."""
    import torch
    from adamw_coat_fp8_amd import inputs
    from adamw_coat_fp8_amd.shard import FP8AdamWShard

    specs = inputs.workload_specs(name)
    numels = [x.numel for x in specs]
    stds = inputs.grad_stds(len(specs))
    sh = FP8AdamWShard(numels, group_size=G, device="cuda")
    inputs.fill_weights(sh)
    for t in range(1, warm + 1):
        inputs.fill_gradients(sh, t, stds)
        sh.step(t, **hp, stream=stream)
    torch.cuda.synchronize()
    ms, _ = time_shard_steps(sh, warm, hp, stream, steps)
    med = sorted(ms)[len(ms) // 2]
    n = sum(numels)
    nbytes = sum(algorithmic_bytes(x, G) for x in numels)
    del sh
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(f"[bench] {name}: {n / (med * 1e-3) / 1e9:.1f} Gparam/s", file=sys.stderr, flush=True)
    return {"params": n, "tensors": len(specs), "warmup": warm, "steps_timed": steps,
            "Gparam_s": round(n / (med * 1e-3) / 1e9, 1),
            "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_ms_median": round(med, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the step is shard-local and would run unchanged on each GPU's shard.",
              file=sys.stderr)
        sys.exit(2)
    if args.path == "act_quant":
        return bench_act(args)
    if args.path == "gemm_group_quant":
        return bench_gemm(args)
    if args.path == "codec":
        return bench_codec(args)
    return bench_step(args)


def bench_step(args):
    import torch
    from adamw_coat_fp8_amd import coat, inputs
    from adamw_coat_fp8_amd.shard import FP8AdamWShard

    G = args.group_size
    hp = dict(inputs.DEFAULT_HPARAMS)
    specs = inputs.workload_specs(args.workload)
    numels = [s.numel for s in specs]
    n_params = sum(numels)
    print(f"[bench] workload {args.workload}: {len(specs)} tensors, {n_params} params, "
          f"G={G}", file=sys.stderr, flush=True)
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    if args.g_sweep_only:
        print(json.dumps({"g_sweep": g_sweep(numels, hp, stream)}), flush=True)
        return
    shard = FP8AdamWShard(numels, group_size=G, device="cuda")
    stds = inputs.grad_stds(len(specs))
    inputs.fill_weights(shard)
    if args.ceiling_only:
        inputs.fill_gradients(shard, 1, stds)
        gbps, ms, nbytes = mix_ceiling(shard, max(args.steps, 2))
        print(f"[bench] math-free copy: avg launch {ms:.4f} ms", file=sys.stderr, flush=True)
        read_gbps, write_gbps = stream_ceilings(shard, max(args.steps, 2))
        print(f"[bench] read-only stream {read_gbps:.1f} GB/s, write-only stream "
              f"{write_gbps:.1f} GB/s", file=sys.stderr, flush=True)
        if args.copy_probe:
            copy_probe()
        print(json.dumps({"mix_ceiling_GBps": round(gbps, 1), "avg_launch_ms": round(ms, 4),
                          "bytes_per_launch": nbytes, "read_stream_GBps": round(read_gbps, 1),
                          "write_stream_GBps": round(write_gbps, 1)}), flush=True)
        return
    call_lists = shard.calls
    call_bytes = [sum(algorithmic_bytes(numels[i], G) for i in c) for c in shard.call_indices]

    def step(t, events=None):
        shard.step(t, **hp, stream=stream, events=events)

    t = 0
    for w in range(args.warmup):
        t += 1
        inputs.fill_gradients(shard, t, stds)
        step(t)
        torch.cuda.synchronize()
        print(f"[bench] warm-up step {t} done", file=sys.stderr, flush=True)
    if args.warmup == 0:
        inputs.fill_gradients(shard, 1, stds)
    torch.cuda.synchronize()

    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in call_lists] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        t += 1
        step(t, events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    launch_ms = [[events[k][j][0].elapsed_time(events[k][j][1]) for j in range(len(call_lists))]
                 for k in range(args.steps)]
    step_ms = sorted(events[k][0][0].elapsed_time(events[k][-1][1]) for k in range(args.steps))
    avg_launch_ms = sum(sum(r) for r in launch_ms) / (args.steps * len(call_lists))
    bytes_per_launch = sum(call_bytes) / len(call_lists)
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    print(f"[bench] {args.steps} timed steps: {ms_per_step:.3f} ms/step, "
          f"{len(call_lists)} launches/step, avg launch {avg_launch_ms:.3f} ms",
          file=sys.stderr, flush=True)

    ceiling_gbps, ceiling_ms, _ = mix_ceiling(shard)
    print(f"[bench] math-free copy of the step's traffic: {ceiling_gbps:.1f} GB/s "
          f"({ceiling_ms:.3f} ms per launch over the whole shard)", file=sys.stderr, flush=True)
    read_gbps, write_gbps = stream_ceilings(shard)     # overwrites the gradients: steps are done
    print(f"[bench] plain streams on the same shard: read-only {read_gbps:.1f} GB/s, "
          f"write-only {write_gbps:.1f} GB/s", file=sys.stderr, flush=True)
    if args.copy_probe:
        copy_probe()

    per_alloc = []
    if args.allocations > 1:
        per_alloc.append(round(n_params / (step_ms[len(step_ms) // 2] * 1e-3) / 1e9, 1))
        for r in range(1, args.allocations):
            del shard
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            shard = FP8AdamWShard(numels, group_size=G, device="cuda")
            inputs.fill_weights(shard)
            inputs.fill_gradients(shard, 1, stds)
            for tt in (1, 2, 3):
                shard.step(tt, **hp, stream=stream)
            ms, _ = time_shard_steps(shard, 3, hp, stream, args.steps)
            per_alloc.append(round(n_params / (sorted(ms)[len(ms) // 2] * 1e-3) / 1e9, 1))
            print(f"[bench] allocation {r}: {per_alloc[-1]} Gparam/s", file=sys.stderr, flush=True)

    traffic = traffic_from_profile(bytes_per_launch)
    value = n_params / (ms_per_step * 1e-3) / 1e9
    ceiling = copy_ceiling_gbps()
    total_bytes = sum(call_bytes)
    sweep = None
    others = {}
    if not (args.no_g_sweep and args.no_other_workloads):
        del shard
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if not args.no_other_workloads and args.workload == "llama2_7b":
        for name, warm, steps in OTHER_WORKLOADS:
            others[name] = time_workload(name, G, hp, stream, warm, steps)
    if not args.no_g_sweep:
        print("[bench] stress recipe, group-size sweep ...", file=sys.stderr, flush=True)
        sweep = g_sweep(numels, hp, stream)
    rec = {
        "metric": "Gparam/s per fused FP8-AdamW step + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(value, 3),
        "unit": "Gparam/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {len(specs)} tensors, {n_params} params, FP32 "
                        f"master weights, BF16 grads, E4M3 m/v with per-group FP32 scale and k",
            "group_size": G,
            "hparams": hp,
            "step_hbm_GBps": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
            "step_frac_of_peak": round(total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": total_bytes,
            "launches_per_step": len(call_lists),
            "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
            "step_ms_min": round(step_ms[0], 4),
            "mix_ceiling_GBps": round(ceiling_gbps, 1),
            "frac_of_mix_ceiling": round(achieved / ceiling_gbps, 4),
            "read_only_stream_GBps": round(read_gbps, 1),
            "write_only_stream_GBps": round(write_gbps, 1),
            # the step's bytes if its reads ran at the read-only rate and its
            # writes at the write-only rate, one after the other (no mixing)
            "separate_streams_bound_GBps": round(separate_streams_gbps(G, read_gbps, write_gbps), 1),
            "copy_ceiling_GBps": round(ceiling, 1),
            "kernel_frac_of_copy_ceiling": round(achieved / ceiling, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": f"adamw_fp8_step_kernel<{G}>",
            "bytes_per_launch": int(bytes_per_launch),
            "avg_launch_ms": round(avg_launch_ms, 4),
        },
    }
    if per_alloc:
        rec["config"]["per_allocation_Gparam_s"] = per_alloc
    if others:
        rec["config"]["other_workloads"] = others
    if sweep is not None:
        rec["config"]["stress_g_sweep"] = sweep
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on samples ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(specs, G, hp, args.cpu_sample)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
