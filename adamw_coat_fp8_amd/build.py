"""Build libcoat_fp8.so (gfx950 HIP kernels + C ABI) in the package folder,
and libcoat_bench.so, the benchmark's measurement kernels (the math-free copy
of the step's traffic and plain read-only and write-only streams; not part
of the library's C ABI).

hipcc cross-compiles for gfx950 without a GPU.  Packed FP32 instructions are
disabled (-packed-fp32-ops): the kernels are written as scalar float code.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("coat_fp8.hip", "coat_act.hip", "coat_gemm.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libcoat_fp8.so")
BENCH_SOURCES = [os.path.join(HERE, "csrc", f) for f in ("coat_mix_ceiling.hip", "coat_stream_ceiling.hip")]
BENCH_LIB = os.path.join(HERE, "libcoat_bench.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Werror", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(lib, sources, verbose, extra=()):
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-o", lib + ".tmp", *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False, extra=()) -> str:
    _compile(LIB, SOURCES, verbose, extra)
    _compile(BENCH_LIB, BENCH_SOURCES, verbose, extra)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
