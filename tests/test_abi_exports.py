"""CPU checks of the C-ABI library: it loads, exports every function that
include/coat_fp8.h declares, reports its ABI version, and the ctypes structs
of the Python binding have the C layout (checked against a C program compiled
from the header).  No compute call is made: there is no GPU here."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coat_fp8.h")


def _ensure_built():
    from adamw_coat_fp8_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    return build.LIB


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coat_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ("coat_adamw_fp8_step", "coat_fp8_expand_quantize",
                 "coat_fp8_dequantize_expand"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    path = _ensure_built()
    lib = ctypes.CDLL(path)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (coat_[a-z0-9_]+)", out))
    assert set(declared_functions()) <= exported


def test_binding_symbol_list_matches_header():
    from adamw_coat_fp8_amd import coat
    assert sorted(coat.EXPORTED_SYMBOLS) == declared_functions()
    assert coat.lib.coat_abi_version() == coat.ABI_VERSION
    assert coat.status_string(coat.COAT_ERR_GROUP_SIZE).startswith("COAT_ERR_GROUP_SIZE")
    assert coat.lib.coat_last_hip_error() == b""


def test_ctypes_layout_matches_c():
    from adamw_coat_fp8_amd import coat
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "coat_fp8.h"
int main(void) {
  printf("%zu %zu %zu\n", sizeof(coat_fp8_state_t), sizeof(coat_adamw_tensor_t),
         sizeof(coat_adamw_hparams_t));
  printf("%zu %zu %zu %zu\n", offsetof(coat_adamw_tensor_t, m), offsetof(coat_adamw_tensor_t, v),
         offsetof(coat_adamw_tensor_t, n), offsetof(coat_adamw_hparams_t, step));
  printf("%zu\n", offsetof(coat_adamw_hparams_t, group_size));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    T, H = coat.AdamWTensor, coat.AdamWHParams
    assert vals == [ctypes.sizeof(coat.FP8State), ctypes.sizeof(T), ctypes.sizeof(H),
                    T.m.offset, T.v.offset, T.n.offset, H.step.offset, H.group_size.offset]
