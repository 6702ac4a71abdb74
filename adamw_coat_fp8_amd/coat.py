"""ctypes binding of libcoat_fp8.so (declared in include/coat_fp8.h).

Argument marshalling only: every step of the optimizer runs in the library's
HIP kernels.  Marshalling includes what the C ABI cannot see through raw
pointers: each buffer's dtype, contiguity, size and device are checked
before the call (ValueError).  torch tensors are accepted for convenience (their device pointers
and torch's current HIP stream are passed through); the library never sees a
torch type.  Importing this module loads the library and fails loudly if it is
missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoat_fp8.so")

ABI_VERSION = 1
GROUP_SIZES = (16, 32, 64, 128)

COAT_OK = 0
COAT_ERR_NULL_POINTER = 1
COAT_ERR_INVALID_VALUE = 2
COAT_ERR_GROUP_SIZE = 3
COAT_ERR_MISALIGNED = 4
COAT_ERR_HIP = 5

EXPORTED_SYMBOLS = (
    "coat_adamw_fp8_step", "coat_fp8_expand_quantize", "coat_fp8_dequantize_expand",
    "coat_e4m3_encode", "coat_e4m3_decode", "coat_fp8_quantize_act",
    "coat_fp8_gemm_group_quant", "coat_fp8_gemm_bf16", "coat_status_string",
    "coat_last_hip_error", "coat_abi_version",
)


class CoatError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class FP8State(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("k", ctypes.c_void_p)]


class AdamWTensor(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("m", FP8State), ("v", FP8State), ("n", ctypes.c_int64)]


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float),
                ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64),
                ("group_size", ctypes.c_int32)]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -c \"import "
            f"__graft_entry__; __graft_entry__.build()\"` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.coat_adamw_fp8_step.restype = ctypes.c_int
    lib.coat_adamw_fp8_step.argtypes = [vp, i32, ctypes.POINTER(AdamWHParams), vp]
    lib.coat_fp8_expand_quantize.restype = ctypes.c_int
    lib.coat_fp8_expand_quantize.argtypes = [vp, i64, i32, FP8State, vp]
    lib.coat_fp8_dequantize_expand.restype = ctypes.c_int
    lib.coat_fp8_dequantize_expand.argtypes = [vp, vp, vp, i64, i32, vp, vp]
    lib.coat_e4m3_encode.restype = ctypes.c_int
    lib.coat_e4m3_encode.argtypes = [vp, i64, vp, vp]
    lib.coat_e4m3_decode.restype = ctypes.c_int
    lib.coat_e4m3_decode.argtypes = [vp, i64, vp, vp]
    lib.coat_fp8_quantize_act.restype = ctypes.c_int
    lib.coat_fp8_quantize_act.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
    f32 = ctypes.c_float
    lib.coat_fp8_gemm_group_quant.restype = ctypes.c_int
    lib.coat_fp8_gemm_group_quant.argtypes = [vp, vp, f32, f32, i64, i64, i64, i32, vp, vp, vp, vp]
    lib.coat_fp8_gemm_bf16.restype = ctypes.c_int
    lib.coat_fp8_gemm_bf16.argtypes = [vp, vp, f32, f32, i64, i64, i64, vp, vp]
    lib.coat_status_string.restype = ctypes.c_char_p
    lib.coat_status_string.argtypes = [ctypes.c_int]
    lib.coat_last_hip_error.restype = ctypes.c_char_p
    lib.coat_last_hip_error.argtypes = []
    lib.coat_abi_version.restype = ctypes.c_int32
    lib.coat_abi_version.argtypes = []
    if lib.coat_abi_version() != ABI_VERSION:
        raise ImportError(f"{path}: ABI version {lib.coat_abi_version()}, "
                          f"binding expects {ABI_VERSION}")
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.coat_status_string(status).decode()


def _check(status: int):
    if status != COAT_OK:
        msg = status_string(status)
        if status == COAT_ERR_HIP:
            msg += ": " + lib.coat_last_hip_error().decode()
        raise CoatError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# dtypes accepted for each kind of buffer (bit-pattern views are fine)
CODE_DTYPES = (torch.uint8, torch.int8, torch.float8_e4m3fn)
BF16_DTYPES = (torch.bfloat16, torch.int16)
F32_DTYPES = (torch.float32,)


def _need(t: torch.Tensor, name: str, dtypes, min_numel: int):
    """Marshalling checks the C ABI cannot make: the kernels read and write
    through raw device pointers, so a buffer of the wrong type, layout, size
    or device would be accessed out of bounds.  Raises ValueError."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")


def _on_device(**tensors):
    """Every given buffer is HIP device memory on the current device, where
    the library launches its kernels (after the type and size checks)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP device) tensor, not {t.device}")
        if dev is None:
            dev = torch.cuda.current_device()
        if t.get_device() != dev:
            raise ValueError(f"{name} is on cuda:{t.get_device()}, but the current device "
                             f"is cuda:{dev}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        # torch's current stream on the current device, as a raw handle: this
        # query costs about 0.1 us per call, torch.cuda.current_stream() about
        # 3 us, as long as a small kernel
        return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def num_groups(n: int, group_size: int) -> int:
    return (n + group_size - 1) // group_size


@dataclass(frozen=True)
class QuantState:
    """One FP8 moment on the device: codes uint8[n], scale/k float32[ng]."""
    codes: torch.Tensor
    scale: torch.Tensor
    k: torch.Tensor

    @classmethod
    def zeros(cls, n: int, group_size: int, device="cuda") -> "QuantState":
        ng = num_groups(n, group_size)
        return cls(torch.zeros(n, dtype=torch.uint8, device=device),
                   torch.zeros(ng, dtype=torch.float32, device=device),
                   torch.zeros(ng, dtype=torch.float32, device=device))

    def as_c(self) -> FP8State:
        return FP8State(_ptr(self.codes), _ptr(self.scale), _ptr(self.k))

    def check(self, n: int, group_size: int, name: str):
        _need(self.codes, f"{name}.codes", CODE_DTYPES, n)
        _need(self.scale, f"{name}.scale", F32_DTYPES, num_groups(n, group_size))
        _need(self.k, f"{name}.k", F32_DTYPES, num_groups(n, group_size))

    def check_device(self, name: str):
        _on_device(**{f"{name}.codes": self.codes, f"{name}.scale": self.scale,
                      f"{name}.k": self.k})


@dataclass(frozen=True)
class ParamSlot:
    """One tensor of an optimizer shard: FP32 weights, BF16 gradient, m, v.
    Frozen, like QuantState: a TensorList copies the tensors' device pointers
    once, so a slot's tensors cannot be swapped after it is built (build a new
    slot, e.g. with dataclasses.replace, and a new TensorList instead)."""
    w: torch.Tensor
    grad: torch.Tensor
    m: QuantState
    v: QuantState

    def as_c(self) -> AdamWTensor:
        return AdamWTensor(_ptr(self.w), _ptr(self.grad), self.m.as_c(),
                           self.v.as_c(), self.w.numel())

    def check(self, group_size: int, name: str = "slot"):
        n = self.w.numel()
        _need(self.w, f"{name}.w", F32_DTYPES, n)
        _need(self.grad, f"{name}.grad", BF16_DTYPES, n)
        self.m.check(n, group_size, f"{name}.m")
        self.v.check(n, group_size, f"{name}.v")
        _on_device(**{f"{name}.w": self.w, f"{name}.grad": self.grad})
        self.m.check_device(f"{name}.m")
        self.v.check_device(f"{name}.v")


class TensorList:
    """Marshalled descriptor array for coat_adamw_fp8_step, built once and
    reused across steps (the pointers stay valid while the tensors live: the
    list holds the slots, and slots are frozen).  The buffer checks run once
    per group size and again whenever the current device differs from the
    one they ran on (the library launches on the current device)."""

    def __init__(self, slots: Sequence[ParamSlot]):
        self.slots = list(slots)
        self.array = (AdamWTensor * max(1, len(self.slots)))(
            *[s.as_c() for s in self.slots])
        self._checked = set()   # (group size, device index) the slots have been checked for

    def check(self, group_size: int):
        key = (group_size, torch.cuda.current_device() if torch.cuda.is_initialized() else -1)
        if key not in self._checked:
            for i, slot in enumerate(self.slots):
                slot.check(group_size, f"tensors[{i}]")
            self._checked.add(key)

    def __len__(self):
        return len(self.slots)


def adamw_fp8_step(tensors, *, lr: float, beta1: float, beta2: float, eps: float,
                   weight_decay: float, step: int, group_size: int = 128, stream=None):
    """One fused FP8 AdamW step over `tensors` (a TensorList or a sequence of
    ParamSlot).  Enqueued on `stream` (torch's current stream by default)."""
    tl = tensors if isinstance(tensors, TensorList) else TensorList(tensors)
    tl.check(group_size)
    hp = AdamWHParams(lr, beta1, beta2, eps, weight_decay, step, group_size)
    _check(lib.coat_adamw_fp8_step(ctypes.addressof(tl.array), len(tl),
                                   ctypes.byref(hp), _stream(stream)))


def adamw_fp8_step_raw(array_ptr: Optional[int], num_tensors: int, hp: AdamWHParams,
                       stream=None) -> int:
    """Direct call with a caller-built descriptor array; returns the status."""
    return lib.coat_adamw_fp8_step(array_ptr, num_tensors,
                                   ctypes.byref(hp) if hp is not None else None,
                                   _stream(stream))


def expand_quantize(x: torch.Tensor, out: QuantState, group_size: int = 128, stream=None):
    _need(x, "x", F32_DTYPES, 0)
    out.check(x.numel(), group_size, "out")
    _on_device(x=x)
    out.check_device("out")
    _check(lib.coat_fp8_expand_quantize(_ptr(x), x.numel(), group_size, out.as_c(),
                                        _stream(stream)))


def dequantize_expand(state: QuantState, out: torch.Tensor, group_size: int = 128,
                      stream=None):
    state.check(state.codes.numel(), group_size, "state")
    _need(out, "out", F32_DTYPES, state.codes.numel())
    state.check_device("state")
    _on_device(out=out)
    _check(lib.coat_fp8_dequantize_expand(
        _ptr(state.codes), _ptr(state.scale), _ptr(state.k), state.codes.numel(),
        group_size, _ptr(out), _stream(stream)))


def e4m3_encode(x: torch.Tensor, codes: torch.Tensor, stream=None):
    _need(x, "x", F32_DTYPES, 0)
    _need(codes, "codes", CODE_DTYPES, x.numel())
    _on_device(x=x, codes=codes)
    _check(lib.coat_e4m3_encode(_ptr(x), x.numel(), _ptr(codes), _stream(stream)))


def e4m3_decode(codes: torch.Tensor, x: torch.Tensor, stream=None):
    _need(codes, "codes", CODE_DTYPES, 0)
    _need(x, "x", F32_DTYPES, codes.numel())
    _on_device(codes=codes, x=x)
    _check(lib.coat_e4m3_decode(_ptr(codes), codes.numel(), _ptr(x), _stream(stream)))


def quantize_act(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                 codes_t: Optional[torch.Tensor] = None, group_size: int = 128,
                 stream=None):
    """Per-group (1 x group_size) E4M3 quantization of a 2-D BF16 matrix x into
    codes (same shape, uint8), scales (rows x cols/group_size, float32) and,
    if given, codes_t (cols x rows, uint8)."""
    if x.dim() != 2:
        raise ValueError("quantize_act expects a 2-D (rows, cols) tensor")
    rows, cols = x.shape
    _need(x, "x", BF16_DTYPES, 0)
    _need(codes, "codes", CODE_DTYPES, rows * cols)
    _need(scales, "scales", F32_DTYPES, rows * (cols // max(group_size, 1)))
    if codes_t is not None:
        _need(codes_t, "codes_t", CODE_DTYPES, rows * cols)
    _on_device(x=x, codes=codes, scales=scales, codes_t=codes_t)
    _check(lib.coat_fp8_quantize_act(_ptr(x), rows, cols, group_size, _ptr(codes),
                                     _ptr(scales), _ptr(codes_t), _stream(stream)))


def gemm_group_quant(a: torch.Tensor, b: torch.Tensor, a_scale: float, b_scale: float,
                     codes: torch.Tensor, scales: torch.Tensor, group_size: int = 128,
                     c_f32: Optional[torch.Tensor] = None, stream=None):
    """C = a_scale * b_scale * a @ b.T from E4M3 codes a (M x K) and b (N x K),
    quantized per 1 x group_size group of each row into codes (M x N) and
    scales (M x N/group_size); optionally also writes C in FP32."""
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    _need(a, "a", CODE_DTYPES, 0)
    _need(b, "b", CODE_DTYPES, 0)
    _need(codes, "codes", CODE_DTYPES, M * N)
    _need(scales, "scales", F32_DTYPES, M * (N // max(group_size, 1)))
    if c_f32 is not None:
        _need(c_f32, "c_f32", F32_DTYPES, M * N)
    _on_device(a=a, b=b, codes=codes, scales=scales, c_f32=c_f32)
    _check(lib.coat_fp8_gemm_group_quant(_ptr(a), _ptr(b), a_scale, b_scale, M, N, K,
                                         group_size, _ptr(codes), _ptr(scales), _ptr(c_f32),
                                         _stream(stream)))


def gemm_bf16(a: torch.Tensor, b: torch.Tensor, a_scale: float, b_scale: float,
              c_bf16: torch.Tensor, stream=None):
    """C = a_scale * b_scale * a @ b.T from E4M3 codes, rounded to BF16."""
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    _need(a, "a", CODE_DTYPES, 0)
    _need(b, "b", CODE_DTYPES, 0)
    _need(c_bf16, "c_bf16", BF16_DTYPES, M * N)
    _on_device(a=a, b=b, c_bf16=c_bf16)
    _check(lib.coat_fp8_gemm_bf16(_ptr(a), _ptr(b), a_scale, b_scale, M, N, K, _ptr(c_bf16),
                                  _stream(stream)))
