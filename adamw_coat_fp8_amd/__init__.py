"""COAT FP8 AdamW step for MI355X (gfx950).

The work happens in ``libcoat_fp8.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/coat_fp8.h``).  ``adamw_coat_fp8_amd.coat`` holds
the thin ctypes binding; it is imported lazily so that ``inputs`` (seeded
synthetic data) can be used without loading the GPU library.
"""
import importlib

__all__ = ["coat", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
