"""An optimizer shard laid out for the fused FP8 AdamW step.

Each state stream lives in ONE flat device buffer (w FP32, grad BF16, m and v
codes u8, per-group scale and k FP32), and every parameter tensor is a view at
an offset rounded up to a multiple of 16 elements, so every tensor meets the
library's 16-byte alignment rule and the whole shard is one allocation per
stream: the FSDP flat-parameter layout, with groups kept inside tensors.
This module allocates and marshals; the arithmetic is in libcoat_fp8.so.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import torch

from . import coat

ALIGN = 16  # elements
MAX_TENSORS_PER_CALL = 40  # the library's per-launch descriptor capacity


def balanced_calls(numels: Sequence[int], limit: int = MAX_TENSORS_PER_CALL) -> List[List[int]]:
    """Split a tensor list into contiguous runs of at most `limit` tensors with
    roughly equal parameter counts; each run is one library call, which the
    library issues as exactly one kernel launch."""
    k = max(1, math.ceil(len(numels) / limit))
    target = sum(numels) / k
    out, cur, acc = [], [], 0
    for i, n in enumerate(numels):
        if cur and (len(cur) == limit or acc + n > 1.05 * target):
            out.append(cur)
            cur, acc = [], 0
        cur.append(i)
        acc += n
    if cur:
        out.append(cur)
    return out


def _round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


class FP8AdamWShard:
    """`storage`, if given, is another shard of the same tensor list whose
    flat buffers this one takes as its own (views of their first elements):
    a shard for another group size over the same memory.  Its per-group
    arrays must be at least as long (the smallest group size has the
    longest)."""

    def __init__(self, numels: Sequence[int], group_size: int = 128, device="cuda",
                 storage: "FP8AdamWShard" = None):
        if group_size not in coat.GROUP_SIZES:
            raise ValueError(f"group_size must be one of {coat.GROUP_SIZES}")
        self.numels = [int(n) for n in numels]
        self.group_size = group_size
        self.device = torch.device(device)
        self.offsets: List[int] = []
        self.goffsets: List[int] = []
        off = goff = 0
        for n in self.numels:
            self.offsets.append(off)
            self.goffsets.append(goff)
            off = _round_up(off + n, ALIGN)
            goff += coat.num_groups(n, group_size)
        self.total_elems = off
        self.total_groups = goff
        dev = self.device
        if storage is not None:
            if storage.total_elems < off or storage.total_groups < goff:
                raise ValueError("storage shard too small for this tensor list and group size")
            self.w = storage.w[:off]
            self.grad = storage.grad[:off]
            self.m_codes = storage.m_codes[:off]
            self.v_codes = storage.v_codes[:off]
            self.m_scale = storage.m_scale[:goff]
            self.m_k = storage.m_k[:goff]
            self.v_scale = storage.v_scale[:goff]
            self.v_k = storage.v_k[:goff]
            self.reset_state()
        else:
            self.w = torch.zeros(off, dtype=torch.float32, device=dev)
            self.grad = torch.zeros(off, dtype=torch.bfloat16, device=dev)
            self.m_codes = torch.zeros(off, dtype=torch.uint8, device=dev)
            self.v_codes = torch.zeros(off, dtype=torch.uint8, device=dev)
            self.m_scale = torch.zeros(goff, dtype=torch.float32, device=dev)
            self.m_k = torch.zeros(goff, dtype=torch.float32, device=dev)
            self.v_scale = torch.zeros(goff, dtype=torch.float32, device=dev)
            self.v_k = torch.zeros(goff, dtype=torch.float32, device=dev)
        self.slots = [self.slot(i) for i in range(len(self.numels))]
        self.call_indices = balanced_calls(self.numels)
        self.calls = [coat.TensorList([self.slots[i] for i in c]) for c in self.call_indices]

    def reset_state(self):
        """Fresh optimizer state: every moment code, scale and k zero (an
        all-zero group), as the library defines a new state."""
        for t in (self.m_codes, self.v_codes, self.m_scale, self.m_k, self.v_scale, self.v_k):
            t.zero_()

    @property
    def num_params(self) -> int:
        return sum(self.numels)

    def _views(self, i: int):
        o, n = self.offsets[i], self.numels[i]
        go, ng = self.goffsets[i], coat.num_groups(self.numels[i], self.group_size)
        return slice(o, o + n), slice(go, go + ng)

    def slot(self, i: int) -> coat.ParamSlot:
        e, g = self._views(i)
        return coat.ParamSlot(
            self.w[e], self.grad[e],
            coat.QuantState(self.m_codes[e], self.m_scale[g], self.m_k[g]),
            coat.QuantState(self.v_codes[e], self.v_scale[g], self.v_k[g]))

    def group_range(self, i: int) -> slice:
        return self._views(i)[1]

    def element_range(self, i: int) -> slice:
        return self._views(i)[0]

    def step(self, step: int, *, lr: float, beta1: float, beta2: float, eps: float,
             weight_decay: float, stream=None, events=None):
        """One fused step over the whole shard: one library call (= one
        launch) per balanced run of tensors.  `events`, if given, is a list of
        (start, end) torch.cuda.Event pairs, one per call, recorded on
        `stream` around each launch."""
        if stream is None:
            stream = torch.cuda.current_stream()
        for j, tl in enumerate(self.calls):
            if events is not None:
                events[j][0].record(stream)
            coat.adamw_fp8_step(tl, lr=lr, beta1=beta1, beta2=beta2, eps=eps,
                                weight_decay=weight_decay, step=step,
                                group_size=self.group_size, stream=stream)
            if events is not None:
                events[j][1].record(stream)

    def state_bytes(self) -> int:
        """Bytes of optimizer state held per shard (codes + scale + k)."""
        return 2 * self.total_elems + 4 * 4 * self.total_groups
