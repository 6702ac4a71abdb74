"""Seeded synthetic inputs for the FP8 AdamW step: shapes, weights, gradients.

This module holds no part of the method's arithmetic.  It only draws random
numbers with torch (on whatever device the caller names) and lays them out the
way an optimizer shard sees them.  Both the GPU library's tests and the CPU
oracle's tests take their inputs from here; the oracle receives host copies.

Workloads (parameter lists shaped like the models the COAT paper trains; the
models themselves, their data and weights are not used):

* ``single_1m``   one 1024x1024 FP32 weight tensor (1,048,576 parameters)
* ``olmo_1b``     OLMo-1B-shaped list, 146 tensors, 1,176,832,000 parameters:
                  d=2048, 16 layers of 4 attention matrices 2048x2048, a SwiGLU
                  FFN with 3 matrices 2048x8192 / 8192x2048, two RMSNorm
                  vectors; 50304x2048 embedding; final norm
* ``llama2_7b``   Llama-2-7B-shaped list, 291 tensors, 6,738,415,616 parameters:
                  32 layers, d=4096, FFN 11008, vocab 32000, embedding and
                  untied LM head
* ``llama2_13b``  Llama-2-13B-shaped list, 363 tensors, 13,015,864,320
                  parameters: 40 layers, d=5120, FFN 13824, vocab 32000

Value recipe: w ~ N(0, 0.02); per-tensor gradient standard deviation drawn
log-uniformly in [1e-5, 1e-2] from seed 0 in tensor order; the step-t gradient
of tensor i is drawn from its own seed (1000 + t, i) in FP32 and rounded to
BF16 (round to nearest even).  The stress recipe replaces the Gaussian with a
Student-t (nu = 3) and plants exact zeros, single-nonzero groups, groups with
tiny magnitudes beside normal ones, and all-zero groups (see ``stress_gradient``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import torch

# Hyperparameters of the single-tensor workload (also the default elsewhere).
DEFAULT_HPARAMS = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                       weight_decay=0.1)
DEFAULT_GROUP_SIZE = 128
WEIGHT_STD = 0.02
GRAD_STD_RANGE = (1e-5, 1e-2)


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        return math.prod(self.shape)


def _decoder_layers(n_layers, d, ffn) -> List[TensorSpec]:
    out = []
    for i in range(n_layers):
        p = f"layers.{i}."
        out += [TensorSpec(p + "attn.q", (d, d)), TensorSpec(p + "attn.k", (d, d)),
                TensorSpec(p + "attn.v", (d, d)), TensorSpec(p + "attn.o", (d, d)),
                TensorSpec(p + "ffn.gate", (ffn, d)), TensorSpec(p + "ffn.up", (ffn, d)),
                TensorSpec(p + "ffn.down", (d, ffn)),
                TensorSpec(p + "attn_norm", (d,)), TensorSpec(p + "ffn_norm", (d,))]
    return out


def workload_specs(name: str) -> List[TensorSpec]:
    if name == "single_1m":
        return [TensorSpec("weight", (1024, 1024))]
    if name == "olmo_1b":
        return ([TensorSpec("embed", (50304, 2048))] + _decoder_layers(16, 2048, 8192)
                + [TensorSpec("final_norm", (2048,))])
    if name == "llama2_7b":
        return ([TensorSpec("embed", (32000, 4096))] + _decoder_layers(32, 4096, 11008)
                + [TensorSpec("final_norm", (4096,)), TensorSpec("lm_head", (32000, 4096))])
    if name == "llama2_13b":
        return ([TensorSpec("embed", (32000, 5120))] + _decoder_layers(40, 5120, 13824)
                + [TensorSpec("final_norm", (5120,)), TensorSpec("lm_head", (32000, 5120))])
    raise KeyError(f"unknown workload {name!r}")


WORKLOADS = ("single_1m", "olmo_1b", "llama2_7b", "llama2_13b")


def total_params(specs: Sequence[TensorSpec]) -> int:
    return sum(s.numel for s in specs)


def generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _seed(*parts: int) -> int:
    """Deterministic seed from a tuple of small integers."""
    s = 0x9E3779B97F4A7C15
    for p in parts:
        s = (s ^ (int(p) + 0x632BE59BD9B4E019 + (s << 6) + (s >> 2))) & 0xFFFFFFFFFFFFFFFF
    return s & 0x7FFFFFFFFFFFFFFF


def grad_stds(num_tensors: int, seed: int = 0) -> List[float]:
    """Per-tensor gradient std, log-uniform in GRAD_STD_RANGE (CPU draw, so the
    values are the same whatever device holds the tensors)."""
    gen = generator("cpu", seed)
    u = torch.rand(num_tensors, generator=gen, dtype=torch.float64)
    lo, hi = math.log(GRAD_STD_RANGE[0]), math.log(GRAD_STD_RANGE[1])
    return [math.exp(lo + (hi - lo) * float(x)) for x in u]


def weights(numel: int, tensor_index: int, device, seed: int = 0) -> torch.Tensor:
    gen = generator(device, _seed(seed, 17, tensor_index))
    return torch.randn(numel, generator=gen, device=device,
                       dtype=torch.float32) * WEIGHT_STD


def gaussian_gradient(numel: int, std: float, step: int, tensor_index: int,
                      device) -> torch.Tensor:
    """Step-`step` BF16 gradient of one tensor: N(0, std) in FP32, then RNE."""
    gen = generator(device, _seed(1000 + step, tensor_index))
    g = torch.randn(numel, generator=gen, device=device, dtype=torch.float32)
    return (g * std).to(torch.bfloat16)


def stress_gradient(numel: int, std: float, step: int, tensor_index: int,
                    device, group_size: int) -> torch.Tensor:
    """Stress recipe, per tensor:

    * values std * t_3 (Student-t, nu = 3), FP32 then BF16;
    * a fixed exact-zero mask (Bernoulli 0.05, seed 2), the same every step;
    * 1% of groups keep exactly one nonzero element (seed 3, fixed position);
    * 1% of groups hold magnitude 4.5e-15 on every fourth element, so their
      second moment (about 1e-30) sits beside normal values;
    * 1% of groups are zero throughout.
    Group membership is by consecutive ``group_size`` elements, the last group
    possibly short."""
    gen = generator(device, _seed(1000 + step, tensor_index, 5))
    z = torch.randn(numel, generator=gen, device=device, dtype=torch.float32)
    chi = torch.randn(3, numel, generator=gen, device=device, dtype=torch.float32)
    t3 = z / torch.sqrt((chi * chi).sum(0) / 3.0)
    g = t3 * std
    # fixed features: independent of the step
    fgen = generator(device, _seed(2, tensor_index))
    zero = torch.rand(numel, generator=fgen, device=device) < 0.05
    g = torch.where(zero, torch.zeros_like(g), g)
    ng = (numel + group_size - 1) // group_size
    sgen = generator(device, _seed(3, tensor_index))
    u = torch.rand(ng, generator=sgen, device=device)
    pos = torch.randint(0, 1 << 30, (ng,), generator=sgen, device=device)
    idx = torch.arange(numel, device=device)
    grp = idx // group_size
    within = idx - grp * group_size
    glen = torch.clamp(numel - grp * group_size, max=group_size)
    ug = u[grp]
    single = ug < 0.01
    keep = within == (pos[grp] % glen)
    sign = torch.where(t3 < 0, -1.0, 1.0)
    g = torch.where(single & ~keep, torch.zeros_like(g), g)
    g = torch.where(single & keep, sign * max(std, 1e-6), g)
    tiny = (ug >= 0.01) & (ug < 0.02) & (within % 4 == 0)
    g = torch.where(tiny, sign * 4.5e-15, g)
    allzero = (ug >= 0.02) & (ug < 0.03)
    g = torch.where(allzero, torch.zeros_like(g), g)
    return g.to(torch.bfloat16)


def gradient(numel: int, std: float, step: int, tensor_index: int, device,
             kind: str = "gaussian", group_size: int = DEFAULT_GROUP_SIZE):
    if kind == "gaussian":
        return gaussian_gradient(numel, std, step, tensor_index, device)
    if kind == "stress":
        return stress_gradient(numel, std, step, tensor_index, device, group_size)
    raise KeyError(kind)


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Raw uint16 view of a BF16 tensor (int16 storage reinterpreted)."""
    assert t.dtype == torch.bfloat16
    return t.view(torch.int16)


# ------------------------------------------------ filling a flat shard
# A "shard" is any object with flat device buffers `w` (float32) and `grad`
# (bfloat16) and per-tensor `element_range(i)` slices (see shard.py).

def fill_weights(shard, seed: int = 0):
    for i in range(len(shard.numels)):
        e = shard.element_range(i)
        shard.w[e].copy_(weights(shard.numels[i], i, shard.w.device, seed=seed))


def fill_moment_like(x: torch.Tensor, numels: Sequence[int], stds: Sequence[float]):
    """An FP32 first-moment-like state in one flat buffer: tensor i's slice is
    N(0, 0.1 * stds[i]) (the size of (1 - beta1) g), seed 1000 + i."""
    off = 0
    for i, (n, sd) in enumerate(zip(numels, stds)):
        x[off:off + n].normal_(0.0, 0.1 * sd, generator=generator(x.device, 1000 + i))
        off += n
    return x


def fill_gradients(shard, step: int, stds: Sequence[float], kind: str = "gaussian"):
    for i in range(len(shard.numels)):
        e = shard.element_range(i)
        shard.grad[e].copy_(gradient(shard.numels[i], stds[i], step, i, shard.grad.device,
                                     kind=kind, group_size=shard.group_size))


# ------------------------------------------------ activation matrices
# Inputs of the per-group activation quantizer: a row-major (tokens, channels)
# BF16 matrix, the output of a non-linear layer.

ACT_OUTLIER_FRACTION = 0.01          # channels with a large, fixed gain
ACT_OUTLIER_GAIN = (10.0, 100.0)     # log-uniform gain of those channels
ACT_TIE_MIDPOINTS = (17.0, 8.5, 19.0, 9.5, 248.0, 3.0 * 2.0 ** -10)


def activation(rows: int, cols: int, seed: int, device, kind: str = "llm",
               group_size: int = DEFAULT_GROUP_SIZE) -> torch.Tensor:
    """Seeded synthetic activation matrix, BF16 of shape (rows, cols).

    ``llm``: N(0, 1) per element times a per-channel gain that is 1 except on
    ACT_OUTLIER_FRACTION of the channels (log-uniform gain in ACT_OUTLIER_GAIN),
    the outlier-channel structure of transformer activations.

    ``stress`` adds, per 1 x group_size group of a row (a uniform draw picks
    the class): 2% all-zero; 2% a single nonzero; 2% magnitudes scaled by
    1e-39 (BF16 subnormals); 2% by 2^-110 (normal, below 2^-100); 2% by 1e30;
    4% tie groups (one element +-448 * s, the rest +-midpoints between
    neighbouring E4M3 values times s, with s = 2^e in half of them and
    s = 0.75 * 2^e, a group max that is not a power of two, in the other half;
    e in {-20, -7, 0, 10}; all exact in BF16); 2% with -0.0 on
    every other element; 2% wide groups (one element +-1e30, the rest N(0,1)
    times 1e-20 in half of them, whose scaled values underflow FP32, and times
    1e-5 in the other half, which scale to tiny normal FP32 values)."""
    if cols % group_size:
        raise ValueError("cols must be a multiple of group_size")
    gen = generator(device, _seed(seed, 31, rows, cols))
    x = torch.randn(rows, cols, generator=gen, device=device, dtype=torch.float32)
    cgen = generator(device, _seed(seed, 32, cols))
    outlier = torch.rand(cols, generator=cgen, device=device) < ACT_OUTLIER_FRACTION
    lo, hi = math.log(ACT_OUTLIER_GAIN[0]), math.log(ACT_OUTLIER_GAIN[1])
    gain = torch.exp(lo + (hi - lo) * torch.rand(cols, generator=cgen, device=device))
    x = x * torch.where(outlier, gain, torch.ones_like(gain))
    if kind == "llm":
        return x.to(torch.bfloat16)
    if kind != "stress":
        raise KeyError(kind)
    ng = cols // group_size
    sgen = generator(device, _seed(seed, 33, rows, cols, group_size))
    u = torch.rand(rows, ng, generator=sgen, device=device)
    u = u.repeat_interleave(group_size, dim=1)           # class of each element's group
    within = torch.arange(cols, device=device).remainder(group_size).expand(rows, cols)
    pick = torch.randint(0, group_size, (rows, ng), generator=sgen, device=device)
    lead = within == pick.repeat_interleave(group_size, dim=1)
    sign = torch.where(torch.rand(rows, cols, generator=sgen, device=device) < 0.5, -1.0, 1.0)
    e = torch.tensor([-20.0, -7.0, 0.0, 10.0], device=device)
    escale = torch.exp2(e[torch.randint(0, 4, (rows, ng), generator=sgen, device=device)])
    escale = escale.repeat_interleave(group_size, dim=1)
    mids = torch.tensor(ACT_TIE_MIDPOINTS, device=device)
    mid = mids[torch.randint(0, len(ACT_TIE_MIDPOINTS), (rows, cols), generator=sgen,
                             device=device)]
    zero = torch.zeros_like(x)
    x = torch.where(u < 0.02, zero, x)
    x = torch.where((u >= 0.02) & (u < 0.04) & ~lead, zero, x)
    x = torch.where((u >= 0.04) & (u < 0.06), x * 1e-39, x)
    x = torch.where((u >= 0.06) & (u < 0.08), x * 2.0 ** -110, x)
    x = torch.where((u >= 0.08) & (u < 0.10), x * 1e30, x)
    tie = (u >= 0.10) & (u < 0.14)
    tscale = escale * torch.where(u < 0.12, 1.0, 0.75)
    x = torch.where(tie, sign * tscale * torch.where(lead, 448.0, mid), x)
    negz = (u >= 0.14) & (u < 0.16) & (within % 2 == 1)
    x = torch.where(negz, torch.full_like(x, -0.0), x)
    wide = (u >= 0.16) & (u < 0.18)
    rest = torch.where(u < 0.17, 1e-20, 1e-5)
    x = torch.where(wide, torch.where(lead, sign * 1e30, x * rest), x)
    return x.to(torch.bfloat16)


# ------------------------------------------------ FP8 linear-layer operands
# Inputs of the group-scaled FP8 linear layer: an activation A (M x K) and a
# weight B (N x K), each already quantized per tensor to E4M3 codes.

E4M3_SMALL_INTS = (0x00, 0x38, 0x40, 0x44, 0x48, 0x4C, 0x50)   # 0, 1, 2, 3, 4, 6, 8


def fp8_operands(M: int, N: int, K: int, seed: int, device, kind: str = "llm"):
    """Returns (a_codes uint8 M x K, b_codes uint8 N x K, a_scale, b_scale).

    ``llm``: A is ``activation(M, K)`` (N(0, 1) with outlier channels) and B
    is N(0, 0.02); each is scaled by max|x| / 448 and cast to E4M3 (nearest
    even), the per-tensor quantization of linear-layer inputs.

    ``exact``: codes of the integers 0, +-1, +-2, +-3, +-4, +-6, +-8 with
    scales 2^-3 and 2^1, so every product sum is an integer below 2^24 for
    K <= 2^18 and C is exact in FP32 whatever the summation order."""
    if kind == "exact":
        gen = generator(device, _seed(seed, 41, M, N, K))
        table = torch.tensor(E4M3_SMALL_INTS, dtype=torch.uint8, device=device)
        def draw(rows):
            idx = torch.randint(0, len(E4M3_SMALL_INTS), (rows, K), generator=gen, device=device)
            sign = torch.randint(0, 2, (rows, K), generator=gen, device=device, dtype=torch.uint8)
            return table[idx] | (sign << 7) * (table[idx] != 0)
        return draw(M).contiguous(), draw(N).contiguous(), 0.125, 2.0
    if kind != "llm":
        raise KeyError(kind)
    x = activation(M, K, seed, device, "llm", 16).float() if K % 16 == 0 else None
    if x is None:
        raise ValueError("K must be a multiple of 16")
    w = torch.randn(N, K, generator=generator(device, _seed(seed, 42, N, K)), device=device,
                    dtype=torch.float32) * WEIGHT_STD
    def quant(t):
        s = float(t.abs().max()) / 448.0
        if s == 0.0:
            s = 1.0
        return (t / s).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), s
    a, sa = quant(x)
    b, sb = quant(w)
    return a, b, sa, sb
