"""A small least-squares training problem for trajectory tests.

min_w 0.5 * mean((X w - y)^2) with X a seeded Gaussian matrix whose columns
carry a log-uniform scale in [1e-2, 10] (so per-coordinate gradient and
second-moment magnitudes spread over several decades, as across a layer's
weights), y = X w* and w* ~ N(0, 0.02).  The gradient is evaluated in float64
from the current weights and rounded to BF16, the precision the optimizer step
takes its gradients in.  Holds no arithmetic of the optimizer itself.
"""
import contextlib

import numpy as np
import torch

from adamw_coat_fp8_amd import inputs


class LeastSquares:
    def __init__(self, d=4096, samples=512, seed=0):
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((samples, d)) / np.sqrt(d)
        self.x = x * np.exp(rng.uniform(np.log(1e-2), np.log(10.0), d))
        self.y = self.x @ (rng.standard_normal(d) * 0.02)
        self.d = d

    def loss(self, w):
        r = self.x @ np.asarray(w, np.float64) - self.y
        return 0.5 * float(np.mean(r * r))

    def grad_bf16(self, w) -> torch.Tensor:
        r = self.x @ np.asarray(w, np.float64) - self.y
        g = torch.from_numpy((self.x.T @ r / len(self.y)).astype(np.float32))
        return g.to(torch.bfloat16)

    def grad_bits(self, w) -> np.ndarray:
        return inputs.bf16_bits(self.grad_bf16(w)).numpy().view(np.uint16).copy()


def torch_adamw_trajectory(prob, steps, hp):
    """Weights after each step of torch.optim.AdamW (FP32 moments) from w = 0,
    fed the same BF16-rounded gradients."""
    p = torch.nn.Parameter(torch.zeros(prob.d, dtype=torch.float32))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False, fused=False)
    out = []
    with one_torch_thread():
        for _ in range(steps):
            p.grad = prob.grad_bf16(p.detach().numpy()).float()
            opt.step()
            out.append(p.detach().numpy().copy())
    return np.array(out)


@contextlib.contextmanager
def one_torch_thread():
    """torch's and numpy's thread pools contend on these small alternating
    operations (a 30x slowdown); torch runs single-threaded inside."""
    threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        yield
    finally:
        torch.set_num_threads(threads)


def relative_deviation(traj, ref):
    """Per step: |traj - ref| / |ref - w0| with w0 = 0 (distance from the
    reference run, relative to how far that run has moved)."""
    return np.linalg.norm(traj - ref, axis=1) / np.linalg.norm(ref, axis=1)
