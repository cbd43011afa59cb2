"""Seeded generators for weights and gradients (torch, any device).

Every tensor is drawn from its own generator seeded by (config, step,
matrix index), so any single matrix can be regenerated alone.  Weights are
drawn with step = -1.  The same bytes that the GPU consumes are the ones the
oracle reads back; nothing here depends on how the step is computed.
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import Workload


def seed_of(cfg: int, step: int, matrix: int, salt: int = 0) -> int:
    ss = np.random.SeedSequence([cfg, step + 1, matrix, salt])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def init_weight(
    wl: Workload, matrix: int, shape, device="cpu", std: float | None = None
) -> torch.Tensor:
    """fp32 weight ~ N(0, std^2) (std = 0.02 unless given)."""
    std = wl.w_std if std is None else std
    g = _gen(device, seed_of(wl.cfg, -1, matrix))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def zero_experts(wl: Workload, n_experts: int) -> np.ndarray:
    """Experts that receive all-zero gradients on every step (unrouted):
    round(zero_fraction * n) of them, fixed per workload."""
    k = int(round(wl.zero_fraction * n_experts))
    rng = np.random.default_rng(np.random.SeedSequence([wl.cfg, 7777]))
    return np.sort(rng.choice(n_experts, size=k, replace=False))


def log_uniform_scale(wl: Workload, matrix: int, lo=-5.0, hi=-1.0) -> float:
    """Per-matrix gradient scale 10**U(lo, hi)."""
    rng = np.random.default_rng(np.random.SeedSequence([wl.cfg, 9191, matrix]))
    return float(10.0 ** rng.uniform(lo, hi))


def grad_tensor(
    wl: Workload,
    step: int,
    matrix: int,
    shape,
    dtype: str = "bf16",
    device="cpu",
) -> torch.Tensor:
    """Gradient for one matrix (or one stacked bank) at one step.

    normal:          N(0, grad_std^2)
    student_t3:      grad_std * t(nu = 3), t = z / sqrt(chi2_3 / 3)
    normal_logscale: N(0, grad_std^2) * 10**U(-5, -1), scale per matrix
    Rounded to bf16 (round-to-nearest-even, torch's cast) when dtype is bf16.
    """
    g = _gen(device, seed_of(wl.cfg, step, matrix))
    f32 = torch.float32
    if wl.grad_dist == "normal":
        x = torch.randn(shape, generator=g, device=device, dtype=f32) * wl.grad_std
    elif wl.grad_dist == "student_t3":
        z = torch.randn(shape, generator=g, device=device, dtype=f32)
        chi2 = torch.zeros(shape, device=device, dtype=f32)
        for _ in range(3):
            chi2 += torch.randn(shape, generator=g, device=device, dtype=f32) ** 2
        x = z / torch.sqrt(chi2 / 3.0) * wl.grad_std
    elif wl.grad_dist == "normal_logscale":
        x = torch.randn(shape, generator=g, device=device, dtype=f32) * (
            wl.grad_std * log_uniform_scale(wl, matrix)
        )
    else:
        raise ValueError(wl.grad_dist)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp32":
        return x
    raise ValueError(dtype)


def matrix_offsets(wl: Workload) -> list[int]:
    """Global index of the first matrix of each spec (banks are expanded:
    matrix b of spec i has global index offsets[i] + b)."""
    out, k = [], 0
    for m in wl.matrices:
        out.append(k)
        k += m.batch
    return out


def bank_weights(wl: Workload, spec: int, device="cpu") -> torch.Tensor:
    """fp32 weights of every matrix of spec `spec`, shape (batch, rows, cols)."""
    m = wl.matrices[spec]
    base = matrix_offsets(wl)[spec]
    out = torch.empty((m.batch, m.rows, m.cols), dtype=torch.float32, device=device)
    for b in range(m.batch):
        out[b] = init_weight(wl, base + b, (m.rows, m.cols), device)
    return out


def bank_grads(
    wl: Workload, step: int, spec: int, device="cpu", out: torch.Tensor | None = None
) -> torch.Tensor:
    """Gradients of every matrix of spec `spec` at `step`, shape
    (batch, rows, cols), in the spec's gradient dtype.  In a bank with a
    zero fraction, the chosen experts get all-zero gradients."""
    m = wl.matrices[spec]
    base = matrix_offsets(wl)[spec]
    dt = torch.bfloat16 if m.grad_dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty((m.batch, m.rows, m.cols), dtype=dt, device=device)
    zero = set(zero_experts(wl, m.batch).tolist()) if wl.zero_fraction else set()
    for b in range(m.batch):
        if b in zero:
            out[b].zero_()
        else:
            out[b] = grad_tensor(wl, step, base + b, (m.rows, m.cols), m.grad_dtype, device)
    return out
