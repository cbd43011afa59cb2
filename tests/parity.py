"""Helpers shared by the GPU parity tests: run the float64 oracle on the
same bytes the HIP path consumed and compare.

Tolerances (relative Frobenius error per NS unit): 1e-4 for the fp32 NS
path, 2e-2 for the bf16-operand path with fp32 accumulation; momentum 1e-6
(fp32 storage).  The weight is compared on the accumulated update:
||W_gpu - W_ref|| <= tol * ||W_ref - W0 d^t|| + 1e-6 ||W_ref||, d = 1 - lr*wd,
because the per-step update is a small fraction of W.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL_NS = {"fp32": 1e-4, "bf16": 2e-2}
TOL_M = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def oracle_hyper(h) -> oracle.Hyper:
    return oracle.Hyper(
        lr=h.lr, mu=h.mu, weight_decay=h.weight_decay, gamma=h.gamma, scale=h.scale,
        schedule=tuple((s, tuple(c)) for s, c in h.stages),
        nesterov_style=h.nesterov_style,
    )


def check_weight(w_gpu, w_ref, w0, t, h, tol, what=""):
    d = (1.0 - h.lr * h.weight_decay) ** t
    upd = np.linalg.norm(w_ref - w0 * d)
    err = np.linalg.norm(np.asarray(w_gpu, np.float64) - w_ref)
    bound = tol * upd + 1e-6 * np.linalg.norm(w_ref)
    assert err <= bound, f"{what}: |dW| {err:.3e} > {bound:.3e} (update norm {upd:.3e})"
    return err / max(upd, 1e-300)
