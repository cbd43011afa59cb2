"""Float64 CPU oracle of the Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
HIP library is checked against.  Only the test suite, the smoke check in
__graft_entry__.py and the CPU-baseline leg of the benchmark may import it; the product path
(the HIP library and its Python binding) never does, and the two share no
code.  It depends on NumPy alone.

Sources (cited by page title and section; every page is a web page):

* [V4-notes]  DeepSeek tech notes, "Muon 优化器" (DeepSeek-V4 Muon).
  - section 1, Algorithm 1: the step G -> M -> Nesterov -> HybridNewtonSchulz
    -> spectral scale sqrt(max(n, m)) * gamma -> decoupled weight decay.
  - section 2 ("Hybrid Newton-Schulz"): Frobenius normalisation, the quintic
    step  M_k = a M + b (M M^T) M + c (M M^T)^2 M,  and the hybrid schedule of
    8 fast steps (3.4445, -4.7750, 2.0315) followed by 2 stable steps
    (2, -1.5, 0.5); its NumPy teaching sketch returns a zero matrix unchanged.
  - section 3: hyper-parameters momentum 0.95, weight decay 0.1, gamma 0.18.
* [RFC-0023]  "RFC-0023: align the MaxText Muon optimizer with Megatron-LM".
  - 方案 1: classic SGD momentum buf = beta*buf + grad followed by the Nesterov
    look-ahead g = grad + beta*buf on the *updated* buffer, no bias correction;
    the optax EMA form (mu = beta*mu + (1-beta)*g with bias correction) is the
    alternative 'ema' style.
  - 方案 3 / background: split_head orthogonalises each head separately, with
    fan_out = head_dim (heads become a batch dimension).
  - 方案 4: muon_batch_update stacks same-shape matrices, runs NS once with a
    leading batch dimension, then unstacks (results are per matrix).
* [PR-3715]  Megatron-LM PR "Scaling for MuP over Muon optimizer":
  spectral scale sqrt(max(fan_in, fan_out)) versus unit_rms_norm
  sqrt(fan_out / fan_in).

Readings where the pages are silent or garbled (each is listed with its
reason in the design notes of the repository):

* rows = fan_out, cols = fan_in (PyTorch [out, in] layout).
* gamma multiplies only the spectral scale; unit_rms_norm has no gamma.
* The Gram side: the pages write M M^T for any shape.  Since
  (X X^T)^k X = X (X^T X)^k exactly, the oracle iterates on the smaller side
  (transposing a tall matrix first); `ns_step_pages_form` keeps the literal
  rows-side form and the tests pin the two against each other.
* A unit whose Frobenius norm is exactly zero returns O = 0 (no epsilon).
* Split heads are contiguous row blocks of the fused weight.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Sequence

import numpy as np

# [V4-notes] section 2: hybrid schedule, 8 fast steps then 2 stable steps.
FAST_COEFFS = (3.4445, -4.7750, 2.0315)
STABLE_COEFFS = (2.0, -1.5, 0.5)
HYBRID_SCHEDULE: tuple[tuple[int, tuple[float, float, float]], ...] = (
    (8, FAST_COEFFS),
    (2, STABLE_COEFFS),
)


@dataclass
class Hyper:
    """Muon hyper-parameters.  Defaults: [V4-notes] section 3 and the
    keyword defaults of its section-2 sketch (lr 2.7e-4, mu 0.95,
    weight decay 0.1, gamma 0.18); spectral scale as in Algorithm 1."""

    lr: float = 2.7e-4
    mu: float = 0.95
    weight_decay: float = 0.1
    gamma: float = 0.18
    scale: str = "spectral"  # or "unit_rms_norm" ([PR-3715])
    schedule: Sequence[tuple[int, tuple[float, float, float]]] = field(
        default_factory=lambda: HYBRID_SCHEDULE
    )
    nesterov_style: str = "sgd"  # or "ema" ([RFC-0023] 方案 1)


# ---------------------------------------------------------------- momentum --
def sgd_momentum(m: np.ndarray, g: np.ndarray, mu: float) -> np.ndarray:
    """[RFC-0023] 方案 1 / [V4-notes] Algorithm 1: M_t = mu*M_{t-1} + G_t."""
    return mu * m + g


def sgd_nesterov(m_new: np.ndarray, g: np.ndarray, mu: float) -> np.ndarray:
    """Nesterov look-ahead on the updated buffer: mu*M_t + G_t
    ([RFC-0023] 方案 1 'sgd' style; [V4-notes] Algorithm 1)."""
    return mu * m_new + g


def ema_momentum(m: np.ndarray, g: np.ndarray, beta: float) -> np.ndarray:
    """[RFC-0023] 方案 1 'ema' style accumulation: mu = beta*mu + (1-beta)*g."""
    return beta * m + (1.0 - beta) * g


def bias_correction(x: np.ndarray, beta: float, count: int) -> np.ndarray:
    """optax-style bias correction x / (1 - beta**count) (the bc(., t) of
    [RFC-0023] 方案 1)."""
    return x / (1.0 - beta**count)


def ema_lookahead(m_new: np.ndarray, g: np.ndarray, beta: float, step: int) -> np.ndarray:
    """EMA-style Nesterov look-ahead with bias correction, with `step` the
    1-based index of the current step ([RFC-0023] 方案 1, read as in optax:
    the momentum term is corrected with count step+1 and the gradient term
    with count step)."""
    return beta * bias_correction(m_new, beta, step + 1) + (1.0 - beta) * bias_correction(
        g, beta, step
    )


# --------------------------------------------------------- Newton-Schulz ----
def frobenius_norm(x: np.ndarray) -> float:
    """sqrt of the sum of squares, in float64 ([V4-notes] section 2)."""
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.sum(x * x)))


def ns_step_pages_form(x: np.ndarray, abc: tuple[float, float, float]) -> np.ndarray:
    """One quintic step exactly as [V4-notes] section 2 writes it, with the
    Gram on the rows side:  a X + b (X X^T) X + c (X X^T)^2 X."""
    a, b, c = abc
    gram = x @ x.T
    gx = gram @ x
    return a * x + b * gx + c * (gram @ gx)


def newton_schulz_pages_form(
    x: np.ndarray, schedule=HYBRID_SCHEDULE
) -> np.ndarray:
    """Hybrid NS on the rows side for any shape ([V4-notes] section 2),
    used by the tests to pin the smaller-side form below."""
    x = np.asarray(x, dtype=np.float64)
    nu = frobenius_norm(x)
    if nu == 0.0:
        return np.zeros_like(x)
    x = x / nu
    for steps, abc in schedule:
        for _ in range(steps):
            x = ns_step_pages_form(x, abc)
    return x


def newton_schulz(x: np.ndarray, schedule=HYBRID_SCHEDULE) -> np.ndarray:
    """Hybrid Newton-Schulz approximation of the polar factor of `x`
    ([V4-notes] section 2), in float64.

    1. nu = ||X||_F; a zero matrix gives O = 0.
    2. X0 = X / nu.
    3. For each (steps, (a, b, c)) of the schedule, `steps` times:
       A = X X^T;  X <- a X + (b A + c A A) X.
    The Gram is taken on the smaller side: a tall X (rows > cols) is
    transposed before the loop and the result transposed back, which equals
    the rows-side form because (X X^T)^k X = X (X^T X)^k.
    """
    x = np.asarray(x, dtype=np.float64)
    nu = frobenius_norm(x)
    if nu == 0.0:
        return np.zeros_like(x)
    tall = x.shape[0] > x.shape[1]
    y = (x / nu).T if tall else x / nu
    for steps, (a, b, c) in schedule:
        for _ in range(steps):
            gram = y @ y.T
            poly = b * gram + c * (gram @ gram)
            y = a * y + poly @ y
    return np.ascontiguousarray(y.T if tall else y)


# ----------------------------------------------------------------- scales ---
def spectral_scale(fan_out: int, fan_in: int, gamma: float) -> float:
    """[V4-notes] Algorithm 1 / [PR-3715]: sqrt(max(fan_in, fan_out)) * gamma."""
    return float(np.sqrt(max(fan_out, fan_in)) * gamma)


def unit_rms_norm_scale(fan_out: int, fan_in: int) -> float:
    """[PR-3715]: sqrt(fan_out / fan_in) (no gamma)."""
    return float(np.sqrt(fan_out / fan_in))


def update_scale(fan_out: int, fan_in: int, hyper: Hyper) -> float:
    if hyper.scale == "spectral":
        return spectral_scale(fan_out, fan_in, hyper.gamma)
    if hyper.scale == "unit_rms_norm":
        return unit_rms_norm_scale(fan_out, fan_in)
    raise ValueError(f"unknown scale mode {hyper.scale!r}")


def decoupled_update(
    w: np.ndarray, o: np.ndarray, scale: float, lr: float, weight_decay: float
) -> np.ndarray:
    """[V4-notes] Algorithm 1: W_t = W_{t-1} (1 - eta*lambda) - eta * O_t,
    with O_t = O'_t * scale."""
    return w * (1.0 - lr * weight_decay) - lr * (o * scale)


# ------------------------------------------------------------------ units ---
def unit_row_blocks(rows: int, split_rows: int) -> list[tuple[int, int]]:
    """NS units of one weight: the whole matrix, or, under split_head, the
    contiguous blocks of `split_rows` rows ([RFC-0023] split_head)."""
    if split_rows in (0, None):
        return [(0, rows)]
    if rows % split_rows:
        raise ValueError("split_rows must divide rows")
    return [(r, split_rows) for r in range(0, rows, split_rows)]


@dataclass
class StepRecord:
    """What one oracle step produced, kept for element-wise comparison."""

    nesterov: np.ndarray  # mu*M_t + G_t
    norms: list[float]  # ||unit||_F per NS unit
    ortho: list[np.ndarray]  # NS output O' per unit (unscaled)
    scales: list[float]  # per-unit update scale


def muon_step(
    w: np.ndarray,
    g: np.ndarray,
    m: np.ndarray,
    hyper: Hyper = Hyper(),
    split_rows: int = 0,
    step: int = 1,
) -> tuple[np.ndarray, np.ndarray, StepRecord]:
    """One Muon step for one 2-D weight ([V4-notes] Algorithm 1 and its
    section-2 sketch; [RFC-0023] 'sgd' Nesterov; [PR-3715] scales).

    w, m: the current weight and momentum (widened to float64);
    g: the gradient (bf16 or fp32 values, widened exactly);
    split_rows: 0, or the head size for split_head;
    step: 1-based step index (only the 'ema' style uses it).
    Returns (w_new, m_new, record).
    """
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    if hyper.nesterov_style == "sgd":
        m_new = sgd_momentum(m, g, hyper.mu)
        look = sgd_nesterov(m_new, g, hyper.mu)
    elif hyper.nesterov_style == "ema":
        m_new = ema_momentum(m, g, hyper.mu)
        look = ema_lookahead(m_new, g, hyper.mu, step)
    else:
        raise ValueError(f"unknown nesterov style {hyper.nesterov_style!r}")

    w_new = np.empty_like(w)
    rec = StepRecord(nesterov=look, norms=[], ortho=[], scales=[])
    cols = w.shape[1]
    for r0, nr in unit_row_blocks(w.shape[0], split_rows):
        block = look[r0 : r0 + nr]
        o = newton_schulz(block, hyper.schedule)
        s = update_scale(nr, cols, hyper)
        w_new[r0 : r0 + nr] = decoupled_update(
            w[r0 : r0 + nr], o, s, hyper.lr, hyper.weight_decay
        )
        rec.norms.append(frobenius_norm(block))
        rec.ortho.append(o)
        rec.scales.append(s)
    return w_new, m_new, rec
