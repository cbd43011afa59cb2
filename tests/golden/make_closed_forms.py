"""Write closed-form worked examples of the Muon step to closed_forms.json.

The values are derived by hand-reduction, not by running any implementation
of the step: for a *diagonal* matrix D every Newton-Schulz step maps each
diagonal entry d to the odd quintic a*d + b*d^3 + c*d^5 (the singular vectors
are the unit vectors), so the whole step reduces to scalar arithmetic, done
here in 60-digit decimal.

Sources (DeepSeek tech notes, "Muon 优化器"): section 1 Algorithm 1 (momentum,
Nesterov on mu*M_t + G_t, spectral scale sqrt(max(n, m))*gamma, decoupled
weight decay W(1 - eta*lambda) - eta*O), section 2 (Frobenius normalisation,
quintic step, hybrid schedule 8 x (3.4445, -4.7750, 2.0315) + 2 x (2, -1.5,
0.5)), section-2 sketch defaults lr 2.7e-4, mu 0.95, wd 0.1, gamma 0.18.
Megatron-LM PR "Scaling for MuP over Muon optimizer": unit_rms_norm scale
sqrt(fan_out / fan_in).  RFC-0023 方案 1: the EMA-style buffer
mu = beta*mu + (1 - beta)*g and its bias-corrected look-ahead
beta*bc(mu, t+1) + (1 - beta)*bc(g, t), with t the 1-based step.

Run:  python tests/golden/make_closed_forms.py
"""

from __future__ import annotations

import json
import os
from decimal import Decimal as D, getcontext

getcontext().prec = 60

FAST = (D("3.4445"), D("-4.7750"), D("2.0315"))
STABLE = (D("2.0"), D("-1.5"), D("0.5"))
LR, MU, WD, GAMMA = D("2.7e-4"), D("0.95"), D("0.1"), D("0.18")


def quintic(x: D, abc) -> D:
    a, b, c = abc
    return a * x + b * x**3 + c * x**5


def phi(x: D) -> D:
    """Scalar map of the hybrid schedule on a normalised singular value."""
    for _ in range(8):
        x = quintic(x, FAST)
    for _ in range(2):
        x = quintic(x, STABLE)
    return x


def ns_diag(d: list[D]) -> list[D]:
    nu = sum(v * v for v in d).sqrt()
    if nu == 0:
        return [D(0)] * len(d)
    return [phi(v / nu) for v in d]


def bc(x: D, count: int) -> D:
    """Bias correction x / (1 - mu^count)."""
    return x / (D(1) - MU**count)


def step_diag(w, g, m, n_rows, n_cols, scale_mode, style="sgd", t=1):
    """One Muon step on a diagonal n_rows x n_cols matrix given by its
    diagonal entries (w is the full matrix as nested lists).  style "sgd":
    classic momentum with the look-ahead on the updated buffer; "ema": the
    buffer is an exponential moving average and the look-ahead combines the
    buffer corrected with count t+1 and the gradient corrected with count t
    (RFC-0023 方案 1), t being the 1-based step."""
    if style == "sgd":
        m_new = [MU * mi + gi for mi, gi in zip(m, g)]
        look = [MU * mi + gi for mi, gi in zip(m_new, g)]
    else:
        m_new = [MU * mi + (D(1) - MU) * gi for mi, gi in zip(m, g)]
        look = [MU * bc(mi, t + 1) + (D(1) - MU) * bc(gi, t) for mi, gi in zip(m_new, g)]
    o = ns_diag(look)
    if scale_mode == "spectral":
        scale = D(max(n_rows, n_cols)).sqrt() * GAMMA
    else:
        scale = (D(n_rows) / D(n_cols)).sqrt()
    decay = D(1) - LR * WD
    w_new = [[wij * decay for wij in row] for row in w]
    for i, oi in enumerate(o):
        w_new[i][i] -= LR * scale * oi
    return w_new, m_new, look, o, scale


def f(x: D) -> str:
    return format(x, "f")


def main():
    cases = []
    # (1) 1x1, two steps, fp32-representable inputs.
    w = [[D("0.5")]]
    m = [D(0)]
    steps = []
    for g in ([D("0.25")], [D("-1.0")]):
        w, m, look, o, scale = step_diag(w, g, m, 1, 1, "spectral")
        steps.append({"g": [f(v) for v in g], "w": [[f(v) for v in r] for r in w],
                      "m": [f(v) for v in m], "nesterov": [f(v) for v in look],
                      "o_diag": [f(v) for v in o], "scale": f(scale)})
    cases.append({"name": "1x1_two_steps", "rows": 1, "cols": 1, "scale": "spectral",
                  "w0": [["0.5"]], "steps": steps})
    # (2) 3x5 rectangular diagonal, spectral, three steps (the third with a zero gradient).
    rows, cols = 3, 5
    w0 = [[D(i * cols + j + 1) / D(64) for j in range(cols)] for i in range(rows)]
    w, m = [r[:] for r in w0], [D(0)] * rows
    steps = []
    for g in ([D(3), D(-4), D("0.5")], [D(1), D(2), D(-2)], [D(0), D(0), D(0)]):
        w, m, look, o, scale = step_diag(w, g, m, rows, cols, "spectral")
        steps.append({"g": [f(v) for v in g], "w": [[f(v) for v in r] for r in w],
                      "m": [f(v) for v in m], "nesterov": [f(v) for v in look],
                      "o_diag": [f(v) for v in o], "scale": f(scale)})
    cases.append({"name": "3x5_diag_spectral", "rows": rows, "cols": cols, "scale": "spectral",
                  "w0": [[f(v) for v in r] for r in w0], "steps": steps})
    # (3) 4x2 tall diagonal, unit_rms_norm, one step.
    rows, cols = 4, 2
    w0 = [[D(i - j) / D(16) for j in range(cols)] for i in range(rows)]
    m = [D(0)] * cols
    g = [D("1.5"), D("-0.75")]
    w, m, look, o, scale = step_diag(w0, g, m, rows, cols, "unit_rms_norm")
    cases.append({"name": "4x2_diag_unit_rms", "rows": rows, "cols": cols,
                  "scale": "unit_rms_norm", "w0": [[f(v) for v in r] for r in w0],
                  "steps": [{"g": [f(v) for v in g], "w": [[f(v) for v in r] for r in w],
                             "m": [f(v) for v in m], "nesterov": [f(v) for v in look],
                             "o_diag": [f(v) for v in o], "scale": f(scale)}]})
    # (4) 3x5 diagonal, EMA-style look-ahead with bias correction, two steps
    # with different gradients (t = 1, 2), spectral scale.
    rows, cols = 3, 5
    w0 = [[D(i * cols + j + 1) / D(64) for j in range(cols)] for i in range(rows)]
    w, m = [r[:] for r in w0], [D(0)] * rows
    steps = []
    for t, g in enumerate(([D(2), D("-0.5"), D(1)], [D("-1.25"), D(3), D("0.75")]), start=1):
        w, m, look, o, scale = step_diag(w, g, m, rows, cols, "spectral", style="ema", t=t)
        steps.append({"g": [f(v) for v in g], "w": [[f(v) for v in r] for r in w],
                      "m": [f(v) for v in m], "nesterov": [f(v) for v in look],
                      "o_diag": [f(v) for v in o], "scale": f(scale)})
    cases.append({"name": "3x5_diag_ema_two_steps", "rows": rows, "cols": cols,
                  "scale": "spectral", "nesterov_style": "ema",
                  "w0": [[f(v) for v in r] for r in w0], "steps": steps})
    # Scalar map values.
    table = {
        "phi(1)": f(phi(D(1))),
        "phi(0.5)": f(phi(D("0.5"))),
        "phi(1e-3)": f(phi(D("1e-3"))),
        "phi(3e-5)": f(phi(D("3e-5"))),
        "phi(1e-6)": f(phi(D("1e-6"))),
        "fast_stage_end(1)": None,
    }
    x = D(1)
    for _ in range(8):
        x = quintic(x, FAST)
    table["fast_stage_end(1)"] = f(x)
    out = {
        "source": "DeepSeek tech notes 'Muon 优化器' sections 1-2 (Algorithm 1, hybrid NS); "
                  "Megatron-LM PR 'Scaling for MuP over Muon optimizer' (unit_rms_norm)",
        "derivation": "diagonal matrices reduce NS to the scalar quintic; 60-digit decimal",
        "hyper": {"lr": "2.7e-4", "mu": "0.95", "weight_decay": "0.1", "gamma": "0.18"},
        "phi": table,
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
