"""Pins of the float64 oracle against facts the pages and the mathematics fix.

None of these re-type the oracle's own code: each checks it against a closed
form, an invariant, a special case with an independent derivation, or a
brute-force construction (SVD).  Citations: DeepSeek tech notes "Muon 优化器"
(section 1 Algorithm 1; section 2 hybrid Newton-Schulz and sketch),
RFC-0023 (方案 1 SGD/Nesterov momentum, split_head), Megatron-LM PR
"Scaling for MuP over Muon optimizer" (spectral vs unit_rms_norm).
"""

import json
import math
import os
from decimal import Decimal

import numpy as np
import pytest

import oracle
from oracle import Hyper

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def phi_scalar(x: float) -> float:
    """Scalar image of a normalised singular value under the hybrid schedule
    (the quintic acts on singular values, section 2 of the DeepSeek notes)."""
    for _ in range(8):
        x = 3.4445 * x - 4.7750 * x**3 + 2.0315 * x**5
    for _ in range(2):
        x = 2.0 * x - 1.5 * x**3 + 0.5 * x**5
    return x


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


# ----------------------------------------------------------- coefficients ---
def test_schedule_is_eight_fast_then_two_stable():
    sched = list(oracle.HYBRID_SCHEDULE)
    assert sched == [(8, (3.4445, -4.7750, 2.0315)), (2, (2.0, -1.5, 0.5))]


def test_stable_step_fixes_one_with_zero_slope():
    # q(x) = 2x - 1.5x^3 + 0.5x^5 has q(1) = 1 and q'(1) = 0: the stable
    # stage's coefficients make 1 a super-attracting fixed point.
    a, b, c = oracle.STABLE_COEFFS
    assert a + b + c == 1.0
    assert a + 3 * b + 5 * c == 0.0


# ------------------------------------------------------------- momentum -----
def test_momentum_closed_form_constant_gradient():
    # With constant G and M0 = 0: M_t = G (1 - mu^t)/(1 - mu) and
    # N_t = mu M_t + G = G (1 + mu (1 - mu^t)/(1 - mu)).
    rng = np.random.default_rng(0)
    g = rng.standard_normal((6, 9))
    w = rng.standard_normal((6, 9)) * 0.02
    m = np.zeros_like(g)
    mu = 0.95
    for t in range(1, 8):
        w, m, rec = oracle.muon_step(w, g, m, Hyper())
        np.testing.assert_allclose(m, g * (1 - mu**t) / (1 - mu), rtol=1e-14, atol=0)
        np.testing.assert_allclose(
            rec.nesterov, g * (1 + mu * (1 - mu**t) / (1 - mu)), rtol=1e-14, atol=0
        )


def test_constant_gradient_weight_closed_form():
    # NS is scale invariant, so constant G gives the same O every step, and
    # W_t = W0 d^t - eta s O sum_{k<t} d^k with d = 1 - eta*lambda.
    rng = np.random.default_rng(1)
    g = rng.standard_normal((5, 12))
    w0 = rng.standard_normal((5, 12)) * 0.02
    h = Hyper()
    o = oracle.newton_schulz(g)
    s = math.sqrt(12) * h.gamma
    d = 1 - h.lr * h.weight_decay
    w, m = w0, np.zeros_like(g)
    for t in range(1, 6):
        w, m, _ = oracle.muon_step(w, g, m, h)
        expect = w0 * d**t - h.lr * s * o * sum(d**k for k in range(t))
        np.testing.assert_allclose(w, expect, rtol=1e-12, atol=1e-16)


def test_zero_gradient_zero_momentum_is_pure_decay():
    rng = np.random.default_rng(2)
    w0 = rng.standard_normal((7, 3))
    w1, m1, rec = oracle.muon_step(w0, np.zeros((7, 3)), np.zeros((7, 3)), Hyper())
    assert np.array_equal(m1, np.zeros((7, 3)))
    assert np.array_equal(rec.ortho[0], np.zeros((7, 3)))
    assert np.array_equal(w1, w0 * (1 - 2.7e-4 * 0.1))


# --------------------------------------------------- Newton-Schulz pins -----
@pytest.mark.parametrize("shape", [(4, 9), (9, 4), (16, 16), (1, 5), (6, 1), (33, 70)])
def test_gram_side_identity(shape):
    # (X X^T)^k X = X (X^T X)^k: iterating on the smaller side equals the
    # pages' rows-side form.
    x = np.random.default_rng(3).standard_normal(shape)
    assert rel(oracle.newton_schulz(x), oracle.newton_schulz_pages_form(x)) < 1e-12


@pytest.mark.parametrize("shape", [(64, 128), (40, 128), (128, 40), (37, 37), (2, 3)])
def test_spectral_map_against_svd(shape):
    # Each quintic step is an odd polynomial of X X^T times X, so it keeps
    # the singular vectors and maps each normalised singular value x to
    # phi(x): NS(X) = U phi(S/||X||_F) V^T.  Rebuilt from a LAPACK SVD.
    x = np.random.default_rng(4).standard_normal(shape)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    nu = np.sqrt(np.sum(s**2))
    expect = (u * np.array([phi_scalar(v / nu) for v in s])) @ vt
    assert rel(oracle.newton_schulz(x), expect) < 1e-10


def test_polar_factor_brute_force():
    # For well-conditioned inputs (normalised singular values >= 3e-5),
    # phi stays within [1, 1.00202], so NS(X) is within that of U V^T.
    rng = np.random.default_rng(5)
    for shape in [(8, 8), (5, 11), (12, 4)]:
        x = rng.standard_normal(shape)
        u, s, vt = np.linalg.svd(x, full_matrices=False)
        assert s.min() / np.sqrt(np.sum(s**2)) >= 3e-5
        o = oracle.newton_schulz(x)
        polar = u @ vt
        assert rel(o, polar) <= 2.02e-3
        so = np.linalg.svd(o, compute_uv=False)
        assert so.min() >= 1.0 - 1e-9 and so.max() <= 1.00202


def test_phi_values_match_decimal_derivation():
    gold = json.load(open(GOLDEN))["phi"]
    for key, x in [("phi(1)", 1.0), ("phi(0.5)", 0.5), ("phi(1e-3)", 1e-3),
                   ("phi(3e-5)", 3e-5), ("phi(1e-6)", 1e-6)]:
        # diag(x, sqrt(1 - x^2)) has unit Frobenius norm, so its first
        # entry is mapped to phi(x).
        y = math.sqrt(1 - x * x)
        got = oracle.newton_schulz(np.array([[x, 0.0], [0.0, y]]))[0, 0]
        assert abs(got - float(Decimal(gold[key]))) <= 1e-13 * max(1.0, abs(got)) / max(x, 1e-3)


def test_one_by_one_and_sign():
    phi1 = 1.000014309583231
    assert abs(oracle.newton_schulz(np.array([[3.0]]))[0, 0] - phi1) < 1e-15
    assert abs(oracle.newton_schulz(np.array([[-0.01]]))[0, 0] + phi1) < 1e-15


def test_scale_invariance_and_oddness():
    x = np.random.default_rng(6).standard_normal((10, 17))
    o = oracle.newton_schulz(x)
    assert rel(oracle.newton_schulz(123.0 * x), o) < 1e-13
    assert rel(oracle.newton_schulz(-x), -o) < 1e-15


def test_rank_one():
    rng = np.random.default_rng(7)
    u, v = rng.standard_normal(6), rng.standard_normal(9)
    x = np.outer(u, v)
    expect = 1.000014309583231 * np.outer(u, v) / (np.linalg.norm(u) * np.linalg.norm(v))
    assert rel(oracle.newton_schulz(x), expect) < 1e-10


def test_diagonal_elementwise():
    d = np.array([3.0, -1.0, 0.5, 2e-3, 0.0])
    nu = np.linalg.norm(d)
    o = oracle.newton_schulz(np.diag(d))
    expect = np.diag([math.copysign(phi_scalar(abs(v) / nu), v) if v else 0.0 for v in d])
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=1e-300)


def test_orthogonal_input():
    q, _ = np.linalg.qr(np.random.default_rng(8).standard_normal((16, 16)))
    # All singular values are 1, normalised to 1/sqrt(16).
    assert rel(oracle.newton_schulz(q), phi_scalar(0.25) * q) < 1e-13


def test_transpose_and_orthogonal_equivariance():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((7, 12))
    o = oracle.newton_schulz(x)
    assert rel(oracle.newton_schulz(x.T), o.T) < 1e-12
    q1, _ = np.linalg.qr(rng.standard_normal((7, 7)))
    q2, _ = np.linalg.qr(rng.standard_normal((12, 12)))
    assert rel(oracle.newton_schulz(q1 @ x @ q2), q1 @ o @ q2) < 1e-11


# ---------------------------------------------------------------- scales ----
@pytest.mark.parametrize(
    "rows,cols,spectral,unit_rms",
    [
        (1024, 1024, 5.76, 1.0),
        (128, 4096, 11.52, 0.1767766952966369),
        (4096, 4096, 11.52, 1.0),
        (14336, 4096, 21.551946547817902, 1.8708286933869707),
        (4096, 14336, 21.551946547817902, 0.5345224838248488),
        (2048, 7168, 15.239527551732042, 0.5345224838248488),
        (64, 128, 2.0364675298172568, 0.7071067811865476),
    ],
)
def test_update_scales(rows, cols, spectral, unit_rms):
    # spectral sqrt(max(fan_out, fan_in)) * 0.18 and unit_rms_norm
    # sqrt(fan_out / fan_in) with rows = fan_out, cols = fan_in.
    assert oracle.update_scale(rows, cols, Hyper()) == pytest.approx(spectral, rel=1e-15)
    assert oracle.update_scale(rows, cols, Hyper(scale="unit_rms_norm")) == pytest.approx(
        unit_rms, rel=1e-15
    )


def test_update_rms_spectral():
    # The spectral scale makes the update RMS gamma * (mean phi), i.e.
    # within gamma * [1, 1.00202] for well-conditioned inputs.
    x = np.random.default_rng(10).standard_normal((32, 96))
    o = oracle.newton_schulz(x) * oracle.update_scale(32, 96, Hyper())
    # ||O||_F^2 = sum phi^2 over min(n, m) = 32 singular values, so
    # RMS(O) = phi_rms / sqrt(max(n, m)).
    rms = np.sqrt(np.mean(o**2))
    assert 0.18 * (1 - 1e-9) <= rms <= 0.18 * 1.00202


# -------------------------------------------------------------- split_head --
def test_split_head_units_are_row_blocks_with_head_scale():
    rng = np.random.default_rng(11)
    heads, hd, cols = 3, 4, 10
    w = rng.standard_normal((heads * hd, cols)) * 0.02
    g = rng.standard_normal((heads * hd, cols))
    w1, m1, rec = oracle.muon_step(w, g, np.zeros_like(g), Hyper(), split_rows=hd)
    assert len(rec.ortho) == heads
    for h in range(heads):
        blk = 1.95 * g[h * hd : (h + 1) * hd]
        u, s, vt = np.linalg.svd(blk, full_matrices=False)
        o = (u * np.array([phi_scalar(v / np.linalg.norm(s)) for v in s])) @ vt
        scale = math.sqrt(cols) * 0.18  # fan_out = head_dim = 4 < fan_in
        expect = w[h * hd : (h + 1) * hd] * (1 - 2.7e-5) - 2.7e-4 * scale * o
        np.testing.assert_allclose(w1[h * hd : (h + 1) * hd], expect, rtol=1e-9, atol=1e-15)


# ---------------------------------------------------- worked examples -------
def test_closed_form_worked_examples():
    gold = json.load(open(GOLDEN))
    for case in gold["cases"]:
        rows, cols = case["rows"], case["cols"]
        h = Hyper(scale=case["scale"], nesterov_style=case.get("nesterov_style", "sgd"))
        w = np.array([[float(v) for v in r] for r in case["w0"]])
        m = np.zeros((rows, cols))
        k = min(rows, cols)
        for t, st in enumerate(case["steps"], start=1):
            g = np.zeros((rows, cols))
            g[np.arange(k), np.arange(k)] = [float(v) for v in st["g"]]
            w, m, rec = oracle.muon_step(w, g, m, h, step=t)
            np.testing.assert_allclose(np.diag(m), [float(v) for v in st["m"]], rtol=1e-15)
            np.testing.assert_allclose(
                np.diag(rec.nesterov), [float(v) for v in st["nesterov"]], rtol=1e-14
            )
            np.testing.assert_allclose(
                np.diag(rec.ortho[0]), [float(v) for v in st["o_diag"]], rtol=1e-13, atol=1e-300
            )
            assert rec.scales[0] == pytest.approx(float(st["scale"]), rel=1e-15)
            np.testing.assert_allclose(
                w, np.array([[float(v) for v in r] for r in st["w"]]), rtol=1e-14, atol=1e-18
            )


# ------------------------------------------------------------ EMA variant ---
def test_ema_without_bias_correction_is_scaled_sgd():
    # Without bias correction the EMA buffer is (1-beta) times the SGD buffer
    # and so is the look-ahead; NS is scale invariant, hence the same O.
    rng = np.random.default_rng(12)
    beta = 0.95
    m_sgd = np.zeros((4, 6))
    m_ema = np.zeros((4, 6))
    for _ in range(4):
        g = rng.standard_normal((4, 6))
        m_sgd = oracle.sgd_momentum(m_sgd, g, beta)
        m_ema = oracle.ema_momentum(m_ema, g, beta)
        np.testing.assert_allclose(m_ema, (1 - beta) * m_sgd, rtol=1e-13)
        la_sgd = oracle.sgd_nesterov(m_sgd, g, beta)
        la_ema = beta * m_ema + (1 - beta) * g
        np.testing.assert_allclose(la_ema, (1 - beta) * la_sgd, rtol=1e-13)
        assert rel(oracle.newton_schulz(la_ema), oracle.newton_schulz(la_sgd)) < 1e-12


def test_ema_bias_correction_recovers_a_constant_gradient():
    # From a zero buffer the EMA after t equal gradients is (1 - beta^t) g,
    # so the bias correction with count t returns g exactly (an off-by-one
    # in the count would not); and both corrections tend to 1, so the
    # look-ahead tends to beta*mu + (1-beta)*g.
    beta = 0.95
    g = np.array([[1.5, -2.0], [0.25, 3.0]])
    m = np.zeros_like(g)
    for t in range(1, 7):
        m = oracle.ema_momentum(m, g, beta)
        np.testing.assert_allclose(oracle.bias_correction(m, beta, t), g, rtol=1e-14)
    m_late = oracle.ema_momentum(np.full_like(g, 0.3), g, beta)
    look = oracle.ema_lookahead(m_late, g, beta, 4000)
    np.testing.assert_allclose(look, beta * m_late + (1 - beta) * g, rtol=1e-12)


def test_ema_lookahead_closed_forms_for_a_constant_gradient():
    # A constant gradient g from a zero buffer gives the EMA buffer
    # (1 - beta^t) g after t steps.  With the look-ahead of RFC-0023 方案 1
    # (the buffer corrected with count t+1, the gradient with count t) the
    # first steps reduce to rational functions of beta alone:
    #   t = 1: (1 + 2 beta) / (1 + beta) * g
    #   t = 2: (beta (1 + beta) / (1 + beta + beta^2) + 1 / (1 + beta)) * g
    #   t = 3: (beta (1 + beta + beta^2) / (1 + beta + beta^2 + beta^3)
    #           + 1 / (1 + beta + beta^2)) * g
    # Swapping the two counts, or shifting them, changes every one of these.
    beta = 0.95
    g = np.array([[2.0, -0.5, 1.25], [0.0, 3.0, -4.0]])
    expect = {
        1: (1 + 2 * beta) / (1 + beta),
        2: beta * (1 + beta) / (1 + beta + beta**2) + 1 / (1 + beta),
        3: beta * (1 + beta + beta**2) / (1 + beta + beta**2 + beta**3) + 1 / (1 + beta + beta**2),
    }
    m = np.zeros_like(g)
    for t in (1, 2, 3):
        m = oracle.ema_momentum(m, g, beta)
        look = oracle.ema_lookahead(m, g, beta, t)
        np.testing.assert_allclose(look, expect[t] * g, rtol=1e-14, atol=0)
    # The whole step: NS is scale invariant, so O is NS(g) at every step,
    # and the step index reaches the look-ahead through muon_step.
    h = Hyper(nesterov_style="ema", mu=beta)
    w0 = np.ones_like(g) * 0.01
    w, m = w0.copy(), np.zeros_like(g)
    for t in (1, 2):
        w, m, rec = oracle.muon_step(w, g, m, h, step=t)
        np.testing.assert_allclose(rec.nesterov, expect[t] * g, rtol=1e-14, atol=0)
