"""Full-size workloads on the GPU, checked against the float64 oracle.

The GPU runs every unit of each workload at its real shape and in the launch
configuration the benchmark uses (one call over all banks, whole shape
groups stacked).  The oracle then checks, on the exact bytes the GPU
consumed (the weights before the first step and every step's gradients,
read back):
  * all 48 split heads of the layer over three steps, and its large units:
    the 4096 x 4096 projection, gate and up (14336 x 4096) and down
    (4096 x 14336) at step 1, down also at step 2;
  * in the MoE bank, one expert of each bank (gate, up, down) over three
    steps, and the all-zero experts exactly;
  * in the ~7B set, on both NS paths over all three steps: the heads of two
    layers and one projection, one gate and one down matrix (the oracle runs
    once per unit; both paths consume the same seeded bytes);
  * as extras beside the oracle: the momentum recurrence of the layer's MLP
    units element by element, the fused update against the NS-only entry
    point on the same look-ahead, and the singular values of the NS output
    (eigenvalues of O O^T in float64), which for these i.i.d. inputs lie in
    phi's band [1, 1.0021] up to the rounding of the products.
"""

import hashlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import TOL_M, TOL_NS, check_weight, f64, oracle_hyper, rel, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


@pytest.fixture(autouse=True)
def _release(gpu_lib):
    yield
    gpu_lib._WS.clear()
    torch.cuda.empty_cache()


def _fma32(a, b, c):
    """fp32 fused multiply-add a*b + c with one rounding, as the momentum
    kernel computes it (the float64 product of two floats is exact)."""
    return (np.float64(np.float32(a)) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _lookahead32(m_prev32, g32, mu):
    m_new = _fma32(mu, m_prev32, g32)
    return m_new, _fma32(mu, m_new, g32)


def _alloc(wl):
    params = [W.bank_weights(wl, i, DEV) for i in range(len(wl.matrices))]
    moms = [torch.zeros_like(p) for p in params]
    splits = [m.split_rows for m in wl.matrices]
    return params, moms, splits


def _digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# Oracle trajectories of single units, kept across tests: the bf16 and the
# fp32 test of the ~7B set consume the same bytes (checked by digest) and
# share one oracle run per unit.
_ORACLE = {}


def _oracle_trajectory(key, w0, grads, hw, split_rows=0):
    """(W_t, M_t) of the oracle for t = 1..len(grads), from W0 and M0 = 0."""
    ident = (key, _digest(w0), tuple(_digest(g) for g in grads))
    if ident not in _ORACLE:
        w, m, out = w0.copy(), np.zeros_like(w0), []
        for t, g in enumerate(grads, start=1):
            w, m, _ = oracle.muon_step(w, g, m, hw, split_rows, t)
            out.append((w, m))
        _ORACLE[ident] = out
    return _ORACLE[ident]


def _run_and_collect(gpu_lib, wl, h, steps, watch):
    """Runs `steps` steps of the whole workload on the GPU (one call over
    all banks per step) and returns, per watched (bank, matrix): W0, the
    gradients of every step and the GPU's W_t and M_t after every step, as
    float64 host copies."""
    params, moms, splits = _alloc(wl)
    rec = {k: {"w0": f64(params[k[0]][k[1]]), "g": [], "w": [], "m": []} for k in watch}
    for t in range(1, steps + 1):
        say(f"   GPU step {t}")
        grads = [W.bank_grads(wl, t - 1, i, DEV) for i in range(len(wl.matrices))]
        gpu_lib.step(params, grads, moms, hyper=h, split_rows=splits)
        torch.cuda.synchronize()
        for (b, e), r in rec.items():
            r["g"].append(f64(grads[b][e]))
            r["w"].append(f64(params[b][e]))
            r["m"].append(f64(moms[b][e]))
        del grads
    del params, moms
    torch.cuda.empty_cache()
    return rec


def _check_trajectory(r, ref, h, tol, what, split_rows=0):
    """Momentum and weight of every step against the oracle's."""
    for t, ((wr, mr), wg, mg) in enumerate(zip(ref, r["w"], r["m"]), start=1):
        em = rel(mg, mr)
        assert em <= TOL_M, f"{what} step {t}: momentum rel err {em:.3e}"
        if split_rows:
            for hd in range(wr.shape[0] // split_rows):
                blk = slice(hd * split_rows, (hd + 1) * split_rows)
                check_weight(wg[blk], wr[blk], r["w0"][blk], t, h, tol, f"{what} head {hd} step {t}")
            say(f"   {what} step {t}: every head within tolerance")
        else:
            e = check_weight(wg, wr, r["w0"], t, h, tol, f"{what} step {t}")
            say(f"   {what} step {t}: relative update error {e:.3e}")


def _spectrum_band(o64, lo, hi, what):
    """Singular values of O from the eigenvalues of the smaller Gram."""
    g = o64 @ o64.T if o64.shape[0] <= o64.shape[1] else o64.T @ o64
    ev = np.linalg.eigvalsh(g)
    sv = np.sqrt(np.clip(ev, 0, None))
    say(f"   {what}: singular values in [{sv.min():.4f}, {sv.max():.4f}]")
    assert lo <= sv.min() and sv.max() <= hi, (sv.min(), sv.max())


def test_transformer_layer_workload(gpu_lib):
    # Hidden 4096: fused QKV of 48 heads x 128 rows (split per head), O
    # 4096^2, gate/up 14336x4096, down 4096x14336; Student-t(3) * 1e-3 bf16
    # grads; spectral scale; bf16 NS products; three steps.
    wl = W.workload(3)
    h = gpu_lib.Hyper(scale=wl.scale, ns_precision="bf16")
    hw = oracle_hyper(h)
    params, moms, splits = _alloc(wl)
    w0 = [f64(p[0]) for p in params]
    heads_ref = w0[0].copy()
    heads_m = np.zeros_like(heads_ref)
    o_ref, o_m = w0[1].copy(), np.zeros_like(w0[1])
    for t in range(1, wl.steps + 1):
        say(f"[layer] step {t}")
        grads = [W.bank_grads(wl, t - 1, i, DEV) for i in range(len(wl.matrices))]
        m_prev = [moms[2 + k][0].cpu().numpy() for k in range(3)]
        w_prev = [f64(p[0]) for p in params[2:]]
        gpu_lib.step(params, grads, moms, hyper=h, split_rows=splits)
        torch.cuda.synchronize()
        # split heads: full oracle
        heads_ref, heads_m, rec = oracle.muon_step(heads_ref, f64(grads[0][0]), heads_m, hw, 128, t)
        assert rel(f64(moms[0][0]), heads_m) <= TOL_M
        wg = f64(params[0][0])
        for hd in range(48):
            blk = slice(hd * 128, (hd + 1) * 128)
            check_weight(wg[blk], heads_ref[blk], w0[0][blk], t, h, TOL_NS["bf16"], f"head {hd}")
        # 4096x4096 output projection: oracle on the first step
        if t == 1:
            o_ref, o_m, _ = oracle.muon_step(o_ref, f64(grads[1][0]), o_m, hw, 0, 1)
            assert rel(f64(moms[1][0]), o_m) <= TOL_M
            e = check_weight(f64(params[1][0]), o_ref, w0[1], 1, h, TOL_NS["bf16"], "o_proj")
            say(f"   o_proj step 1 relative update error {e:.3e}")
        # MLP units: momentum recurrence and update consistency
        for k, spec in enumerate(wl.matrices[2:]):
            g32 = grads[2 + k][0].float().cpu().numpy()
            m_new, look32 = _lookahead32(m_prev[k], g32, h.mu)
            m_exp = hw.mu * m_prev[k].astype(np.float64) + g32
            assert rel(f64(moms[2 + k][0]), m_exp) <= TOL_M, spec.name
            # the NS-only entry point on the very look-ahead the step formed
            look = torch.from_numpy(look32).to(DEV)
            o, _ = gpu_lib.newton_schulz([look], hyper=h)
            torch.cuda.synchronize()
            o64 = f64(o[0])
            scale = oracle.update_scale(spec.rows, spec.cols, hw)
            w_exp = oracle.decoupled_update(w_prev[k], o64, scale, hw.lr, hw.weight_decay)
            # same products, same rounding: the fused and NS-only paths agree
            # to fp32 accuracy on the update
            upd = np.linalg.norm(w_exp - w_prev[k] * (1 - hw.lr * hw.weight_decay))
            err = np.linalg.norm(f64(params[2 + k][0]) - w_exp)
            assert err <= 1e-5 * upd + 1e-6 * np.linalg.norm(w_exp), (spec.name, err / upd)
            if t == 1:
                _spectrum_band(o64, 0.95, 1.05, spec.name)
        del grads
    torch.cuda.empty_cache()


LAYER_UNITS = {"o_proj": (1, 1), "gate": (2, 1), "up": (3, 1), "down": (4, 2)}  # bank, steps


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(LAYER_UNITS))
def test_layer_large_units_against_oracle(gpu_lib, name):
    # The layer's 4096-wide units (O 4096^2, gate and up 14336 x 4096, down
    # 4096 x 14336) against the oracle: step 1 for each, step 2 for down.
    wl = W.workload(3)
    bank, steps = LAYER_UNITS[name]
    say(f"[layer {name}] {wl.matrices[bank].rows}x{wl.matrices[bank].cols}, {steps} step(s)")
    h = gpu_lib.Hyper(scale=wl.scale, ns_precision="bf16")
    hw = oracle_hyper(h)
    r = _run_and_collect(gpu_lib, wl, h, steps, [(bank, 0)])[(bank, 0)]
    ref = _oracle_trajectory(("layer", name), r["w0"], r["g"], hw)
    _check_trajectory(r, ref, h, TOL_NS["bf16"], name)


def test_moe_bank_workload(gpu_lib):
    # 128 experts x {gate, up 2048x7168, down 7168x2048}, bf16 N(0, 1e-3)
    # grads, 13 experts all-zero on every step, three steps.
    wl = W.workload(4)
    h = gpu_lib.Hyper(scale=wl.scale, ns_precision="bf16")
    hw = oracle_hyper(h)
    params, moms, splits = _alloc(wl)
    zero = W.zero_experts(wl, 128)
    live = [e for e in range(128) if e not in set(zero.tolist())]
    # one live expert per bank: gate, up (2048 x 7168) and down (7168 x 2048)
    samples = {0: live[0], 1: live[len(live) // 2], 2: live[-1]}
    rec = {b: {"w0": f64(params[b][e]), "g": [], "w": [], "m": []} for b, e in samples.items()}
    z0 = [f64(params[b][zero]) for b in range(3)]
    for t in range(1, wl.steps + 1):
        say(f"[moe] step {t}")
        grads = [W.bank_grads(wl, t - 1, i, DEV) for i in range(3)]
        gpu_lib.step(params, grads, moms, hyper=h, split_rows=splits)
        torch.cuda.synchronize()
        d = np.float32(1.0 - np.float64(np.float32(h.lr)) * np.float64(np.float32(h.weight_decay)))
        for b in range(3):
            # unrouted experts: momentum stays zero, the weight only decays
            assert torch.count_nonzero(moms[b][zero]).item() == 0
            expect = z0[b].astype(np.float32)
            for _ in range(t):
                expect = expect * d
            np.testing.assert_array_max_ulp(f64(params[b][zero]).astype(np.float32), expect, maxulp=2 * t)
        for b, e in samples.items():
            rec[b]["g"].append(f64(grads[b][e]))
            rec[b]["w"].append(f64(params[b][e]))
            rec[b]["m"].append(f64(moms[b][e]))
        del grads
    del params, moms
    torch.cuda.empty_cache()
    for b, e in samples.items():
        ref = _oracle_trajectory(("moe", b, e), rec[b]["w0"], rec[b]["g"], hw)
        _check_trajectory(rec[b], ref, h, TOL_NS["bf16"], f"bank {b} expert {e}")


# The ~7B set's watched matrices: (bank, layer, split_rows): the fused QKV of
# layers 0 and 31 (48 heads each), one projection, one gate, one down.
SEVEN_B_WATCH = [(0, 0, 128), (0, 31, 128), (1, 3, 0), (2, 11, 0), (4, 29, 0)]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_seven_billion_matrix_set(gpu_lib, prec):
    # 32 transformer layers of the hidden-4096 shapes (6.98e9 parameters,
    # 1664 units), unit_rms_norm scale, N(0, 1e-3) grads times a per-matrix
    # scale drawn log-uniform in [1e-5, 1e-1]; three steps on each NS path.
    wl = W.workload(5)
    say(f"[7B {prec}] {wl.units} units, {wl.steps} steps")
    h = gpu_lib.Hyper(scale=wl.scale, ns_precision=prec)
    hw = oracle_hyper(h)
    rec = _run_and_collect(gpu_lib, wl, h, wl.steps, [(b, L) for b, L, _ in SEVEN_B_WATCH])
    for b, L, split in SEVEN_B_WATCH:
        name = f"{wl.matrices[b].name} layer {L}"
        say(f"   oracle: {name}")
        r = rec[(b, L)]
        ref = _oracle_trajectory(("7b", b, L), r["w0"], r["g"], hw, split)
        _check_trajectory(r, ref, h, TOL_NS[prec], name, split)
    # extra: the NS-only entry point on the step-1 look-ahead of the down
    # projection; O's singular values sit in phi's band
    g32 = rec[(4, 29)]["g"][0].astype(np.float32)
    _, look32 = _lookahead32(np.zeros_like(g32), g32, h.mu)
    o, _ = gpu_lib.newton_schulz([torch.from_numpy(look32).to(DEV)], hyper=h)
    torch.cuda.synchronize()
    tol = 0.05 if prec == "bf16" else 1e-3
    _spectrum_band(f64(o[0]), 1.0 - tol, 1.0021 + tol, "down layer 29, step 1")
