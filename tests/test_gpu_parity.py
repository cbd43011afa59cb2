"""GPU parity of the HIP Muon path against the float64 oracle.

Small cases run the oracle in full (several tiles, ragged tails, tall and
wide units, split heads); the benchmark workload (32 x 1024^2, bf16
gradients) is checked on sampled units over every step.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import TOL_M, TOL_NS, check_weight, f64, oracle_hyper, rel, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _seeded(shape, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(DEV)


# ------------------------------------------------------------ NS only -------
NS_SHAPES = [
    (64, 128),    # the single-matrix workload, one padded 128-tile
    (128, 64),    # tall
    (200, 300),   # ragged on both sides, 128 tiles
    (300, 200),   # ragged tall
    (1, 7),
    (7, 1),
    (1, 1),
    (256, 512),   # 256 tiles
    (600, 260),   # 256 tiles, ragged tall
    (384, 1000),  # 256 tiles, ragged wide, several tiles each way
    (128, 300),   # small-unit path (whole NS on chip): 128 rows, ragged columns
    (100, 1000),  # small-unit path: ragged rows, eight 128-column blocks
    (100, 125),   # one-block small unit, odd width
]


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", NS_SHAPES, ids=[f"{r}x{c}" for r, c in NS_SHAPES])
def test_ns_only_matches_oracle(gpu_lib, shape, prec):
    say(f"[ns] shape={shape} prec={prec}")
    x = _seeded(shape, 1000 + shape[0] * 7 + shape[1])
    h = gpu_lib.Hyper(ns_precision=prec)
    outs, _ = gpu_lib.newton_schulz([x], hyper=h)
    torch.cuda.synchronize()
    o_ref = oracle.newton_schulz(f64(x))
    e = rel(f64(outs[0]), o_ref)
    say(f"   rel err {e:.3e}")
    assert e <= TOL_NS[prec], f"rel err {e:.3e}"


# Wide units of at most 128 rows and more than eight 128-column blocks: the
# default schedule runs many of them (at least half the CUs) on chip one
# workgroup each and a few of them on chip split over several workgroups
# (partial Grams summed through memory); the forced schedules always tile.
@pytest.mark.parametrize("sched", ["auto", "persistent", "launches"])
@pytest.mark.parametrize("batch,rows,cols", [(12, 128, 1100), (160, 96, 1100)],
                         ids=["few-long", "many-long"])
def test_ns_long_small_units_every_schedule(gpu_lib, sched, batch, rows, cols):
    say(f"[ns long small units] {batch}x{rows}x{cols} schedule={sched}")
    x = _seeded((batch, rows, cols), 4242 + batch)
    h = gpu_lib.Hyper(ns_precision="bf16", schedule=sched)
    outs, _ = gpu_lib.newton_schulz([x], hyper=h)
    torch.cuda.synchronize()
    worst = 0.0
    for i in sorted({0, batch // 2, batch - 1}):
        worst = max(worst, rel(f64(outs[0][i]), oracle.newton_schulz(f64(x[i]))))
    say(f"   worst rel err {worst:.3e}")
    assert worst <= TOL_NS["bf16"]


def test_step_split_small_units_with_a_zero_unit(gpu_lib):
    # 12 units of 128 x 1100 are too few to fill the GPU one workgroup each:
    # each is split over several workgroups that sum their partial Grams.
    # Unit 5's gradient stays zero (its groups only decay the weight and
    # never wait on each other); two steps against the oracle.
    say("[step split small units]")
    shape = (12, 128, 1100)
    w0 = _seeded(shape, 71, 0.02)
    grads = []
    for t in range(2):
        g = _seeded(shape, 720 + t, 1e-3)
        g[5].zero_()
        grads.append(g.to(torch.bfloat16))
    h = gpu_lib.Hyper()
    tr = gpu_lib.Trace(gpu_lib.KERNEL_NS_SMALL, 2)
    gpu_lib.step([w0.clone()], [grads[0]], [torch.zeros_like(w0)], hyper=h, trace=tr)
    torch.cuda.synchronize()
    assert tr.info() == [(128, 1100, 12, 128)]  # one on-chip launch for the pass
    w = w0.clone()
    m = torch.zeros_like(w0)
    hw = oracle_hyper(h)
    w_ref = {i: f64(w0[i]) for i in (0, 5, 11)}
    m_ref = {i: np.zeros((128, 1100)) for i in (0, 5, 11)}
    for t, g in enumerate(grads, start=1):
        gpu_lib.step([w], [g], [m], hyper=h)
        torch.cuda.synchronize()
        for i in w_ref:
            w_ref[i], m_ref[i], _ = oracle.muon_step(w_ref[i], f64(g[i]), m_ref[i], hw, 0, t)
            assert rel(f64(m[i]), m_ref[i]) <= TOL_M
            check_weight(f64(w[i]), w_ref[i], f64(w0[i]), t, h, TOL_NS["bf16"], f"step {t} unit {i}")
    assert torch.count_nonzero(m[5]).item() == 0


# The tiled bf16 path folds 1/||N|| into the first iteration (its fp32 Gram
# accumulates products of N's raw entries) inside a range of norms and
# scales the iterate first outside it; NS is scale invariant, so every scale
# must give the oracle's result.
@pytest.mark.parametrize("sched", ["persistent", "launches"])
@pytest.mark.parametrize("scale", [2.0**-70, 2.0**-30, 1.0, 2.0**30, 2.0**70],
                         ids=["2^-70", "2^-30", "1", "2^30", "2^70"])
def test_ns_bf16_folded_normalisation_any_scale(gpu_lib, scale, sched):
    say(f"[ns fold] scale={scale:.3e} schedule={sched}")
    worst = 0.0
    for shape in [(2, 300, 200), (2, 200, 520)]:
        x = _seeded(shape, 606 + shape[2], scale)
        h = gpu_lib.Hyper(ns_precision="bf16", schedule=sched)
        outs, _ = gpu_lib.newton_schulz([x], hyper=h)
        torch.cuda.synchronize()
        for i in range(shape[0]):
            worst = max(worst, rel(f64(outs[0][i]), oracle.newton_schulz(f64(x[i]))))
    say(f"   worst rel err {worst:.3e}")
    assert worst <= TOL_NS["bf16"]


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_ns_split_heads_and_banks(gpu_lib, prec):
    # A (batch=3, 6*32, 96) bank split into 32-row heads: 18 units.
    say(f"[ns split] prec={prec}")
    x = _seeded((3, 192, 96), 77)
    h = gpu_lib.Hyper(ns_precision=prec)
    outs, _ = gpu_lib.newton_schulz([x], hyper=h, split_rows=[32])
    torch.cuda.synchronize()
    xo, oo = f64(x), f64(outs[0])
    worst = 0.0
    for b in range(3):
        for hd in range(6):
            blk = slice(hd * 32, (hd + 1) * 32)
            worst = max(worst, rel(oo[b, blk], oracle.newton_schulz(xo[b, blk])))
    say(f"   worst rel err {worst:.3e}")
    assert worst <= TOL_NS[prec]


# A caller's own schedule of up to four stages: a zero-step stage (skipped),
# a cubic stage (c = 0: X <- 1.5 X - 0.5 (X X^T) X) and the two of the pages.
CUSTOM_STAGES = [(3, (3.4445, -4.7750, 2.0315)), (0, (1.0, 1.0, 1.0)), (2, (1.5, -0.5, 0.0)),
                 (1, (2.0, -1.5, 0.5))]


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 256, 512), (2, 200, 300), (2, 128, 300)],
                         ids=["tiles-256", "tiles-128", "128-rows"])  # 128 rows: on chip in bf16
def test_ns_custom_stages_match_oracle(gpu_lib, shape, prec):
    say(f"[ns custom stages] shape={shape} prec={prec}")
    x = _seeded(shape, 777 + shape[1])
    h = gpu_lib.Hyper(ns_precision=prec, stages=CUSTOM_STAGES)
    outs, _ = gpu_lib.newton_schulz([x], hyper=h)
    torch.cuda.synchronize()
    sched = tuple((k, tuple(c)) for k, c in CUSTOM_STAGES)
    worst = 0.0
    for i in range(shape[0]):
        ref = oracle.newton_schulz(f64(x[i]), schedule=sched)
        worst = max(worst, rel(f64(outs[0][i]), ref))
    say(f"   worst rel err {worst:.3e}")
    assert worst <= TOL_NS[prec]


def test_ns_zero_unit_gives_zero(gpu_lib):
    x = _seeded((2, 64, 128), 5)
    x[1].zero_()
    outs, _ = gpu_lib.newton_schulz([x], hyper=gpu_lib.Hyper())
    torch.cuda.synchronize()
    assert torch.count_nonzero(outs[0][1]).item() == 0
    assert rel(f64(outs[0][0]), oracle.newton_schulz(f64(x[0]))) <= TOL_NS["bf16"]


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_batch_vs_single_bitwise(gpu_lib, prec):
    # RFC-0023 risk list: stacking must not change results.  The kernels
    # are deterministic and per-unit, so stacked, chunked and single runs
    # must agree bit for bit.
    say(f"[batch-vs-single] prec={prec}")
    xs = _seeded((5, 200, 300), 11)
    h = gpu_lib.Hyper(ns_precision=prec)
    stacked, _ = gpu_lib.newton_schulz([xs], hyper=h)
    h2 = gpu_lib.Hyper(ns_precision=prec, batch_update_size=2)
    chunked, _ = gpu_lib.newton_schulz([xs], hyper=h2)
    singles = [gpu_lib.newton_schulz([xs[i].clone()], hyper=h)[0][0] for i in range(5)]
    torch.cuda.synchronize()
    assert torch.equal(stacked[0], chunked[0])
    for i in range(5):
        assert torch.equal(stacked[0][i], singles[i])


# The NS-only entry may write its output over its input: tiled (96 x 160),
# and the one-launch step, which reads the whole unit before it writes any
# of it (64 x 128 bf16, 48 x 100 fp32).
@pytest.mark.parametrize("shape,prec", [((96, 160), "fp32"), ((64, 128), "bf16"), ((48, 100), "fp32")],
                         ids=["tiled", "one-launch-bf16", "one-launch-fp32"])
def test_ns_in_place(gpu_lib, shape, prec):
    x = _seeded(shape, 21)
    ref = oracle.newton_schulz(f64(x))
    gpu_lib.newton_schulz([x], outs=[x], hyper=gpu_lib.Hyper(ns_precision=prec))
    torch.cuda.synchronize()
    assert rel(f64(x), ref) <= TOL_NS[prec]


# -------------------------------------------------------------- step --------
def _run_steps(gpu_lib, w0, grads, h, split_rows=0):
    """Run len(grads) GPU steps and the oracle alongside; return per-step
    (W_gpu, M_gpu, W_ref, M_ref)."""
    w = w0.clone()
    m = torch.zeros_like(w0)
    hw = oracle_hyper(h)
    w_ref = f64(w0)
    m_ref = np.zeros_like(w_ref)
    out = []
    for t, g in enumerate(grads, start=1):
        ht = dataclasses.replace(h, step=t)  # the EMA style's bias corrections use the step index
        gpu_lib.step([w], [g], [m], hyper=ht, split_rows=[split_rows])
        torch.cuda.synchronize()
        g64 = f64(g)
        if w_ref.ndim == 3:
            for b in range(w_ref.shape[0]):
                w_ref[b], m_ref[b], _ = oracle.muon_step(w_ref[b], g64[b], m_ref[b], hw, split_rows, t)
        else:
            w_ref, m_ref, _ = oracle.muon_step(w_ref, g64, m_ref, hw, split_rows, t)
        out.append((f64(w), f64(m), w_ref.copy(), m_ref.copy()))
    return out


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_step_single_fp32_matrix_workload(gpu_lib, prec):
    # 64x128 fp32 weight ~ N(0, 0.02), five steps of fp32 N(0, 1) grads,
    # momentum from zero, spectral scale.
    say(f"[step 64x128] prec={prec}")
    wl = W.workload(1)
    w0 = W.init_weight(wl, 0, (64, 128)).to(DEV)
    grads = [W.grad_tensor(wl, t, 0, (64, 128), "fp32").to(DEV) for t in range(wl.steps)]
    h = gpu_lib.Hyper(ns_precision=prec)
    res = _run_steps(gpu_lib, w0, grads, h)
    w0_64 = f64(w0)
    for t, (wg, mg, wr, mr) in enumerate(res, start=1):
        assert rel(mg, mr) <= TOL_M, f"step {t} momentum"
        e = check_weight(wg, wr, w0_64, t, h, TOL_NS[prec], f"step {t}")
        say(f"   step {t}: rel update err {e:.3e}")


# Every block-count variant of the one-launch small step (rows and columns
# in 32-blocks: 1 <= BS <= BL <= 4 with bf16 products, BS <= 2 with fp32
# ones; fp32 units of more than 64 rows take the tiled products), NS only,
# two units each.
ONE_BLOCK_NS = [(31, 32), (20, 50), (10, 90), (1, 100), (33, 64), (40, 70), (64, 128), (70, 90),
                (65, 128), (100, 128)]


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", ONE_BLOCK_NS, ids=[f"{r}x{c}" for r, c in ONE_BLOCK_NS])
def test_ns_one_block_variants(gpu_lib, shape, prec):
    say(f"[ns one-block] shape={shape} prec={prec}")
    x = _seeded((2, *shape), 3300 + shape[0] * 131 + shape[1])
    outs, _ = gpu_lib.newton_schulz([x], hyper=gpu_lib.Hyper(ns_precision=prec))
    torch.cuda.synchronize()
    worst = max(rel(f64(outs[0][i]), oracle.newton_schulz(f64(x[i]))) for i in range(2))
    say(f"   worst rel err {worst:.3e}")
    assert worst <= TOL_NS[prec]


# Units whose wide form fits one 128 x 128 block take the one-launch step
# (momentum, norm, on-chip Newton-Schulz and update in one workgroup per
# unit): 32-row heads, an odd width (the scalar loads and stores), a single
# row, fp32 and bf16 gradients, both look-ahead styles, and a unit whose
# gradient stays zero (pure decay); bf16 products, and fp32 ones where the
# units have at most 64 rows.
ONE_BLOCK = [
    ((3, 96, 128), 32, "bf16", "sgd", "bf16"),
    ((5, 100, 125), 0, "fp32", "sgd", "bf16"),
    ((2, 1, 7), 0, "fp32", "ema", "bf16"),
    ((4, 64, 128), 0, "bf16", "ema", "bf16"),
    ((3, 96, 128), 32, "bf16", "sgd", "fp32"),
    ((5, 60, 125), 0, "fp32", "sgd", "fp32"),
    ((4, 64, 128), 0, "bf16", "ema", "fp32"),
]


@pytest.mark.parametrize("case", range(len(ONE_BLOCK)),
                         ids=["heads", "odd-width", "one-row", "ema-zero-unit", "heads-fp32",
                              "odd-width-fp32", "ema-zero-unit-fp32"])
def test_step_one_block_units(gpu_lib, case):
    shape, split, gdt, style, prec = ONE_BLOCK[case]
    say(f"[step one-block] shape={shape} split={split} grads={gdt} style={style} ns={prec}")
    w0 = _seeded(shape, 61 + case, 0.02)
    grads = []
    for t in range(3):
        g = _seeded(shape, 610 + 10 * case + t, 1e-3)
        if shape == (4, 64, 128):
            g[1].zero_()
        grads.append(g.to(torch.bfloat16) if gdt == "bf16" else g)
    h = gpu_lib.Hyper(ns_precision=prec, nesterov_style=style)
    res = _run_steps(gpu_lib, w0, grads, h, split_rows=split)
    w0_64 = f64(w0)
    rows = split or shape[1]
    for t, (wg, mg, wr, mr) in enumerate(res, start=1):
        assert rel(mg, mr) <= TOL_M, f"step {t} momentum"
        for b in range(shape[0]):
            for hd in range(shape[1] // rows):
                blk = slice(hd * rows, (hd + 1) * rows)
                check_weight(wg[b, blk], wr[b, blk], w0_64[b, blk], t, h, TOL_NS[prec],
                             f"step {t} matrix {b} head {hd}")
    if shape == (4, 64, 128):
        assert torch.count_nonzero(torch.from_numpy(res[-1][1][1])).item() == 0


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_step_ema_nesterov_style(gpu_lib, prec):
    # The EMA look-ahead with bias corrections (RFC-0023 方案 1, optax
    # style), four steps, split heads and one all-zero unit in the bank.
    say(f"[step ema] prec={prec}")
    w0 = _seeded((3, 256, 384), 41, 0.02)
    grads = []
    for t in range(4):
        g = _seeded((3, 256, 384), 500 + t, 1e-3)
        g[1, 128:].zero_()  # the second head of matrix 1 stays zero
        grads.append(g.to(torch.bfloat16))
    h = gpu_lib.Hyper(ns_precision=prec, nesterov_style="ema")
    res = _run_steps(gpu_lib, w0, grads, h, split_rows=128)
    w0_64 = f64(w0)
    for t, (wg, mg, wr, mr) in enumerate(res, start=1):
        assert rel(mg, mr) <= TOL_M, f"step {t} momentum"
        for b in range(3):
            for hd in range(2):
                blk = slice(hd * 128, (hd + 1) * 128)
                check_weight(wg[b, blk], wr[b, blk], w0_64[b, blk], t, h, TOL_NS[prec],
                             f"step {t} matrix {b} head {hd}")


def test_step_zero_gradient_is_pure_decay(gpu_lib):
    w0 = _seeded((2, 200, 300), 3, 0.02)
    g = torch.zeros_like(w0, dtype=torch.bfloat16)
    w = w0.clone()
    m = torch.zeros_like(w0)
    gpu_lib.step([w], [g], [m])
    torch.cuda.synchronize()
    d = np.float32(1.0 - np.float64(np.float32(2.7e-4)) * np.float64(np.float32(0.1)))
    expect = f64(w0).astype(np.float32) * d
    assert torch.count_nonzero(m).item() == 0
    np.testing.assert_array_max_ulp(f64(w).astype(np.float32), expect, maxulp=1)


def test_step_split_heads_bf16_studentt(gpu_lib):
    # A fused 6-head QKV-like bank with 64-row heads, Student-t grads.
    say("[step split heads]")
    w0 = _seeded((384, 256), 8, 0.02)
    grads = []
    for t in range(3):
        g = torch.Generator(device="cpu").manual_seed(900 + t)
        z = torch.randn((384, 256), generator=g)
        chi = sum(torch.randn((384, 256), generator=g) ** 2 for _ in range(3))
        grads.append((z / torch.sqrt(chi / 3) * 1e-3).to(torch.bfloat16).to(DEV))
    h = gpu_lib.Hyper()
    res = _run_steps(gpu_lib, w0, grads, h, split_rows=64)
    w0_64 = f64(w0)
    for t, (wg, mg, wr, mr) in enumerate(res, start=1):
        assert rel(mg, mr) <= TOL_M
        for hd in range(6):
            blk = slice(hd * 64, (hd + 1) * 64)
            check_weight(wg[blk], wr[blk], w0_64[blk], t, h, TOL_NS["bf16"], f"step {t} head {hd}")


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_step_stacked_1024_workload_sampled(gpu_lib, prec):
    # The benchmark workload: 32 stacked 1024x1024 fp32 weights, bf16 grads
    # N(0, 1e-3), ten steps, spectral scale.  The GPU updates the whole
    # stack; the oracle follows three sampled matrices through every step.
    say(f"[step 32x1024^2] prec={prec}")
    wl = W.workload(2)
    w = W.bank_weights(wl, 0, DEV)
    w0 = f64(w)
    m = torch.zeros_like(w)
    h = gpu_lib.Hyper(ns_precision=prec)
    hw = oracle_hyper(h)
    sample = [0, 13, 31]
    w_ref = {i: w0[i].copy() for i in sample}
    m_ref = {i: np.zeros((1024, 1024)) for i in sample}
    steps = wl.steps if prec == "bf16" else 3
    for t in range(1, steps + 1):
        g = W.bank_grads(wl, t - 1, 0, DEV)
        gpu_lib.step([w], [g], [m], hyper=h)
        torch.cuda.synchronize()
        for i in sample:
            w_ref[i], m_ref[i], _ = oracle.muon_step(w_ref[i], f64(g[i]), m_ref[i], hw, 0, t)
        for i in sample:
            assert rel(f64(m[i]), m_ref[i]) <= TOL_M
            e = check_weight(f64(w[i]), w_ref[i], w0[i], t, h, TOL_NS[prec], f"step {t} mat {i}")
        say(f"   step {t}: last rel update err {e:.3e}")


# ---------------------------------------- tall and wide units in one pass ---
# A tall unit and a wide unit of the same two sides stack in one pass, in the
# tall form: the wide unit's look-ahead is transposed into the iterate and its
# update written back transposed.  unit_rms_norm gives them different scales
# (sqrt(fan_out / fan_in)).  Odd caller widths take the scalar paths of the
# transposing kernels; split heads of 128 x 600 are transposed head by head.
MIXED = [
    [(2, 600, 260, 0), (3, 260, 600, 0)],            # 256 tiles, both forms
    [(1, 1001, 300, 0), (2, 300, 1001, 0)],          # odd caller widths
    [(1, 512, 600, 128), (2, 600, 128, 0)],          # transposed heads with tall units
]


@pytest.mark.parametrize("sched", ["auto", "persistent", "launches"])
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("case", range(len(MIXED)))
def test_step_tall_and_wide_units_in_one_pass(gpu_lib, case, prec, sched):
    banks = MIXED[case]
    say(f"[mixed] {banks} prec={prec} sched={sched}")
    h = gpu_lib.Hyper(ns_precision=prec, schedule=sched, scale="unit_rms_norm")
    hw = oracle_hyper(h)
    g = torch.Generator(device="cpu").manual_seed(77 + case)
    w0 = [torch.randn((b, r, c), generator=g) * 0.02 for b, r, c, _ in banks]
    grads = [[(torch.randn((b, r, c), generator=g) * 1e-3).to(torch.bfloat16)
              for b, r, c, _ in banks] for _ in range(2)]
    splits = [s for *_, s in banks]
    params = [w.to(DEV) for w in w0]
    moms = [torch.zeros_like(p) for p in params]
    refs = [[(f64(w[i]), np.zeros(w[i].shape)) for i in range(w.shape[0])] for w in w0]
    for t in (1, 2):
        gpu_lib.step(params, [gr.to(DEV) for gr in grads[t - 1]], moms, hyper=h, split_rows=splits)
        torch.cuda.synchronize()
        for k, (b, r, c, sp) in enumerate(banks):
            for i in range(b):
                wr, mr = refs[k][i]
                wr, mr, _ = oracle.muon_step(wr, f64(grads[t - 1][k][i]), mr, hw, sp, t)
                refs[k][i] = (wr, mr)
                assert rel(f64(moms[k][i]), mr) <= TOL_M
                blocks = [slice(0, r)] if not sp else [slice(j, j + sp) for j in range(0, r, sp)]
                for blk in blocks:
                    check_weight(f64(params[k][i])[blk], wr[blk], f64(w0[k][i])[blk], t, h,
                                 TOL_NS[prec], f"bank {k} unit {i} rows {blk}")


@pytest.mark.parametrize("sched", ["persistent", "launches"])
def test_wide_unit_alone_or_stacked_with_tall_units_bitwise(gpu_lib, sched):
    # a unit's form depends on its own shape only: a wide unit gives the same
    # bits alone and stacked with tall units of the same sides
    say(f"[mixed bitwise] sched={sched}")
    g = torch.Generator(device="cpu").manual_seed(5)
    wide = (torch.randn((2, 300, 700), generator=g) * 0.02).to(DEV)
    tall = (torch.randn((3, 700, 300), generator=g) * 0.02).to(DEV)
    gw = (torch.randn((2, 300, 700), generator=g) * 1e-3).to(torch.bfloat16).to(DEV)
    gt = (torch.randn((3, 700, 300), generator=g) * 1e-3).to(torch.bfloat16).to(DEV)
    h = gpu_lib.Hyper(schedule=sched)
    a_w, a_m = wide.clone(), torch.zeros_like(wide)
    gpu_lib.step([a_w], [gw], [a_m], hyper=h)
    b_w, b_m = wide.clone(), torch.zeros_like(wide)
    t_w, t_m = tall.clone(), torch.zeros_like(tall)
    gpu_lib.step([t_w, b_w], [gt, gw], [t_m, b_m], hyper=h)
    torch.cuda.synchronize()
    assert torch.equal(a_w, b_w) and torch.equal(a_m, b_m)
