"""The persistent NS launch (one launch per stacked pass, workgroups
claiming tiles and waiting on per-panel completion counts) against one launch
per product: both run the same tile code on the same inputs, so their
results must agree bit for bit, and the persistent launch must report a
clean status."""

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"

# (banks as (batch, rows, cols, split_rows), grad dtype, NS precision)
CASES = [
    ([(6, 256, 384, 0)], "bf16", "bf16"),            # 256 tiles, ragged
    ([(4, 100, 200, 0), (3, 300, 200, 0)], "fp32", "bf16"),  # 128 tiles, wide and tall
    ([(2, 512, 256, 128)], "bf16", "bf16"),           # split heads
    ([(3, 640, 256, 0)], "bf16", "fp32"),             # tall, fp32 products
    ([(5, 256, 256, 0)], "fp32", "fp32"),             # fp32 path, 256 tiles
    ([(1, 1024, 2048, 0)], "bf16", "bf16"),           # one unit, many tiles
    # full-size units: 16 panels of 256 on the small side
    ([(2, 14336, 4096, 0)], "bf16", "bf16"),          # the layer's gate/up, one queue
    ([(1, 4096, 14336, 0)], "bf16", "bf16"),          # its down projection
    ([(16, 2048, 7168, 0)], "bf16", "bf16"),          # MoE experts, one queue per XCC
]


def _bank(shape, seed, gdtype):
    b, r, c, _ = shape
    g = torch.Generator(device="cpu").manual_seed(seed)
    w = (torch.randn((b, r, c), generator=g) * 0.02).to(DEV)
    gr = (torch.randn((b, r, c), generator=g) * 1e-3).to(DEV)
    if b > 1:
        gr[b // 2].zero_()  # one all-zero unit per bank
    return w, gr.to(torch.bfloat16 if gdtype == "bf16" else torch.float32)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_step_schedules_agree_bitwise(gpu_lib, case):
    banks, gdtype, prec = CASES[case]
    print(f"[schedule] case {case}: {banks} grads {gdtype} products {prec}", flush=True)
    splits = [s[3] for s in banks]
    inputs = [_bank(s, 100 + 17 * i, gdtype) for i, s in enumerate(banks)]
    out = {}
    for sched in ("launches", "persistent"):
        h = gpu_lib.Hyper(ns_precision=prec, schedule=sched)
        params = [w.clone() for w, _ in inputs]
        moms = [torch.zeros_like(w) for w, _ in inputs]
        ws = gpu_lib.workspace(gpu_lib.workspace_size(params, h, splits), torch.device(DEV))
        for t in range(2):  # two steps: the second starts from a live momentum
            gpu_lib.step(params, [g for _, g in inputs], moms, hyper=h, split_rows=splits, ws=ws)
        gpu_lib.workspace_status(ws)
        out[sched] = (params, moms)
    for i in range(len(banks)):
        assert torch.equal(out["launches"][0][i], out["persistent"][0][i]), f"params of bank {i}"
        assert torch.equal(out["launches"][1][i], out["persistent"][1][i]), f"momenta of bank {i}"


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_ns_only_schedules_agree_bitwise(gpu_lib, prec):
    print(f"[schedule ns] prec {prec}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(9)
    xs = [torch.randn((7, 384, 256), generator=g).to(DEV), torch.randn((2, 130, 700), generator=g).to(DEV)]
    res = {}
    for sched in ("launches", "persistent"):
        h = gpu_lib.Hyper(ns_precision=prec, schedule=sched)
        outs, _ = gpu_lib.newton_schulz(xs, hyper=h)
        torch.cuda.synchronize()
        res[sched] = outs
    for a, b in zip(res["launches"], res["persistent"]):
        assert torch.equal(a, b)


def test_persistent_trace_brackets_one_launch_per_pass(gpu_lib):
    print("[schedule trace]", flush=True)
    x = torch.randn((4, 256, 300), device=DEV)
    h = gpu_lib.Hyper(schedule="persistent")
    tr = gpu_lib.Trace(gpu_lib.KERNEL_NS, 4)
    _, n = gpu_lib.newton_schulz([x], hyper=h, trace=tr)
    torch.cuda.synchronize()
    assert n == 1
    assert tr.ms()[0] > 0
    assert tr.info() == [(256, 300, 4, 256)]  # s, l, units, tile
    h = gpu_lib.Hyper(schedule="launches")
    tr = gpu_lib.Trace(gpu_lib.KERNEL_APPLY, 4)
    _, n = gpu_lib.newton_schulz([x], hyper=h, trace=tr)
    torch.cuda.synchronize()
    assert n == 10 and tr.recorded == 4
    tr = gpu_lib.Trace(gpu_lib.KERNEL_MOMENTUM, 2)
    _, n = gpu_lib.newton_schulz([x], hyper=h, trace=tr)
    torch.cuda.synchronize()
    # NS only: the fp32 input read (4 B) and N written into the bf16 iterate (2 B)
    assert n == 1 and tr.info() == [(4 * 256 * 300, 6 * 4 * 256 * 300, 4, 0)]


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_one_block_units_take_one_launch(gpu_lib, prec):
    # Wide units of at most 128 x 128 (at most 64 rows with fp32 products):
    # the whole step is one launch of the small-unit kernel, with no
    # momentum or norm launches.
    print(f"[schedule one-block] prec={prec}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(12)
    w = (torch.randn((3, 64, 128), generator=g) * 0.02).to(DEV)
    gr = (torch.randn((3, 64, 128), generator=g) * 1e-3).to(DEV)
    m = torch.zeros_like(w)
    h = gpu_lib.Hyper(ns_precision=prec)
    counts = {}
    for kind in (gpu_lib.KERNEL_MOMENTUM, gpu_lib.KERNEL_NORMALIZE, gpu_lib.KERNEL_NS_SMALL):
        tr = gpu_lib.Trace(kind, 2)
        counts[kind] = gpu_lib.step([w], [gr], [m], hyper=h, trace=tr)
        torch.cuda.synchronize()
        if kind == gpu_lib.KERNEL_NS_SMALL:
            assert tr.info() == [(64, 128, 3, 128)]
    assert counts == {gpu_lib.KERNEL_MOMENTUM: 0, gpu_lib.KERNEL_NORMALIZE: 0, gpu_lib.KERNEL_NS_SMALL: 1}


@pytest.mark.parametrize("workgroups", [1, 3])
def test_persistent_with_xccs_left_without_workgroups(gpu_lib, workgroups, monkeypatch):
    # 16 units spread over one queue per XCC; a capped grid leaves most XCCs
    # without a workgroup, and the last workgroup to leave runs their queues.
    print(f"[schedule orphan] workgroups {workgroups}", flush=True)
    inputs = [_bank((16, 256, 256, 0), 321, "bf16")]
    out = {}
    for sched in ("launches", "persistent"):
        if sched == "persistent":
            monkeypatch.setenv("MUON_PERSISTENT_WORKGROUPS", str(workgroups))
        h = gpu_lib.Hyper(schedule=sched)
        params = [w.clone() for w, _ in inputs]
        moms = [torch.zeros_like(w) for w, _ in inputs]
        ws = gpu_lib.workspace(gpu_lib.workspace_size(params, h, [0]), torch.device(DEV))
        gpu_lib.step(params, [g for _, g in inputs], moms, hyper=h, split_rows=[0], ws=ws)
        gpu_lib.workspace_status(ws)
        out[sched] = params[0]
    monkeypatch.delenv("MUON_PERSISTENT_WORKGROUPS")
    assert torch.equal(out["launches"], out["persistent"])


# A single 256-tile unit under AUTO runs inside the persistent launch of a
# stacked pass (ns_persistent2) when that pass takes one claim queue.
# (banks, grad dtype, NS precision, index of a bank whose gradient is zero,
# other hyperparameters)
EMA_STAGES = dict(nesterov_style="ema", step=3,
                  stages=((3, (3.4445, -4.7750, 2.0315)), (0, (1.0, 0.0, 0.0)), (2, (2.0, -1.5, 0.5))))
RIDING = [
    # the transformer layer's O projection beside its MLP units (down transposed)
    ([(1, 4096, 4096, 0), (2, 14336, 4096, 0), (1, 4096, 14336, 0)], "bf16", "bf16", None, {}),
    # ragged: s = 300 and 520 on 256 tiles, a zero unit in the stacked pass
    ([(3, 1100, 300, 0), (1, 700, 520, 0)], "bf16", "bf16", None, {}),
    # a riding unit with a zero gradient (pure decay in its final epilogue)
    ([(2, 640, 256, 0), (1, 512, 384, 0)], "fp32", "bf16", 1, {}),
    # fp32 products; the riding unit is wide, stored transposed
    ([(2, 640, 256, 0), (1, 300, 700, 0)], "bf16", "fp32", None, {}),
    # EMA look-ahead, three stages (one of zero steps), unit_rms_norm scale
    ([(2, 640, 256, 0), (1, 300, 700, 0)], "bf16", "bf16", None, dict(EMA_STAGES, scale="unit_rms_norm")),
    # batch_update_size cuts one bank into passes of two units and one: the
    # single unit rides with a pass of its own shape
    ([(3, 768, 512, 0)], "bf16", "bf16", None, dict(batch_update_size=2)),
]


def _run_steps(gpu_lib, banks, inputs, sched, prec, trace_kinds=(), extra=None):
    splits = [b[3] for b in banks]
    h = gpu_lib.Hyper(ns_precision=prec, schedule=sched, **(extra or {}))
    params = [w.clone() for w, _ in inputs]
    moms = [torch.zeros_like(w) for w, _ in inputs]
    ws = gpu_lib.workspace(gpu_lib.workspace_size(params, h, splits), torch.device(DEV))
    traces = {}
    for t in range(2):  # the second step starts from a live momentum
        gpu_lib.step(params, [g for _, g in inputs], moms, hyper=h, split_rows=splits, ws=ws)
    for kind in trace_kinds:
        tr = gpu_lib.Trace(kind, 8)
        n = gpu_lib.step([w.clone() for w in params], [g for _, g in inputs],
                         [m.clone() for m in moms], hyper=h, split_rows=splits, ws=ws, trace=tr)
        torch.cuda.synchronize()
        traces[kind] = (n, tr.info()[:n])
    gpu_lib.workspace_status(ws)
    return params, moms, traces


@pytest.mark.parametrize("case", range(len(RIDING)))
def test_riding_pass_agrees_bitwise_with_launches(gpu_lib, case):
    banks, gdtype, prec, zero, extra = RIDING[case]
    print(f"[schedule riding] case {case}: {banks} grads {gdtype} products {prec} {extra}", flush=True)
    inputs = [_bank(s, 500 + 13 * i, gdtype) for i, s in enumerate(banks)]
    if zero is not None:
        inputs[zero][1].zero_()
    kinds = (gpu_lib.KERNEL_NS, gpu_lib.KERNEL_GRAM)
    pa, ma, tra = _run_steps(gpu_lib, banks, inputs, "auto", prec, kinds, extra)
    pl, ml, _ = _run_steps(gpu_lib, banks, inputs, "launches", prec, extra=extra)
    for i in range(len(banks)):
        assert torch.equal(pa[i], pl[i]), f"params of bank {i}"
        assert torch.equal(ma[i], ml[i]), f"momenta of bank {i}"
    # one NS launch carries both passes, and no per-product launch runs
    n_ns, info = tra[gpu_lib.KERNEL_NS]
    assert n_ns == 1 and tra[gpu_lib.KERNEL_GRAM][0] == 0
    passes = gpu_lib.ns_passes(info[0])
    assert len(passes) == 2 and passes[1][2] == 1 and all(p[3] == 256 for p in passes)
    if zero is not None:
        w0 = inputs[zero][0]
        decay = 1.0 - 2.7e-4 * 0.1
        expect = w0 * decay * decay
        assert torch.allclose(pa[zero], expect, rtol=1e-6, atol=0)


def test_riding_pass_ns_only(gpu_lib):
    # the NS-only entry: the riding unit's final epilogue writes its output
    print("[schedule riding ns-only]", flush=True)
    g = torch.Generator(device="cpu").manual_seed(31)
    xs = [torch.randn((3, 384, 256), generator=g).to(DEV), torch.randn((1, 300, 520), generator=g).to(DEV)]
    res = {}
    for sched in ("auto", "launches"):
        tr = gpu_lib.Trace(gpu_lib.KERNEL_NS, 4)
        outs, n = gpu_lib.newton_schulz(xs, hyper=gpu_lib.Hyper(schedule=sched), trace=tr)
        torch.cuda.synchronize()
        res[sched] = (outs, n, tr.info()[:n])
    for a, b in zip(res["auto"][0], res["launches"][0]):
        assert torch.equal(a, b)
    assert res["auto"][1] == 1 and gpu_lib.ns_passes(res["auto"][2][0]) == [(256, 384, 3, 256),
                                                                         (300, 520, 1, 256)]
    assert res["launches"][1] == 0


@pytest.mark.parametrize("workgroups", [1, 3])
def test_riding_pass_with_few_workgroups(gpu_lib, workgroups, monkeypatch):
    # A capped grid: one or three workgroups claim every item of both passes
    # in order, which still completes (each item waits only for earlier
    # ones) and gives the per-product launches' result.
    print(f"[schedule riding] {workgroups} workgroups", flush=True)
    banks = [(2, 640, 256, 0), (1, 512, 384, 0)]
    inputs = [_bank(s, 900 + i, "bf16") for i, s in enumerate(banks)]
    pl, ml, _ = _run_steps(gpu_lib, banks, inputs, "launches", "bf16")
    monkeypatch.setenv("MUON_PERSISTENT_WORKGROUPS", str(workgroups))
    pa, ma, tra = _run_steps(gpu_lib, banks, inputs, "auto", "bf16", (gpu_lib.KERNEL_NS,))
    monkeypatch.delenv("MUON_PERSISTENT_WORKGROUPS")
    assert tra[gpu_lib.KERNEL_NS][0] == 1 and len(gpu_lib.ns_passes(tra[gpu_lib.KERNEL_NS][1][0])) == 2
    for i in range(len(banks)):
        assert torch.equal(pa[i], pl[i]) and torch.equal(ma[i], ml[i]), f"bank {i}"


def test_no_riding_beside_xcc_local_queues(gpu_lib):
    # A stacked pass that spreads over one queue per XCC keeps them; the
    # single unit then runs its own launches (results unchanged).
    print("[schedule riding local queues]", flush=True)
    banks = [(16, 256, 256, 0), (1, 512, 256, 0)]
    inputs = [_bank(s, 700 + i, "bf16") for i, s in enumerate(banks)]
    kinds = (gpu_lib.KERNEL_NS, gpu_lib.KERNEL_GRAM)
    pa, _, tra = _run_steps(gpu_lib, banks, inputs, "auto", "bf16", kinds)
    pl, _, _ = _run_steps(gpu_lib, banks, inputs, "launches", "bf16")
    for a, b in zip(pa, pl):
        assert torch.equal(a, b)
    n_ns, info = tra[gpu_lib.KERNEL_NS]
    assert n_ns == 1 and gpu_lib.ns_passes(info[0]) == [(256, 256, 16, 256)]
    assert tra[gpu_lib.KERNEL_GRAM][0] == 10


_FRESH = r"""
import sys
import torch
sys.path.insert(0, sys.argv[1])
from newton_schulz_matrix_muon_amd import muon
g = torch.Generator().manual_seed(int(sys.argv[2]))
shapes = [(4, 100, 200), (3, 300, 200), (6, 256, 384)]  # one queue each; 128- and 256-row tiles
xs = [torch.randn(s, generator=g).cuda() for s in shapes]
res = {}
for sched in ("persistent", "launches"):  # the persistent launch is the process's first
    outs, _ = muon.newton_schulz(xs, hyper=muon.Hyper(schedule=sched))
    torch.cuda.synchronize()
    res[sched] = [o.cpu() for o in outs]
same = all(torch.equal(a, b) for a, b in zip(res["persistent"], res["launches"]))
print("agree" if same else "differ", flush=True)
sys.exit(0 if same else 3)
"""


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_single_queue_first_launch_of_a_fresh_process(seed):
    # Units on one queue run their tiles on several XCCs, so a tile is
    # published through an L2 write-back; the first persistent launch of a
    # fresh process, on small single-queue units, is checked bit for bit
    # against the per-product launches.  One child process at a time.
    import os
    import subprocess
    import sys

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print(f"[schedule fresh process] seed {seed}", flush=True)
    r = subprocess.run([sys.executable, "-c", _FRESH, root, str(seed)], capture_output=True, text=True,
                       timeout=180)
    assert r.returncode == 0 and "agree" in r.stdout, (r.returncode, r.stdout[-500:], r.stderr[-2000:])
