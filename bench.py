"""Benchmark of the MI355X Muon step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--ns bf16|fp32]
                    [--no-sub-configs] [--no-cpu-baseline]

A step is one Muon update (momentum, Nesterov look-ahead, Frobenius
normalisation, ten hybrid Newton-Schulz iterations, scale and decoupled
weight decay) of every matrix of a workload, with its inputs resident in
HBM.  The headline workload is the largest one that fits one GPU: 32
transformer layers of hidden 4096 (~7B parameters, 1664 NS units: 1536
split heads of 128 x 4096, 32 projections of 4096 x 4096, 96 MLP matrices
of 4096 x 14336 / 14336 x 4096), unit_rms_norm scale, bf16 NS products
with fp32 accumulation.  Its W warm-up steps are followed by exactly K
timed steps.

The one JSON line also carries, measured in the same run:
  * `configs`: every other workload (the single 64 x 128 fp32 matrix on both
    NS paths, 32 stacked 1024^2, one transformer layer, the MoE bank) and a
    sampled step of the headline workload on the fp32 NS path;
  * `roofline`: the dominant NS kernel of the headline step, its nominal
    FLOPs per launch over its average launch duration (HIP events around
    each launch, on the step's stream, over the timed steps);
  * `cpu_baseline`: the float64 oracle on one sampled unit per unit shape,
    extrapolated to a whole step.
A line is printed only if no persistent launch stopped early (the
workspace status is read after the warm-up, the traced and the timed
steps).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp32": 157.3}  # MI355X dense MFMA
HBM_GBS = 8000.0
HEADLINE = 5
# Other workloads of the same run: (config, NS path, timed steps, warm-up
# steps, per-class traced steps)
SUB_CONFIGS = [
    (1, "fp32", 200, 20, True),
    (1, "bf16", 200, 20, True),
    (2, "bf16", 50, 5, True),
    (3, "bf16", 10, 2, True),
    (4, "bf16", 3, 1, True),
]
FP32_SAMPLE_STEPS = 1  # the headline workload on the fp32 NS path

KERNEL_NAMES = {
    "ns": "ns_persistent",
    "ns_small": "k_ns_small",
    "gram": "ns_gemm gram",
    "poly": "ns_gemm poly",
    "apply": "ns_gemm apply",
}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=HEADLINE, help="headline workload (1-5)")
    ap.add_argument("--ns", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--schedule", default="auto", choices=["auto", "persistent", "launches"],
                    help="NS schedule: the library's choice per pass, or force one persistent "
                         "launch per pass, or one launch per product")
    ap.add_argument("--grad-sets", type=int, default=2, help="distinct resident gradient batches")
    ap.add_argument("--no-sub-configs", action="store_true",
                    help="measure the headline workload only (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=40.0,
                    help="budget of the CPU-oracle sample; shape groups beyond it are scaled "
                         "by FLOPs from the measured rate")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain copy kernel over this many MiB "
                         "(int32 bitwise-not, read once and written once) for counter calibration")
    return ap.parse_args(argv)


# ------------------------------------------------------------ accounting ---
def kernel_sources_sha256():
    """Digest of the HIP sources, tying a stored counter record to the
    kernels it was taken on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "newton_schulz_matrix_muon_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(kernel, workload, ns, pdir=None, digest=None):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE runs, scaled by a copy kernel of known size),
    or None when there is none for this kernel and workload or the kernel
    sources have changed since it was taken."""
    pdir = pdir or os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    digest = digest or kernel_sources_sha256()
    for name in sorted(os.listdir(pdir)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(pdir, name), encoding="utf-8") as f:
            for line in f:
                if not line.startswith("traffic_record: "):
                    continue
                rec = json.loads(line[len("traffic_record: "):])
                if (rec.get("kernel"), rec.get("workload"), rec.get("ns")) != (kernel, workload, ns):
                    continue
                if rec.get("sources_sha256") != digest:
                    return None
                return rec
    return None


def shape_groups(wl):
    """{(s, l): (units, units with a non-zero gradient)} over the workload's
    NS units, s and l the smaller and the larger side (tall and wide units of
    one (s, l) together); all-zero experts count only in the first figure."""
    import workloads as W

    out = {}
    for spec in wl.matrices:
        r, c = spec.unit_shape
        n = spec.batch * spec.units_per_matrix
        nz = n
        if wl.zero_fraction:
            nz -= len(W.zero_experts(wl, spec.batch)) * spec.units_per_matrix
        key = (min(r, c), max(r, c))
        a, b = out.get(key, (0, 0))
        out[key] = (a + n, b + nz)
    return out


def unit_flops(s, l):
    """Nominal NS FLOPs of one unit per iteration: X X^T (2 s^2 l), A A
    (2 s^3) and B X (2 s^2 l)."""
    return 4.0 * s * s * l + 2.0 * s**3


def ns_flops_per_step(wl, iters):
    """Nominal NS FLOPs of one step over the units with a non-zero gradient."""
    return sum(live * iters * unit_flops(s, l) for (s, l), (_, live) in shape_groups(wl).items())


def executed_fraction(s, tile):
    """Share of a symmetric s x s product's tiles that run (upper triangle of
    the tile grid)."""
    t = -(-s // tile)
    return (t * (t + 1) / 2) / (t * t)


def launch_flops(cls, info, groups, iters):
    """Nominal and executed FLOPs of one NS launch from what the library
    reports it covered (s, l, units, tile), counting only the share of
    units with a non-zero gradient in that unit shape.  One launch of class
    "ns" or "ns_small" runs every iteration; one of "gram", "poly" or
    "apply" runs one.  A persistent launch that also ran a single-unit pass
    reports both passes (muon.ns_passes); their FLOPs add."""
    from newton_schulz_matrix_muon_amd.muon import ns_passes

    nom = exe = 0.0
    for one in ns_passes(info):
        a, b = _pass_flops(cls, one, groups, iters)
        nom += a
        exe += b
    return nom, exe


def _pass_flops(cls, info, groups, iters):
    s, l, units, tile = info
    total, live = groups.get((s, l), (units, units))
    n = units * (live / total if total else 1.0)
    gram, poly, apply = 2.0 * s * s * l, 2.0 * s**3, 2.0 * s * s * l
    if cls == "ns_small":
        if l <= 128:
            # one launch per step: products over the unit's 32-blocks
            sp, lp = -(-s // 32) * 32, -(-l // 32) * 32
        else:
            # streamed: whole products on rows padded to 128, columns to 128-multiples
            sp, lp = 128, -(-l // 128) * 128
        exe = 2.0 * sp * sp * lp * 2 + 2.0 * sp**3
        return n * iters * (gram + poly + apply), n * iters * exe
    f = executed_fraction(s, tile)
    if cls == "ns":
        return n * iters * (gram + poly + apply), n * iters * (f * gram + f * poly + apply)
    nom = {"gram": gram, "poly": poly, "apply": apply}[cls]
    return n * nom, n * nom * (f if cls in ("gram", "poly") else 1.0)


# -------------------------------------------------------------- the runs ---
def build_inputs(wl, dev, grad_sets):
    import torch

    import workloads as W

    params, moms, grads, splits = [], [], [], []
    for i, spec in enumerate(wl.matrices):
        params.append(W.bank_weights(wl, i, dev))
        moms.append(torch.zeros((spec.batch, spec.rows, spec.cols), dtype=torch.float32, device=dev))
        splits.append(spec.split_rows)
    for k in range(grad_sets):
        grads.append([W.bank_grads(wl, k, i, dev) for i in range(len(wl.matrices))])
    return params, moms, grads, splits


def measure(wl, ns, steps, warmup, dev, inputs, schedule="auto", trace_classes=True):
    """Times `steps` steps of workload `wl` after `warmup` untimed ones.

    With trace_classes, one traced step per kernel class (after the warm-up)
    gives each class's kernel time and what its launches covered; the
    timed steps then bracket every launch of the dominant NS class with HIP
    events on the step's stream.  Raises if a persistent launch stopped."""
    import torch

    from newton_schulz_matrix_muon_amd import muon

    params, moms, grads, splits = inputs
    hyper = muon.Hyper(scale=wl.scale, ns_precision=ns, schedule=schedule)
    ws = muon.workspace(muon.workspace_size(params, hyper, splits), dev)
    iters = sum(k for k, _ in hyper.stages)
    groups = shape_groups(wl)

    def one_step(k, trace=None):
        return muon.step(params, grads[k % len(grads)], moms, hyper=hyper, split_rows=splits,
                         ws=ws, trace=trace, check=False)

    for k in range(warmup):
        one_step(k)
    muon.workspace_status(ws)

    classes = {"momentum": muon.KERNEL_MOMENTUM, "normalize": muon.KERNEL_NORMALIZE,
               "ns": muon.KERNEL_NS, "ns_small": muon.KERNEL_NS_SMALL, "gram": muon.KERNEL_GRAM,
               "poly": muon.KERNEL_POLY, "apply": muon.KERNEL_APPLY}
    per_class = {}  # name -> (ms per launch, info per launch) of one step
    if trace_classes:
        for name, kind in classes.items():
            tr = muon.Trace(kind, 1024)
            one_step(warmup, tr)
            torch.cuda.synchronize()
            if tr.count:
                assert tr.count <= tr.capacity, (name, tr.count)
                per_class[name] = (tr.ms(), tr.info())
        muon.workspace_status(ws)
    ns_classes = [n for n in ("ns", "ns_small", "gram", "poly", "apply") if n in per_class]
    dominant = max(ns_classes, key=lambda n: sum(per_class[n][0])) if ns_classes else None

    traces = []
    if dominant:
        count = len(per_class[dominant][0])
        traces = [muon.Trace(classes[dominant], count) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        one_step(k, traces[k] if traces else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    muon.workspace_status(ws)
    sec = (t1 - t0) / steps

    nsf = ns_flops_per_step(wl, iters)
    out = {
        "workload": wl.title,
        "config_index": wl.cfg,
        "ns_path": ns,
        "units": wl.units,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": sec * 1e3,
        "matrices_per_s": wl.units / sec,
        "ns_tflop_per_step": nsf / 1e12,
        # NS FLOPs over the whole step's wall time (elementwise kernels included)
        "ns_tflops_step": nsf / sec / 1e12,
    }
    if not dominant:
        return out, None
    # The dominant class's time per step from the timed steps (the single
    # traced step can run at a different clock); other classes from theirs.
    launch_ms, launch_info = [], []
    for tr in traces:
        launch_ms += tr.ms()
        launch_info += tr.info()
    kernel_ms = {n: sum(per_class[n][0]) for n in per_class}
    kernel_ms[dominant] = sum(launch_ms) / steps
    ns_ms = sum(kernel_ms[n] for n in ns_classes)
    peak = PEAK_TFLOPS[ns]
    out.update({
        "ns_ms_per_step": ns_ms,
        "ns_tflops": nsf / (ns_ms * 1e-3) / 1e12,
        "ns_frac_of_peak": nsf / (ns_ms * 1e-3) / 1e12 / peak,
        "kernel_ms_per_step": {n: round(v, 4) for n, v in kernel_ms.items()},
    })
    mom = per_class.get("momentum")
    if mom:
        mom_bytes = sum(i[1] for i in mom[1])
        out["elementwise_gbs"] = mom_bytes / (sum(mom[0]) * 1e-3) / 1e9
        out["elementwise_frac_of_hbm"] = out["elementwise_gbs"] / HBM_GBS
    nom = exe = 0.0
    for info in launch_info:
        a, b = launch_flops(dominant, info, groups, iters)
        nom += a
        exe += b
    t = sum(launch_ms) * 1e-3
    kernel = kernel_label(dominant, launch_info)
    roof = {
        "bound": "mfma",
        "kernel": kernel,
        "achieved": nom / t / 1e12,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": nom / t / 1e12 / peak,
        "flops_per_launch": nom / len(launch_ms),
        # the symmetric products run only their upper-triangle tiles: the
        # FLOPs the matrix cores execute, and their share of the peak
        "achieved_executed": exe / t / 1e12,
        "frac_executed": exe / t / 1e12 / peak,
        "avg_launch_ms": sum(launch_ms) / len(launch_ms),
        "launches_timed": len(launch_ms),
    }
    out["dominant_kernel"] = roof["kernel"]
    out["dominant_frac"] = roof["frac"]
    out["dominant_passes"] = pass_breakdown(dominant, launch_ms, launch_info, groups, iters, peak)
    return out, roof


def graph_step_us(wl, ns, dev, inputs, reps=500):
    """Microseconds per step of workload `wl` with one step captured in a
    HIP graph and replayed `reps` times: the step's launches without the
    host-side work of each call (argument marshalling, planning).  The
    replays reuse the first gradient set."""
    import torch

    from newton_schulz_matrix_muon_amd import muon

    params, moms, grads, splits = inputs
    hyper = muon.Hyper(scale=wl.scale, ns_precision=ns)
    ws = muon.workspace(muon.workspace_size(params, hyper, splits), dev)

    def one():
        muon.step(params, grads[0], moms, hyper=hyper, split_rows=splits, ws=ws, check=False)

    one()  # first-call set-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one()
    for _ in range(20):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    muon.workspace_status(ws)
    del graph
    return dt * 1e6


def kernel_label(cls, launch_info):
    """Name of the kernel a class's timed launches ran: a persistent launch
    that also ran a single-unit pass is ns_persistent2's."""
    if cls != "ns":
        return KERNEL_NAMES[cls]
    from newton_schulz_matrix_muon_amd.muon import ns_passes

    two = [len(ns_passes(i)) > 1 for i in launch_info]
    return " + ".join(k for k, on in (("ns_persistent", not all(two)), ("ns_persistent2", any(two))) if on)


def pass_breakdown(cls, launch_ms, launch_info, groups, iters, peak):
    """The dominant class's timed launches grouped by the pass they ran
    (unit shape and count): launches, mean ms and nominal TFLOP/s each."""
    from newton_schulz_matrix_muon_amd.muon import ns_passes

    by = {}
    for ms, info in zip(launch_ms, launch_info):
        key = " + ".join(f"{u} x {s}x{l}" for s, l, u, _ in ns_passes(info))
        nom, _ = launch_flops(cls, info, groups, iters)
        e = by.setdefault(key, [0, 0.0, 0.0])
        e[0] += 1
        e[1] += ms
        e[2] += nom
    out = []
    for key, (n, ms, nom) in sorted(by.items(), key=lambda kv: -kv[1][1]):
        out.append({"pass": key, "launches": n, "ms_per_launch": ms / n,
                    "tflops": nom / (ms * 1e-3) / 1e12, "frac": nom / (ms * 1e-3) / 1e12 / peak})
    return out


def hbm_copy_rate(dev, mib=1024, reps=5):
    """Best rate of a plain device copy (torch's copy kernel) over `mib` MiB,
    read once and written once, in GB/s: the streaming rate the elementwise
    kernels are read against (the nominal 8 TB/s is not reached by any
    streaming kernel)."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    best = float("inf")
    for r in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        if r > 0:
            best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2 * n * 4 / (best * 1e-3) / 1e9


def blas_rate():
    """float64 FLOP/s of the host BLAS on a 1024^3 product (the best of
    three), used only to predict whether a shape fits the sample budget."""
    import numpy as np

    a = np.random.default_rng(1).standard_normal((1024, 1024))
    a @ a
    best = float("inf")
    for _ in range(3):
        t0 = time.perf_counter()
        a @ a
        best = min(best, time.perf_counter() - t0)
    return 2.0 * 1024**3 / best


def cpu_baseline(wl, budget_s):
    """The float64 oracle (as it stands) on one seeded unit per unit shape
    (s, l), one Muon step each, cheapest shape first; the step's oracle time
    is extrapolated as the sum over shapes of the per-unit time times the
    units with a non-zero gradient.  A shape whose predicted time (its FLOPs
    at the host BLAS rate) would take the sample past the budget is not run
    but scaled by FLOPs from the largest shape measured."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        threads = blas[0]["num_threads"] if blas else os.cpu_count()
        blas_name = blas[0].get("internal_api", "?") if blas else "?"
    except Exception:  # pragma: no cover
        threads, blas_name = os.cpu_count(), "?"
    ho = oracle.Hyper(scale=wl.scale)
    groups = sorted(shape_groups(wl).items(), key=lambda kv: unit_flops(*kv[0]))
    rng = np.random.default_rng(0)
    probe = blas_rate()
    per_unit, spent, rate, notes = {}, 0.0, None, []
    for (s, l), (n, live) in groups:
        fl = 10 * unit_flops(s, l)
        if rate is not None and spent + fl / probe > budget_s:
            per_unit[(s, l)] = fl / rate
            notes.append(f"{s}x{l}: scaled by FLOPs")
            continue
        w = rng.standard_normal((s, l)) * 0.02
        g = rng.standard_normal((s, l)) * 1e-3
        t0 = time.perf_counter()
        oracle.muon_step(w, g, np.zeros((s, l)), ho)
        dt = time.perf_counter() - t0
        spent += dt
        per_unit[(s, l)] = dt
        rate = fl / dt
        notes.append(f"{s}x{l}: {dt:.2f} s per unit")
    step_s = sum(per_unit[k] * live for k, (_, live) in groups)
    return {
        "value": wl.units / step_s,
        "unit": "matrices/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"one seeded unit per unit shape, one float64 NumPy Muon step each ({spent:.1f} s, "
                   f"{blas_name}); step time extrapolated as the sum over shapes of per-unit time x "
                   f"units ({step_s:.0f} s per step): " + "; ".join(notes)),
    }


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(
            f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
            "(the multi-GPU design shards whole matrices and is not built)",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def free():
        import gc

        from newton_schulz_matrix_muon_amd import muon

        muon._WS.clear()
        gc.collect()
        torch.cuda.empty_cache()

    wl = W.workload(args.config)
    inputs = build_inputs(wl, dev, args.grad_sets)
    head, roof = measure(wl, args.ns, args.steps, args.warmup, dev, inputs, args.schedule)
    subs = {}
    if not args.no_sub_configs and args.config == HEADLINE and args.ns == "bf16":
        free()
        r, _ = measure(wl, "fp32", FP32_SAMPLE_STEPS, 1, dev, inputs, args.schedule,
                       trace_classes=False)
        r["sample"] = f"{FP32_SAMPLE_STEPS} step after 1 warm-up step"
        subs[f"{args.config}_fp32"] = r
    del inputs
    free()
    copy_gbs = hbm_copy_rate(dev)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.zeros(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_sub_configs:
        for cfg, ns, steps, warmup, tc in SUB_CONFIGS:
            if cfg == args.config and ns == args.ns:
                continue
            w = W.workload(cfg)
            inp = build_inputs(w, dev, 2)
            r, _ = measure(w, ns, steps, warmup, dev, inp, "auto", trace_classes=tc)
            if cfg == 1:
                r["us_per_step"] = r["ms_per_step"] * 1e3
                # the same step replayed from a HIP graph (no per-call host
                # work); an extra figure, so a capture failure does not cost
                # the line
                try:
                    r["graph_us_per_step"] = graph_step_us(w, ns, dev, inp)
                except Exception as e:  # noqa: BLE001
                    r["graph_us_per_step"] = None
                    r["graph_error"] = f"{type(e).__name__}: {e}"[:200]
            subs[f"{cfg}_{ns}"] = r
            del inp
            free()

    traffic = stored_traffic(roof["kernel"], wl.title, args.ns) if roof else None
    if roof:
        roof["traffic"] = traffic["bytes_per_launch"] if traffic else None
    line = {
        "metric": "Muon matrices/sec + NS TFLOP/s (% of MI355X bf16 MFMA peak) per config",
        "value": head["matrices_per_s"],
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.ns,
        "data": "synthetic",
        "config": {
            "workload": wl.title,
            "config_index": args.config,
            "units": wl.units,
            "unit_shapes": sorted({f"{m.unit_shape[0]}x{m.unit_shape[1]}" for m in wl.matrices}),
            "grad_dtype": wl.matrices[0].grad_dtype,
            "scale": wl.scale,
            "ns_path": args.ns,
            "schedule": args.schedule,
            "parallelism": "single GPU",
        },
        **{k: head[k] for k in ("ns_tflops", "ns_frac_of_peak", "ns_ms_per_step", "ns_tflops_step",
                                "kernel_ms_per_step", "elementwise_gbs", "elementwise_frac_of_hbm",
                                "dominant_passes")
           if k in head},
        "hbm_copy_gbs": copy_gbs,
        "roofline": roof,
        "configs": subs,
    }
    if "elementwise_gbs" in head:
        line["elementwise_frac_of_copy"] = head["elementwise_gbs"] / copy_gbs
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
