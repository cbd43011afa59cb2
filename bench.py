"""Benchmark of the MI355X Muon step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--ns bf16|fp32]

A step is one Muon update (momentum, Nesterov, Frobenius normalisation, ten
hybrid Newton-Schulz iterations, scale and decoupled weight decay) of every
matrix of the workload, with inputs resident in HBM.  The default workload
is 32 stacked 1024x1024 fp32 weights with bf16 gradients N(0, 1e-3),
spectral scale, bf16 NS products (fp32 accumulation).

Prints one JSON line with matrices/s (the metric), NS TFLOP/s and its
fraction of the bf16 MFMA peak, the roofline of the dominant kernel class
(timed live with HIP events around each of its launches on the step's
stream), a float64 CPU-oracle baseline on a bounded sample, and the same NS
iterations written with torch's bf16 batched products on the workload's
largest group of equal-shape units (a vendor-library reference on this GPU).
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--ns", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--batch-update-size", type=int, default=0)
    ap.add_argument("--schedule", default="auto", choices=["auto", "persistent", "launches"],
                    help="NS schedule: the library's choice per pass, or force one persistent "
                         "launch per pass, or one launch per product")
    ap.add_argument("--grad-sets", type=int, default=4, help="distinct resident gradient batches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-library-baseline", action="store_true",
                    help="skip timing the same NS iterations written with torch's bf16 batched "
                         "products on the largest unit group")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain copy kernel over this many MiB "
                         "(int32 bitwise-not, read once and written once) for counter calibration")
    return ap.parse_args()


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


def unit_groups(wl):
    """(rows, cols, units, non-zero units) of every NS unit shape, banks of
    one unit shape merged as the library stacks them; all-zero experts are
    excluded from the second count."""
    import workloads as W

    out = {}
    for spec in wl.matrices:
        r, c = spec.unit_shape
        n = spec.batch * spec.units_per_matrix
        nz = n
        if wl.zero_fraction:
            nz -= len(W.zero_experts(wl, spec.batch)) * spec.units_per_matrix
        a, b = out.get((r, c), (0, 0))
        out[(r, c)] = (a + n, b + nz)
    return [(r, c, n, nz) for (r, c), (n, nz) in out.items()]


def ns_route(rows, cols, n_units, ns, schedule, cus):
    """Kernel class that runs the NS of a stacked pass: "ns" (one launch per
    pass: the on-chip small-unit kernel or the persistent kernel) or
    "launches" (one launch per product).  Mirrors the library's AUTO rule
    for attributing FLOPs to the traced kernel classes."""
    if schedule == "persistent":
        return "ns"
    if schedule == "launches":
        return "launches"
    if on_chip(rows, cols, n_units, ns, schedule, cus):
        return "ns"
    return "ns" if min(rows, cols) >= 256 else "launches"


def on_chip(rows, cols, n_units, ns, schedule, cus):
    """Whether the library runs a stacked pass on the on-chip small-unit
    kernel (AUTO schedule, bf16 products, wide units with at most 128 rows,
    short units or at least half as many units as CUs)."""
    return (schedule == "auto" and ns == "bf16" and rows <= cols and rows <= 128
            and (-(-cols // 128) <= 8 or 2 * n_units >= cus))


def momentum_bytes(matrix_specs, ns, schedule, cus, units_of_shape):
    """Algorithmic bytes of the momentum kernel per step: G read (2 or 4 B
    per element), M read and written (8 B), N written: into the bf16
    iterate (2 B) on the tiled bf16 path, else in fp32 (4 B)."""
    total = 0
    for m in matrix_specs:
        r, c = m.unit_shape
        small = on_chip(r, c, units_of_shape[(r, c)], ns, schedule, cus)
        n_bytes = 2 if ns == "bf16" and not small else 4
        total += m.numel * ((2 if m.grad_dtype == "bf16" else 4) + 8 + n_bytes)
    return total


def kernel_flops(units):
    """Algorithmic FLOPs of each NS kernel class per iteration, summed over
    (s, l, count) shape groups: X X^T and A*A as full products (2 s^2 l and
    2 s^3), B*X as 2 s^2 l."""
    gram = sum(n * 2.0 * s * s * l for s, l, n in units)
    poly = sum(n * 2.0 * s**3 for s, l, n in units)
    apply = sum(n * 2.0 * s * s * l for s, l, n in units)
    return {"gram": gram, "poly": poly, "apply": apply}


def executed_fraction(s):
    """Share of a symmetric s x s product's tiles that run (upper triangle
    of the tile grid; tiles are 256, or 128 when s < 256)."""
    tile = 256 if s >= 256 else 128
    t = -(-s // tile)
    return (t * (t + 1) / 2) / (t * t)


def class_flops(groups, ns, schedule, cus):
    """Per NS kernel class ("ns", "gram", "poly", "apply"): algorithmic FLOPs
    per iteration, and the FLOPs the kernels execute (symmetric products run
    their upper-triangle tiles only; the on-chip small-unit kernel runs
    whole 128 x 128 products)."""
    alg = dict.fromkeys(("ns", "gram", "poly", "apply"), 0.0)
    exe = dict(alg)
    for r, c, n, nz in groups:
        s, l = min(r, c), max(r, c)
        f = kernel_flops([(s, l, nz)])
        frac = executed_fraction(s)
        e = {"gram": f["gram"] * frac, "poly": f["poly"] * frac, "apply": f["apply"]}
        if ns_route(r, c, n, ns, schedule, cus) == "ns":
            alg["ns"] += sum(f.values())
            exe["ns"] += sum(e.values())
        else:
            for k in ("gram", "poly", "apply"):
                alg[k] += f[k]
                exe[k] += e[k]
    return alg, exe


def cpu_baseline(wl, hyper_o, seconds):
    """The float64 oracle on a bounded sample of the workload's units."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        threads = blas[0]["num_threads"] if blas else os.cpu_count()
        blas_name = blas[0].get("internal_api", "?") if blas else "?"
    except Exception:  # pragma: no cover
        threads, blas_name = os.cpu_count(), "?"
    spec = max(wl.matrices, key=lambda m: m.batch)
    r, c = spec.unit_shape
    rng = np.random.default_rng(0)
    done, t0 = 0, time.perf_counter()
    while True:
        w = rng.standard_normal((r, c)) * 0.02
        g = rng.standard_normal((r, c)) * 1e-3
        oracle.muon_step(w, g, np.zeros((r, c)), hyper_o)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {
        "value": done / el,
        "unit": "matrices/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} units of {r}x{c}, one float64 NumPy Muon step each ({el:.1f} s, {blas_name})",
    }


def library_group(groups):
    """The unit shape with the most nominal NS FLOPs, and its unit count."""
    def work(g):
        r, c, n, _ = g
        sm, lg = min(r, c), max(r, c)
        return n * (4 * sm * sm * lg + 2 * sm ** 3)
    r, c, n, _ = max(groups, key=work)
    return r, c, n


def gpu_library_baseline(groups, dev, stages, reps=3):
    """The same Newton-Schulz iterations on the workload's largest group of
    equal-shape units, written with torch's bf16 batched products (the ROCm
    GEMM libraries): per iteration A = X X^T, B = b*A + c*A*A, X = a*X + B X
    (baddbmm for the last two, X^T made contiguous first).  Units start as
    normalised N(0, 1) matrices on the smaller side.  Timed with HIP events
    on the current stream, median over `reps` runs after one warm-up."""
    import torch

    r, c, n = library_group(groups)
    sm, lg = min(r, c), max(r, c)
    gen = torch.Generator(device=dev).manual_seed(0)
    x0 = torch.randn((n, sm, lg), device=dev, generator=gen)
    x0 = (x0 / torch.linalg.vector_norm(x0, dim=(1, 2), keepdim=True)).to(torch.bfloat16)

    def run():
        x = x0.clone()
        for steps, (a, b, cc) in stages:
            for _ in range(steps):
                xt = x.transpose(1, 2).contiguous()
                am = torch.bmm(x, xt)
                bm = torch.baddbmm(am, am, am, beta=b, alpha=cc)
                x = torch.baddbmm(x, bm, x, beta=a, alpha=1.0)
        return x

    run()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    iters = sum(k for k, _ in stages)
    flops = n * iters * (4 * sm * sm * lg + 2 * sm ** 3)
    return {
        "ns_ms": ms,
        "ns_tflops": flops / (ms * 1e-3) / 1e12,
        "kind": "torch.bmm/baddbmm, bf16",
        "sample": f"{n} units of {sm}x{lg}, {iters} NS iterations, median of {reps} runs",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(
            f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
            "(the multi-GPU design shards whole matrices and is not built)",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import workloads as W
    from newton_schulz_matrix_muon_amd import muon

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.workload(args.config)
    hyper = muon.Hyper(scale=wl.scale, ns_precision=args.ns, batch_update_size=args.batch_update_size,
                       schedule=args.schedule)
    params, moms, grads, splits = build_inputs(wl, dev, args.grad_sets)
    ws_bytes = muon.workspace_size(params, hyper, splits)
    ws = muon.workspace(ws_bytes, dev)
    torch.cuda.synchronize()

    groups = unit_groups(wl)
    n_units = wl.units
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def one_step(k, trace=None):
        return muon.step(params, grads[k % len(grads)], moms, hyper=hyper, split_rows=splits,
                         ws=ws, trace=trace)

    iters = sum(s for s, _ in hyper.stages)
    n_groups = len({(m.unit_shape, m.grad_dtype) for m in wl.matrices})
    per_step = iters * n_groups * 64  # upper bound on launches of one class per step
    s0 = torch.cuda.current_stream()

    def make_events(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for e in ev:  # create the underlying HIP events
            e.record(s0)
        return ev

    def traced_ms(kind, k, ev):
        cnt = one_step(k, trace=(kind, ev))
        torch.cuda.synchronize()
        n = min(cnt, len(ev) // 2)
        return [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]

    # Warm-up (untimed), then one traced step per kernel class to find the
    # dominant NS class.
    for k in range(args.warmup):
        one_step(k)
    ev1 = make_events(per_step)
    torch.cuda.synchronize()
    kinds = {"ns": muon.KERNEL_NS, "gram": muon.KERNEL_GRAM, "poly": muon.KERNEL_POLY,
             "apply": muon.KERNEL_APPLY}
    per_kind = {}
    for name, kind in kinds.items():
        ms = traced_ms(kind, 0, ev1)
        if ms:
            per_kind[name] = sum(ms)
    mom_ms = traced_ms(muon.KERNEL_MOMENTUM, 0, ev1)
    norm_ms = traced_ms(muon.KERNEL_NORMALIZE, 0, ev1)
    dominant = max(per_kind, key=per_kind.get)

    # Timed region: exactly `steps` steps; every launch of the dominant class
    # is bracketed by HIP events on the step's stream, read back afterwards.
    launches = one_step(0, trace=(kinds[dominant], ev1[:2]))  # launches per step
    evs = [make_events(launches) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    counts = [one_step(k, trace=(kinds[dominant], evs[k])) for k in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / args.steps
    launch_ms = []
    for ev, cnt in zip(evs, counts):
        launch_ms += [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(min(cnt, len(ev) // 2))]
    # The dominant class's time per step from the timed steps (the one
    # traced step after warm-up can run at a different clock); the other
    # classes keep their traced step.
    per_kind[dominant] = sum(launch_ms) / max(1, args.steps)

    flops, exe = class_flops(groups, args.ns, args.schedule, cus)
    ns_flops_step = sum(flops.values()) * iters
    avg_launch_ms = sum(launch_ms) / max(1, len(launch_ms))
    # algorithmic FLOPs of one launch: the class's FLOPs per step (every
    # iteration, every non-zero unit) over its launches per step
    flops_per_launch = flops[dominant] * iters / launches
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12
    ns_ms = sum(per_kind.values())
    ns_tflops = ns_flops_step / (ns_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.ns]
    elem_bytes = momentum_bytes(wl.matrices, args.ns, args.schedule, cus,
                                {(r, c): n for r, c, n, _ in groups})
    if dominant != "ns":
        kernel_name = f"ns_gemm {dominant}"
    elif any(ns_route(r, c, n, args.ns, args.schedule, cus) == "ns" and min(r, c) < 256
             for r, c, n, _ in groups):
        kernel_name = "k_ns_small" if all(min(r, c) < 256 for r, c, _, _ in groups) else "ns"
    else:
        kernel_name = "ns_persistent"
    traffic = stored_traffic(kernel_name, wl.title, args.ns)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.zeros(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    line = {
        "metric": "Muon matrices/sec + NS TFLOP/s (% of MI355X bf16 MFMA peak) per config",
        "value": n_units / sec_per_step,
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.ns,
        "data": "synthetic",
        "config": {
            "workload": wl.title,
            "config_index": args.config,
            "units": n_units,
            "unit_shapes": sorted({f"{m.unit_shape[0]}x{m.unit_shape[1]}" for m in wl.matrices}),
            "grad_dtype": wl.matrices[0].grad_dtype,
            "scale": wl.scale,
            "ns_path": args.ns,
            "schedule": args.schedule,
            "parallelism": "single GPU",
        },
        "ns_tflops": ns_tflops,
        "ns_frac_of_peak": ns_tflops / peak,
        "ns_ms_per_step": ns_ms,
        "kernel_ms_per_step": {
            **{k: round(v, 4) for k, v in per_kind.items()},
            "momentum": round(sum(mom_ms), 4),
            "normalize": round(sum(norm_ms), 4),
        },
        # FLOPs the kernels execute: the symmetric products run only their
        # upper-triangle tiles
        "kernel_tflops_executed": {
            k: round(exe[k] * iters / (per_kind[k] * 1e-3) / 1e12, 2) for k in per_kind
        },
        "elementwise_gbs": elem_bytes / (sum(mom_ms) * 1e-3) / 1e9 if mom_ms else None,
        "roofline": {
            "bound": "mfma",
            "kernel": kernel_name,
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic["bytes_per_launch"] if traffic else None,
            "flops_per_launch": flops_per_launch,
            # the symmetric products run only their upper-triangle tiles:
            # the FLOPs the matrix cores execute, and their share of the peak
            "achieved_executed": exe[dominant] * iters / launches / (avg_launch_ms * 1e-3) / 1e12,
            "frac_executed": exe[dominant] * iters / launches / (avg_launch_ms * 1e-3) / 1e12 / peak,
            "avg_launch_ms": avg_launch_ms,
            "launches_timed": len(launch_ms),
        },
    }
    if not args.no_library_baseline and args.ns == "bf16":
        lib = gpu_library_baseline(groups, dev, hyper.stages)
        if len(groups) == 1:
            # one unit shape: the same units as this step's NS time
            lib["this_library_speedup"] = lib["ns_ms"] / ns_ms
        line["gpu_library_baseline"] = lib
    if not args.no_cpu_baseline:
        import oracle

        ho = oracle.Hyper(scale=wl.scale)
        line["cpu_baseline"] = cpu_baseline(wl, ho, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
