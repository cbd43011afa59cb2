"""Host-side pieces of bench.py (no GPU): the workload FLOP counts, the
FLOPs of a launch from what the library reports it covered, the executed
share of the symmetric products, the CPU-baseline extrapolation and the
stored-traffic lookup."""

import json

import pytest

import bench
import workloads as W


def test_step_flops_match_the_workload_total():
    for cfg in (1, 2, 3, 5):
        wl = W.workload(cfg)
        assert bench.ns_flops_per_step(wl, 10) == pytest.approx(wl.ns_flops(), rel=1e-12)
    # the MoE bank: 13 of 128 experts per bank have zero gradients and no NS work
    wl = W.workload(4)
    assert bench.ns_flops_per_step(wl, 10) == pytest.approx(wl.ns_flops() * 115 / 128, rel=1e-12)


def test_shape_groups_merge_tall_and_wide_units():
    g = bench.shape_groups(W.workload(3))
    assert g[(128, 4096)] == (48, 48)        # Q, K and V heads
    assert g[(4096, 14336)] == (3, 3)        # gate, up (tall) and down (wide)
    assert g[(4096, 4096)] == (1, 1)
    g4 = bench.shape_groups(W.workload(4))
    assert g4 == {(2048, 7168): (384, 345)}
    assert sum(n for n, _ in bench.shape_groups(W.workload(5)).values()) == W.workload(5).units


def test_executed_fraction_of_symmetric_tiles():
    assert bench.executed_fraction(1024, 256) == 10 / 16   # 4 x 4 tiles of 256
    assert bench.executed_fraction(256, 256) == 1.0
    assert bench.executed_fraction(128, 128) == 1.0
    assert bench.executed_fraction(4096, 256) == (16 * 17 / 2) / 256
    assert bench.executed_fraction(1024, 128) == 36 / 64


def test_launch_flops():
    groups = {(1024, 1024): (32, 32), (2048, 7168): (384, 345)}
    s, l = 1024, 1024
    nom, exe = bench.launch_flops("ns", (s, l, 32, 256), groups, 10)
    assert nom == 32 * 10 * (4 * s * s * l + 2 * s**3)
    assert exe == pytest.approx(32 * 10 * (2 * s * s * l * (10 / 16) + 2 * s**3 * (10 / 16) + 2 * s * s * l))
    # one product per launch under the per-product schedule
    assert bench.launch_flops("apply", (s, l, 32, 256), groups, 10) == (32 * 2 * s * s * l,) * 2
    g, ge = bench.launch_flops("gram", (s, l, 32, 256), groups, 10)
    assert (g, ge) == (32 * 2 * s * s * l, 32 * 2 * s * s * l * 10 / 16)
    # only units with a non-zero gradient count
    nom, _ = bench.launch_flops("ns", (2048, 7168, 384, 256), groups, 10)
    assert nom == pytest.approx(345 * 10 * (4 * 2048**2 * 7168 + 2 * 2048**3))
    # the one-launch kernel: products over the unit's 32-blocks (64 x 128
    # is exact); the streaming kernel: whole 128-row products
    nom, exe = bench.launch_flops("ns_small", (64, 128, 1, 128), {}, 10)
    assert nom == exe == 10 * (4 * 64 * 64 * 128 + 2 * 64**3)
    nom, exe = bench.launch_flops("ns_small", (100, 125, 2, 128), {}, 10)
    assert exe == 2 * 10 * (4 * 128 * 128 * 128 + 2 * 128**3)
    nom, exe = bench.launch_flops("ns_small", (128, 4096, 48, 128), {}, 10)
    assert nom == exe == 48 * 10 * (4 * 128 * 128 * 4096 + 2 * 128**3)
    nom, exe = bench.launch_flops("ns_small", (96, 1100, 3, 128), {}, 10)
    assert exe == 3 * 10 * (4 * 128 * 128 * 1152 + 2 * 128**3)


def test_pass_breakdown_groups_launches_by_pass():
    groups = {(4096, 4096): (32, 32), (4096, 14336): (96, 96)}
    ms = [80.0, 680.0, 82.0, 682.0]
    info = [(4096, 4096, 32, 256), (4096, 14336, 96, 256)] * 2
    rows = bench.pass_breakdown("ns", ms, info, groups, 10, 2516.6)
    assert [r["pass"] for r in rows] == ["96 x 4096x14336", "32 x 4096x4096"]
    assert rows[0]["launches"] == 2 and rows[0]["ms_per_launch"] == pytest.approx(681.0)
    nom = 96 * 10 * (4 * 4096**2 * 14336 + 2 * 4096**3)
    assert rows[0]["tflops"] == pytest.approx(nom / 0.681 / 1e12)


def test_two_pass_launch_counts_both_passes():
    # a persistent launch that ran the layer's MLP units and, beside them,
    # the O projection: the second pass in bits 32-63 (muon.h, muon_trace)
    groups = {(4096, 14336): (3, 3), (4096, 4096): (1, 1)}
    packed = (4096 | 4096 << 32, 14336 | 4096 << 32, 3 | 1 << 32, 256)
    mlp, mlp_e = bench.launch_flops("ns", (4096, 14336, 3, 256), groups, 10)
    o, o_e = bench.launch_flops("ns", (4096, 4096, 1, 256), groups, 10)
    assert bench.launch_flops("ns", packed, groups, 10) == (mlp + o, mlp_e + o_e)
    rows = bench.pass_breakdown("ns", [22.0, 24.0], [packed] * 2, groups, 10, 2516.6)
    assert [r["pass"] for r in rows] == ["3 x 4096x14336 + 1 x 4096x4096"]
    assert rows[0]["tflops"] == pytest.approx((mlp + o) / 0.023 / 1e12)


def test_kernel_label_names_the_two_pass_launch():
    packed = (4096 | 4096 << 32, 14336 | 4096 << 32, 3 | 1 << 32, 256)
    single = (4096, 4096, 32, 256)
    assert bench.kernel_label("ns", [single, single]) == "ns_persistent"
    assert bench.kernel_label("ns", [packed] * 3) == "ns_persistent2"
    assert bench.kernel_label("ns", [single, packed]) == "ns_persistent + ns_persistent2"
    assert bench.kernel_label("ns_small", [(128, 4096, 48, 128)]) == "k_ns_small"


def test_cpu_baseline_extrapolates_over_shapes(monkeypatch):
    import oracle

    calls = []

    def fake_step(w, g, m, h):
        calls.append(w.shape)

    monkeypatch.setattr(oracle, "muon_step", fake_step)
    t = iter([0.0, 1.0, 1.0, 3.0])  # two measured shapes: 1 s and 2 s per unit
    monkeypatch.setattr(bench.time, "perf_counter", lambda: next(t))
    # a host BLAS rate at which O (4.1e12 FLOPs) is predicted at 2 s and the
    # MLP shape at 5.3 s
    monkeypatch.setattr(bench, "blas_rate", lambda: 10 * bench.unit_flops(4096, 4096) / 2.0)
    wl = W.workload(3)
    # heads first (cheapest), then O; the MLP shape is predicted past the
    # budget and scaled by FLOPs from O's measured rate
    r = bench.cpu_baseline(wl, budget_s=5.0)
    assert calls == [(128, 4096), (4096, 4096)]
    mlp = 2.0 * bench.unit_flops(4096, 14336) / bench.unit_flops(4096, 4096)
    step = 48 * 1.0 + 1 * 2.0 + 3 * mlp
    assert r["value"] == pytest.approx(wl.units / step)
    assert "scaled by FLOPs" in r["sample"] and r["kind"] == "oracle"


def test_stored_traffic_lookup(tmp_path):
    rec = {"kernel": "ns_persistent", "workload": "w", "ns": "bf16", "sources_sha256": "abc",
           "bytes_per_launch": 123}
    (tmp_path / "x_traffic.md").write_text("# t\n\ntraffic_record: " + json.dumps(rec) + "\n")
    got = bench.stored_traffic("ns_persistent", "w", "bf16", pdir=str(tmp_path), digest="abc")
    assert got["bytes_per_launch"] == 123
    # other kernel, other workload, or changed sources: no figure
    assert bench.stored_traffic("ns_gemm apply", "w", "bf16", pdir=str(tmp_path), digest="abc") is None
    assert bench.stored_traffic("ns_persistent", "v", "bf16", pdir=str(tmp_path), digest="abc") is None
    assert bench.stored_traffic("ns_persistent", "w", "bf16", pdir=str(tmp_path), digest="def") is None


def test_committed_traffic_records_are_well_formed():
    import os

    pdir = os.path.join(bench.ROOT, "profiles")
    for name in os.listdir(pdir):
        for line in open(os.path.join(pdir, name), encoding="utf-8"):
            if line.startswith("traffic_record: "):
                rec = json.loads(line[len("traffic_record: "):])
                assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
                assert len(rec["sources_sha256"]) == 64


def test_multi_gpu_request_exits_with_a_message():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
