"""Host-side pieces of bench.py (no GPU): the workload FLOP counts, the
executed share of the symmetric products and the stored-traffic lookup."""

import json

import bench
import workloads as W


def test_kernel_flops_match_the_workload_total():
    wl = W.workload(2)
    units = [(min(r, c), max(r, c), nz) for r, c, _, nz in bench.unit_groups(wl)]
    f = bench.kernel_flops(units)
    iters = 10
    # one NS iteration: X X^T (2 s^2 l) + A A (2 s^3) + B X (2 s^2 l)
    assert (f["gram"] + f["poly"] + f["apply"]) * iters == wl.ns_flops()


def test_executed_fraction_of_symmetric_tiles():
    assert bench.executed_fraction(1024) == 10 / 16   # 4 x 4 tiles of 256
    assert bench.executed_fraction(256) == 1.0
    assert bench.executed_fraction(128) == 1.0        # one 128 tile
    assert bench.executed_fraction(4096) == (16 * 17 / 2) / 256


def test_unit_groups_merge_heads_of_one_shape():
    wl = W.workload(3)  # Q, K and V heads are all 128 x 4096
    g = {(r, c): (n, nz) for r, c, n, nz in bench.unit_groups(wl)}
    assert g[(128, 4096)] == (48, 48)
    assert sum(n for n, _ in g.values()) == wl.units


def test_library_baseline_takes_the_group_with_the_most_work():
    # the transformer layer: 48 heads of 128 x 4096 carry far less NS work
    # than the three 4096 x 14336 MLP matrices (two of one unit shape)
    r, c, n = bench.library_group(bench.unit_groups(W.workload(3)))
    assert (min(r, c), max(r, c)) == (4096, 14336) and n == 2
    assert bench.library_group([(1024, 1024, 32, 32)]) == (1024, 1024, 32)
    assert bench.library_group([(128, 4096, 1536, 1536), (4096, 4096, 32, 32)]) == (4096, 4096, 32)


def test_ns_route_follows_the_auto_rule():
    r = bench.ns_route
    assert r(1024, 1024, 32, "bf16", "auto", 256) == "ns"            # 256 tiles: persistent
    assert r(128, 4096, 48, "bf16", "auto", 256) == "launches"       # few long heads
    assert r(128, 4096, 128, "bf16", "auto", 256) == "ns"            # many heads: on chip
    assert r(64, 128, 1, "bf16", "auto", 256) == "ns"                # short: on chip
    assert r(64, 128, 1, "fp32", "auto", 256) == "launches"          # fp32 products: tiled
    assert r(300, 128, 4, "bf16", "auto", 256) == "launches"         # tall
    assert r(128, 4096, 512, "bf16", "launches", 256) == "launches"
    assert r(64, 128, 1, "bf16", "persistent", 256) == "ns"


def test_momentum_bytes_follow_the_route():
    # 32 x 1024^2, bf16 grads: G 2 + M 8 + N 2 (written into the bf16
    # iterate of the tiled path) = 12 B per element; with fp32 products N is
    # written in fp32 (14 B)
    wl = W.workload(2)
    shapes = {(r, c): n for r, c, n, _ in bench.unit_groups(wl)}
    numel = sum(m.numel for m in wl.matrices)
    assert bench.momentum_bytes(wl.matrices, "bf16", "auto", 256, shapes) == 12 * numel
    assert bench.momentum_bytes(wl.matrices, "fp32", "auto", 256, shapes) == 14 * numel
    # the layer's 48 heads run tiled (few long heads): 12 B everywhere; with
    # many heads they run on chip, which reads N in fp32 (14 B for the heads)
    wl3 = W.workload(3)
    g3 = {(r, c): n for r, c, n, _ in bench.unit_groups(wl3)}
    n3 = sum(m.numel for m in wl3.matrices)
    assert bench.momentum_bytes(wl3.matrices, "bf16", "auto", 256, g3) == 12 * n3
    many = dict(g3)
    many[(128, 4096)] = 1536
    heads = sum(m.numel for m in wl3.matrices if m.unit_shape == (128, 4096))
    assert bench.momentum_bytes(wl3.matrices, "bf16", "auto", 256, many) == 12 * n3 + 2 * heads


def test_class_flops_split_by_route():
    groups = [(1024, 1024, 4, 4), (128, 4096, 48, 40)]
    alg, exe = bench.class_flops(groups, "bf16", "auto", 256)
    big = bench.kernel_flops([(1024, 1024, 4)])
    heads = bench.kernel_flops([(128, 4096, 40)])
    assert alg["ns"] == sum(big.values())
    for k in ("gram", "poly", "apply"):
        assert alg[k] == heads[k]
    assert exe["ns"] < alg["ns"]                     # symmetric tiles of 1024 squares
    assert exe["gram"] == alg["gram"]                # one 128 tile


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


def test_multi_gpu_request_exits_with_a_message(capsys):
    import subprocess
    import sys

    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
