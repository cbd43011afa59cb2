"""The C ABI without a GPU: the library loads, exports every symbol that
include/muon.h declares, fills the pages' defaults, sizes workspaces, and
rejects invalid arguments before touching any memory (no launch happens on
an error path, so fake device addresses are safe here)."""

import ctypes
import os
import re

import pytest

from newton_schulz_matrix_muon_amd import muon

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "muon.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(muon.EXPORTED)
    for n in names:
        assert hasattr(muon.LIB, n), n


def test_defaults_are_the_pages_values():
    h = muon.default_hyper_c()
    assert h.lr == pytest.approx(2.7e-4) and h.mu == pytest.approx(0.95)
    assert h.weight_decay == pytest.approx(0.1) and h.gamma == pytest.approx(0.18)
    assert h.scale_mode == muon.SCALE_SPECTRAL and h.ns_precision == muon.NS_BF16
    assert h.n_stages == 2
    assert (h.stages[0].steps, h.stages[1].steps) == (8, 2)
    assert (h.stages[0].a, h.stages[0].b, h.stages[0].c) == pytest.approx((3.4445, -4.7750, 2.0315))
    assert (h.stages[1].a, h.stages[1].b, h.stages[1].c) == (2.0, -1.5, 0.5)
    assert h.schedule == muon.SCHEDULE_AUTO and h.reserved == 0
    assert h.nesterov_style == muon.NESTEROV_SGD and h.step == 1


def _desc(shapes):
    arr = (muon.MatrixDesc * max(1, len(shapes)))()
    for i, s in enumerate(shapes):
        b, r, c, sp = s
        arr[i].batch, arr[i].rows, arr[i].cols, arr[i].split_rows = b, r, c, sp
        arr[i].grad_dtype = muon.DTYPE_BF16
    return arr


def ws_size(shapes, h=None):
    h = h or muon.default_hyper_c()
    out = ctypes.c_size_t(0)
    st = muon.LIB.muon_workspace_size(_desc(shapes), len(shapes), ctypes.byref(h), ctypes.byref(out))
    return st, out.value


def test_workspace_sizes():
    mib = 1024 * 1024
    st, n = ws_size([(32, 1024, 1024, 0)])
    assert st == 0
    # bf16 path, tiled products: two bf16 iterates (momentum writes N into
    # the first; no transposed copies: the products read X K-major), bf16
    # Gram, bf16 polynomial = 8 bytes per element, plus the status header,
    # per-unit norms and schedule counters
    assert 32 * mib * 8 <= n < 32 * mib * 8 + mib
    h = muon.default_hyper_c()
    h.batch_update_size = 8
    st, n8 = ws_size([(32, 1024, 1024, 0)], h)
    assert st == 0 and 8 * mib * 8 <= n8 < 8 * mib * 8 + mib
    h.ns_precision = muon.NS_FP32
    st, nf = ws_size([(32, 1024, 1024, 0)], h)
    # fp32 path: two fp32 iterates and their two transposes, fp32 Gram and
    # polynomial = 24 bytes
    assert st == 0 and 8 * mib * 24 <= nf < 8 * mib * 24 + mib
    assert ws_size([])[0] == 0


def test_bf16_workspace_holds_only_bf16_iterates():
    # The bf16 paths (tiled and on chip) fold 1/||N|| into the first
    # iteration, so no fp32 copy of N exists: two bf16 iterates (2 x 2 bytes
    # per element of the 128 x 4096 iterate) plus two 128 x 128 bf16
    # matrices per unit, under any schedule.  Under AUTO, 48 such units (too
    # few to fill 256 CUs) may be split over min(32 blocks, 8, 256 / 48) = 5
    # workgroups each, with two buffers of fp32 128 x 128 partial Grams per
    # workgroup.
    per_unit = 128 * 4096 * 4 + 2 * 128 * 128 * 2
    split = 2 * 5 * 128 * 128 * 4
    st, n = ws_size([(48, 128, 4096, 0)])
    assert st == 0 and 48 * (per_unit + split) <= n < 48 * (per_unit + split) + (1 << 20)
    # 128 such units fill the CUs one workgroup each: no partials
    st, n128 = ws_size([(128, 128, 4096, 0)])
    assert st == 0 and 128 * per_unit <= n128 < 128 * per_unit + (1 << 20)
    h = muon.default_hyper_c()
    h.schedule = muon.SCHEDULE_PERSISTENT
    st, nt = ws_size([(48, 128, 4096, 0)], h)
    assert st == 0 and 48 * per_unit <= nt < 48 * per_unit + (1 << 20)
    # the fp32 path keeps X and X^T in fp32, twice
    h = muon.default_hyper_c()
    h.ns_precision = muon.NS_FP32
    st, nf = ws_size([(48, 128, 4096, 0)], h)
    assert st == 0 and nf >= 48 * 128 * 4096 * 16


def test_workspace_holds_a_riding_pass():
    # AUTO: a single 256-tile unit (4096 x 4096) may run inside the
    # persistent launch of a stacked pass with the same orientation (three
    # tall 14336 x 4096 units), so the workspace holds both passes' buffers
    # one after the other; forced schedules run the passes one by one and
    # reuse one carve-up.
    mib = 1024 * 1024
    per_mlp = 14336 * 4096 * 4 + 2 * 4096 * 4096 * 2   # two bf16 iterates, bf16 A and B'
    per_o = 4096 * 4096 * 8
    shapes = [(1, 4096, 4096, 0), (2, 14336, 4096, 0), (1, 4096, 14336, 0)]
    st, n = ws_size(shapes)
    assert st == 0 and 3 * per_mlp + per_o <= n < 3 * per_mlp + per_o + mib
    for sched in (muon.SCHEDULE_PERSISTENT, muon.SCHEDULE_LAUNCHES):
        h = muon.default_hyper_c()
        h.schedule = sched
        st, nf = ws_size(shapes, h)
        assert st == 0 and 3 * per_mlp <= nf < 3 * per_mlp + mib
    # tiled passes take the tall form (wide units transposed), so wide
    # units pair as well
    st, n = ws_size([(1, 4096, 4096, 0), (3, 4096, 14336, 0)])
    assert st == 0 and 3 * per_mlp + per_o <= n < 3 * per_mlp + per_o + mib
    # one riding pass per stacked pass: the first in pass order (units in
    # their own form before transposed ones), here the 4096 x 4096 unit
    st, n = ws_size([(1, 2048, 4096, 0), (3, 4096, 14336, 0), (1, 4096, 4096, 0)])
    assert st == 0 and 3 * per_mlp + per_o <= n < 3 * per_mlp + per_o + mib
    # fp32 products read rows of X and X^T on every pass: any stacked pass
    h = muon.default_hyper_c()
    h.ns_precision = muon.NS_FP32
    st, n = ws_size([(1, 512, 512, 0), (2, 1024, 512, 0)], h)
    per_a = 1024 * 512 * 16 + 2 * 512 * 512 * 4
    per_b = 512 * 512 * 16 + 2 * 512 * 512 * 4
    assert st == 0 and 2 * per_a + per_b <= n < 2 * per_a + per_b + mib


def test_pairing_many_passes_is_fast():
    # 20000 shapes of three 256-tile units, cut two per pass: 20000 stacked
    # passes and 20000 single-unit passes to pair (one rider each)
    import time

    shapes = [(3, 256 + i, 256, 0) for i in range(20000)]
    h = muon.default_hyper_c()
    h.batch_update_size = 2
    t0 = time.perf_counter()
    st, n = ws_size(shapes, h)
    assert st == 0 and n > 0
    assert time.perf_counter() - t0 < 2.0


@pytest.mark.parametrize(
    "shape,code",
    [
        ((1, 0, 5, 0), -2),
        ((1, 5, 0, 0), -2),
        ((0, 5, 5, 0), -2),
        ((1, 10, 5, 3), -2),   # split does not divide rows
        ((1, 10, 5, -1), -2),
    ],
)
def test_bad_shapes_rejected(shape, code):
    assert ws_size([shape])[0] == code


def test_unit_size_limit():
    # A unit's bf16 iterate, padded to the tile (256), must stay under 2^31
    # bytes (its K-major copies address it with 32-bit offsets):
    # 32768 x 32512 pads to itself and fits; one more column pads to
    # 32768 x 32768 = 2^31 bytes and is rejected.
    assert ws_size([(1, 32768, 32512, 0)])[0] == 0
    assert ws_size([(1, 32768, 32513, 0)])[0] == -2
    # the limit is per unit: a batch of large units is fine
    assert ws_size([(2, 16384, 16384, 0)])[0] == 0


def test_pass_count_limit():
    # At most 2^20 stacked passes per call, refused before any is planned
    # (2^30 one-unit passes would otherwise be built on the host).
    h = muon.default_hyper_c()
    h.batch_update_size = 1
    assert ws_size([(1 << 20, 4, 4, 0)], h)[0] == 0
    assert ws_size([(1 << 20, 4, 4, 0), (1, 4, 4, 0)], h)[0] == -2
    assert ws_size([(1 << 30, 4, 4, 1)], h)[0] == -2
    h.batch_update_size = 0
    assert ws_size([(1 << 30, 4, 4, 1)], h)[0] == 0


def test_bad_hyper_rejected():
    h = muon.default_hyper_c()
    h.n_stages = 0
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6
    h = muon.default_hyper_c()
    h.lr = float("nan")
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6
    h = muon.default_hyper_c()
    h.scale_mode = 7
    assert ws_size([(1, 4, 4, 0)], h)[0] == -3
    h = muon.default_hyper_c()
    h.stages[0].steps = 0
    h.stages[1].steps = 0
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6
    h = muon.default_hyper_c()
    h.schedule = 3
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6
    h = muon.default_hyper_c()
    h.reserved = 1
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6
    h = muon.default_hyper_c()
    h.schedule = muon.SCHEDULE_LAUNCHES
    assert ws_size([(1, 4, 4, 0)], h)[0] == 0
    h = muon.default_hyper_c()
    h.nesterov_style = 2
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6
    h = muon.default_hyper_c()
    h.nesterov_style = muon.NESTEROV_EMA
    assert ws_size([(1, 4, 4, 0)], h)[0] == 0
    h.step = 0                       # the bias corrections need t >= 1
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6
    h.step = 3
    h.mu = 1.0                       # 1 - mu^t would be 0
    assert ws_size([(1, 4, 4, 0)], h)[0] == -6


def _step(ptrs_w, ptrs_g, ptrs_m, shapes, ws=0x10000000, ws_bytes=1 << 40, h=None):
    n = len(shapes)
    P = ctypes.c_void_p * max(1, n)
    h = h or muon.default_hyper_c()
    return muon.LIB.muon_step_batched(
        P(*ptrs_w), P(*ptrs_g), P(*ptrs_m), _desc(shapes), n, ctypes.byref(h),
        ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None,
    )


BASE = 0x7F0000000000


def test_step_error_paths_touch_nothing():
    s = [(1, 64, 128, 0)]
    sz = 64 * 128 * 4
    ok = ([BASE], [BASE + 2 * sz], [BASE + 4 * sz])
    assert _step([0], ok[1], ok[2], s) == -1                      # NULL param
    assert _step(ok[0], ok[1], ok[2], s, ws=0, ws_bytes=0) == -5   # no workspace
    assert _step(ok[0], ok[1], ok[2], s, ws_bytes=16) == -5        # too small
    assert _step([BASE + 4], ok[1], ok[2], s) == -4                # misaligned
    assert _step(ok[0], ok[1], ok[2], s, ws=0x10000010) == -4      # workspace alignment
    assert _step(ok[0], ok[1], [BASE + 112], s) == -8              # params overlap momenta
    assert _step(ok[0], [BASE + 64], ok[2], s) == -8               # grads overlap params
    assert _step(ok[0], ok[1], ok[2], [(1, 64, 128, 5)]) == -2     # bad split
    h = muon.default_hyper_c()
    h.ns_precision = 3
    assert _step(ok[0], ok[1], ok[2], s, h=h) == -3
    assert _step([], [], [], []) == 0                              # no-op


def test_planner_fuzz():
    # Random bank lists and hyper-parameters through the host planner
    # (validation, grouping, chunking, workspace carve-up): every call
    # returns a defined status; accepted ones give a 256-byte-aligned size
    # of at least the status header; adding a bank never shrinks the
    # workspace and a batch_update_size cap never grows it.  Under the
    # sanitizer build (tests/test_sanitizers.py) this also checks the
    # planner's arithmetic for overflow and its memory accesses.
    import numpy as np

    rng = np.random.default_rng(2024)
    valid = {0, -2, -3, -6}
    for _ in range(400):
        n = int(rng.integers(0, 6))
        shapes = []
        for _ in range(n):
            rows = int(rng.choice([1, 2, 63, 64, 127, 128, 129, 255, 256, 1000, 4096, 14336, 1 << 20]))
            cols = int(rng.choice([1, 3, 64, 128, 300, 1024, 4096, 7168, 1 << 16]))
            split = int(rng.choice([0, 0, 0, 1, 7, 128, rows]))
            batch = int(rng.choice([1, 2, 13, 128, 1 << 20]))
            shapes.append((batch, rows, cols, split))
        h = muon.default_hyper_c()
        h.ns_precision = int(rng.integers(0, 2))
        h.schedule = int(rng.integers(0, 3))
        h.batch_update_size = int(rng.choice([0, 1, 3, 16]))
        h.stages[0].steps = int(rng.choice([0, 1, 8, 1000]))
        st, size = ws_size(shapes, h)
        assert st in valid, (shapes, st)
        if st != 0:
            continue
        assert size >= 256 and size % 256 == 0
        if n > 0:
            st2, size2 = ws_size(shapes[:-1], h)
            assert st2 == 0 and size2 <= size
        if h.batch_update_size == 0:
            h.batch_update_size = 2
            st3, size3 = ws_size(shapes, h)
            # more passes: refused only for exceeding the 2^20 pass limit
            assert (st3 == 0 and size3 <= size) or st3 == -2


def test_noalloc_error_paths_touch_nothing():
    # the scratch entry point validates like muon_step_batched and refuses a
    # step that needs more than its 128 MiB before looking up the scratch
    f = muon.LIB.muon_step_batched_noalloc
    P = ctypes.c_void_p * 1

    def call(w, g, m, shapes, h=None):
        h = h or muon.default_hyper_c()
        return f(P(w), P(g), P(m), _desc(shapes), len(shapes), ctypes.byref(h), None)

    s = [(1, 64, 128, 0)]
    sz = 64 * 128 * 4
    assert call(0, BASE + 2 * sz, BASE + 4 * sz, s) == -1
    assert call(BASE + 4, BASE + 2 * sz, BASE + 4 * sz, s) == -4
    assert call(BASE, BASE + 2 * sz, BASE + 4 * sz, [(1, 64, 128, 5)]) == -2
    big = [(40, 1024, 1024, 0)]  # 320 MiB of workspace
    n = 40 * 1024 * 1024 * 4
    assert call(BASE, BASE + 2 * n, BASE + 4 * n, big) == -5
    assert f(P(), P(), P(), _desc([]), 0, ctypes.byref(muon.default_hyper_c()), None) == 0


def test_workspace_status_argument_errors():
    st = muon.LIB.muon_workspace_status
    assert st(None, 1 << 20, None) == -1
    assert st(ctypes.c_void_p(0x10000000), 128, None) == -5
    assert st(ctypes.c_void_p(0x10000010), 1 << 20, None) == -4


def test_status_strings():
    for code in range(-9, 1):
        assert muon.status_string(code) != "unknown status"
    assert muon.status_string(12345) == "unknown status"
    assert muon.LIB.muon_abi_version() == 6
