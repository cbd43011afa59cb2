"""Python binding of the Muon C ABI (include/muon.h) via ctypes.

Argument marshalling only: tensors are turned into device pointers and bank
descriptors, the stream is torch's current stream, and the workspace is a
cached torch byte tensor.  Every step of the computation runs in the HIP
library; if it is missing this module raises on import.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MUON_LIBRARY selects another build of the same library (the sanitizer
# build of the CPU tests); by default the in-tree libmuon.so.
LIB_PATH = os.environ.get("MUON_LIBRARY") or os.path.join(_HERE, "libmuon.so")

MUON_OK = 0
STATUS_NAMES = {
    0: "MUON_OK",
    -1: "MUON_ERR_NULL",
    -2: "MUON_ERR_SHAPE",
    -3: "MUON_ERR_DTYPE",
    -4: "MUON_ERR_ALIGN",
    -5: "MUON_ERR_WORKSPACE",
    -6: "MUON_ERR_HYPER",
    -7: "MUON_ERR_HIP",
    -8: "MUON_ERR_ALIAS",
    -9: "MUON_ERR_SCHEDULE",
}
DTYPE_F32, DTYPE_BF16 = 0, 1
SCALE_SPECTRAL, SCALE_UNIT_RMS_NORM = 0, 1
NS_FP32, NS_BF16 = 0, 1
KERNEL_MOMENTUM, KERNEL_NORMALIZE, KERNEL_GRAM, KERNEL_POLY, KERNEL_APPLY = 1, 2, 3, 4, 5
KERNEL_NS, KERNEL_NS_SMALL = 6, 7
SCHEDULE_AUTO, SCHEDULE_PERSISTENT, SCHEDULE_LAUNCHES = 0, 1, 2
NESTEROV_SGD, NESTEROV_EMA = 0, 1
MAX_STAGES = 4

EXPORTED = (
    "muon_hyper_default",
    "muon_workspace_size",
    "muon_step_batched",
    "muon_newton_schulz_batched",
    "muon_step_batched_traced",
    "muon_newton_schulz_batched_traced",
    "muon_step_batched_noalloc",
    "muon_workspace_status",
    "muon_status_string",
    "muon_abi_version",
)


class MatrixDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("split_rows", ctypes.c_int64),
        ("grad_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class NsStage(ctypes.Structure):
    _fields_ = [
        ("steps", ctypes.c_int32),
        ("a", ctypes.c_float),
        ("b", ctypes.c_float),
        ("c", ctypes.c_float),
    ]


class HyperC(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("mu", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("gamma", ctypes.c_float),
        ("scale_mode", ctypes.c_int32),
        ("ns_precision", ctypes.c_int32),
        ("batch_update_size", ctypes.c_int32),
        ("n_stages", ctypes.c_int32),
        ("stages", NsStage * MAX_STAGES),
        ("schedule", ctypes.c_int32),
        ("nesterov_style", ctypes.c_int32),
        ("step", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class TraceC(ctypes.Structure):
    _fields_ = [
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("info", ctypes.POINTER(ctypes.c_int64)),
        ("capacity", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("count", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m newton_schulz_matrix_muon_amd.build` (hipcc, gfx950)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.muon_hyper_default.argtypes = [ctypes.POINTER(HyperC)]
    lib.muon_hyper_default.restype = None
    lib.muon_workspace_size.argtypes = [
        ctypes.POINTER(MatrixDesc), ctypes.c_int64, ctypes.POINTER(HyperC),
        ctypes.POINTER(ctypes.c_size_t),
    ]
    lib.muon_workspace_size.restype = ctypes.c_int
    step_args = [
        ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(MatrixDesc),
        ctypes.c_int64, ctypes.POINTER(HyperC), P, ctypes.c_size_t, P,
    ]
    ns_args = [
        ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(MatrixDesc), ctypes.c_int64,
        ctypes.POINTER(HyperC), P, ctypes.c_size_t, P,
    ]
    lib.muon_step_batched.argtypes = step_args
    lib.muon_step_batched.restype = ctypes.c_int
    lib.muon_step_batched_traced.argtypes = step_args + [ctypes.POINTER(TraceC)]
    lib.muon_step_batched_traced.restype = ctypes.c_int
    lib.muon_newton_schulz_batched.argtypes = ns_args
    lib.muon_newton_schulz_batched.restype = ctypes.c_int
    lib.muon_newton_schulz_batched_traced.argtypes = ns_args + [ctypes.POINTER(TraceC)]
    lib.muon_newton_schulz_batched_traced.restype = ctypes.c_int
    lib.muon_step_batched_noalloc.argtypes = step_args[:6] + [P]
    lib.muon_step_batched_noalloc.restype = ctypes.c_int
    lib.muon_workspace_status.argtypes = [P, ctypes.c_size_t, P]  # workspace, bytes, stream
    lib.muon_workspace_status.restype = ctypes.c_int
    lib.muon_status_string.argtypes = [ctypes.c_int]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_abi_version.argtypes = []
    lib.muon_abi_version.restype = ctypes.c_int
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.muon_status_string(status).decode()


@dataclass
class Hyper:
    """Mirror of `muon_hyper`; defaults come from the library
    (lr 2.7e-4, mu 0.95, wd 0.1, gamma 0.18, spectral, bf16 NS products,
    8 x (3.4445, -4.7750, 2.0315) + 2 x (2, -1.5, 0.5), AUTO NS
    schedule)."""

    lr: float = 2.7e-4
    mu: float = 0.95
    weight_decay: float = 0.1
    gamma: float = 0.18
    scale: str = "spectral"  # or "unit_rms_norm"
    ns_precision: str = "bf16"  # or "fp32"
    batch_update_size: int = 0
    stages: Sequence[tuple[int, tuple[float, float, float]]] = field(
        default_factory=lambda: ((8, (3.4445, -4.7750, 2.0315)), (2, (2.0, -1.5, 0.5)))
    )
    schedule: str = "auto"  # or "persistent" / "launches" (tiled products only)
    nesterov_style: str = "sgd"  # or "ema" (bias-corrected; needs `step`)
    step: int = 1  # 1-based index of this step (EMA style only)

    def to_c(self) -> HyperC:
        h = HyperC()
        h.lr, h.mu, h.weight_decay, h.gamma = self.lr, self.mu, self.weight_decay, self.gamma
        h.scale_mode = {"spectral": SCALE_SPECTRAL, "unit_rms_norm": SCALE_UNIT_RMS_NORM}[self.scale]
        h.ns_precision = {"fp32": NS_FP32, "bf16": NS_BF16}[self.ns_precision]
        h.batch_update_size = self.batch_update_size
        h.schedule = {"auto": SCHEDULE_AUTO, "persistent": SCHEDULE_PERSISTENT,
                      "launches": SCHEDULE_LAUNCHES}[self.schedule]
        h.nesterov_style = {"sgd": NESTEROV_SGD, "ema": NESTEROV_EMA}[self.nesterov_style]
        h.step = self.step
        h.reserved = 0
        if not 1 <= len(self.stages) <= MAX_STAGES:
            raise ValueError("between 1 and 4 NS stages")
        h.n_stages = len(self.stages)
        for i, (steps, (a, b, c)) in enumerate(self.stages):
            h.stages[i].steps, h.stages[i].a, h.stages[i].b, h.stages[i].c = steps, a, b, c
        return h


def default_hyper_c() -> HyperC:
    h = HyperC()
    LIB.muon_hyper_default(ctypes.byref(h))
    return h


def _as3d(t: torch.Tensor) -> tuple[int, int, int]:
    if t.dim() == 2:
        return 1, t.shape[0], t.shape[1]
    if t.dim() == 3:
        return t.shape[0], t.shape[1], t.shape[2]
    raise ValueError("expected a (rows, cols) or (batch, rows, cols) tensor")


def _descs(tensors, split_rows, grad_dtypes) -> ctypes.Array:
    arr = (MatrixDesc * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        b, r, c = _as3d(t)
        arr[i].batch, arr[i].rows, arr[i].cols = b, r, c
        arr[i].split_rows = int(split_rows[i] or 0)
        arr[i].grad_dtype = grad_dtypes[i]
        arr[i].reserved = 0
    return arr


def _ptrs(tensors) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


# Cached workspaces, one per (device, stream): calls on one stream run in
# order and may share a workspace; calls on different streams may overlap
# and must not.
_WS: dict[tuple[int, int], torch.Tensor] = {}

# Whether step() and newton_schulz() check the schedule status after each
# call when their `check` argument is None (the check waits for the stream).
check_default = False


def workspace(nbytes: int, device: torch.device, stream=None) -> torch.Tensor:
    """A cached byte workspace of at least `nbytes` on `device` for calls on
    `stream` (torch's current stream when None)."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    dev = device.index if device.index is not None else torch.cuda.current_device()
    key = (dev, s.cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        # The old buffer may still be in use by work queued on `s`; it was
        # recorded on `s` when handed out, so the allocator keeps it until
        # that work is done.
        _WS.pop(key, None)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = ws
    if s != torch.cuda.current_stream(device):
        ws.record_stream(s)
    return ws


def workspace_status(ws: torch.Tensor, stream=None) -> None:
    """Waits for the stream and raises MuonError(MUON_ERR_SCHEDULE) if any
    call on `ws` since the previous check had an NS launch (persistent, or
    small units split on chip) stop early (muon_workspace_status; the report
    is sticky until read)."""
    st = LIB.muon_workspace_status(ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
                                   ctypes.c_void_p(_stream_ptr(stream)))
    if st != MUON_OK:
        raise MuonError(st, "muon_workspace_status")


def workspace_size(tensors, hyper: Hyper | HyperC, split_rows=None) -> int:
    split_rows = split_rows or [0] * len(tensors)
    d = _descs(tensors, split_rows, [DTYPE_F32] * len(tensors))
    hc = hyper.to_c() if isinstance(hyper, Hyper) else hyper
    out = ctypes.c_size_t(0)
    st = LIB.muon_workspace_size(d, len(tensors), ctypes.byref(hc), ctypes.byref(out))
    if st != MUON_OK:
        raise MuonError(st, "muon_workspace_size")
    return out.value


def _check(ts, dtype, name, device):
    for t in ts:
        if t.device != device:
            raise ValueError(f"{name}: all tensors must be on {device}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous")


def _stream_ptr(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Trace:
    """Brackets every launch of one kernel class (muon_trace): `capacity`
    pairs of timing events, recorded on the call's stream, and what each
    launch covered (`info`, four values per launch as muon.h describes)."""

    def __init__(self, kind: int, capacity: int, stream=None):
        self.kind = kind
        self.capacity = capacity
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * capacity)]
        s = stream if stream is not None else torch.cuda.current_stream()
        for e in self.events:  # create the underlying HIP events
            e.record(s)
        self._ev = (ctypes.c_void_p * max(1, 2 * capacity))()
        for i, e in enumerate(self.events):
            self._ev[i] = e.cuda_event
        self._info = (ctypes.c_int64 * max(1, 4 * capacity))()
        self.count = 0

    def c(self) -> TraceC:
        tr = TraceC()
        tr.events = ctypes.cast(self._ev, ctypes.POINTER(ctypes.c_void_p))
        tr.info = ctypes.cast(self._info, ctypes.POINTER(ctypes.c_int64))
        tr.capacity = self.capacity
        tr.kind = self.kind
        tr.count = 0
        tr.reserved = 0
        return tr

    @property
    def recorded(self) -> int:
        return min(self.count, self.capacity)

    def ms(self) -> list[float]:
        """Duration of each recorded launch (the stream must have passed them)."""
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(self.recorded)]

    def info(self) -> list[tuple[int, int, int, int]]:
        return [tuple(self._info[4 * i: 4 * i + 4]) for i in range(self.recorded)]

    def passes(self) -> list[list[tuple[int, int, int, int]]]:
        """For NS classes: the passes each recorded launch ran, as
        (smaller side, larger side, units, tile) tuples (see ns_passes)."""
        return [ns_passes(i) for i in self.info()]


def ns_passes(info) -> list[tuple[int, int, int, int]]:
    """The passes one NS launch ran, from its four trace values: its own
    pass, and a single-unit pass it ran beside it, whose values sit in bits
    32-63 of the first three (muon.h, muon_trace)."""
    s, l, units, tile = (int(v) for v in info)
    lo = (1 << 32) - 1
    out = [(s & lo, l & lo, units & lo, tile)]
    if units >> 32:
        out.append((s >> 32, l >> 32, units >> 32, tile))
    return out


def _run_traced(fn, args, trace: Trace | None):
    if trace is None:
        return fn(*args)
    tr = trace.c()
    st = fn(*args, ctypes.byref(tr))
    trace.count = tr.count
    return st


def step(
    params: Sequence[torch.Tensor],
    grads: Sequence[torch.Tensor],
    momenta: Sequence[torch.Tensor],
    hyper: Hyper | None = None,
    split_rows: Sequence[int] | None = None,
    stream=None,
    ws: torch.Tensor | None = None,
    trace: Trace | None = None,
    check: bool | None = None,
) -> int:
    """One Muon step, in place on `params` and `momenta` (muon_step_batched).

    params/momenta: fp32 (rows, cols) or (batch, rows, cols) banks;
    grads: bf16 or fp32 of the same shapes; split_rows: per bank, 0 or the
    head size.  `trace` (a Trace) brackets every launch of one kernel
    class.  `check` (default: `check_default`) waits for the stream
    afterwards and raises MuonError if an NS launch whose workgroups wait on
    each other stopped, in which case params and momenta are undefined.
    Returns the number of launches of the traced class (0 without a
    trace).

    Under HIP graph capture (torch.cuda.graph), pass a workspace `ws` and
    check=False, and make one eager call on the device first: the call then
    only enqueues kernels, and the captured step replays like a fresh one
    (tests/test_gpu_graph.py)."""
    hyper = hyper or Hyper()
    n = len(params)
    if not (len(grads) == len(momenta) == n):
        raise ValueError("params, grads and momenta must have the same length")
    if n == 0:
        return 0
    dev = params[0].device
    _check(params, torch.float32, "params", dev)
    _check(momenta, torch.float32, "momenta", dev)
    _check(grads, None, "grads", dev)
    gd = []
    for p, g, m in zip(params, grads, momenta):
        if p.shape != g.shape or p.shape != m.shape:
            raise ValueError("params, grads and momenta shapes differ")
        if g.dtype == torch.bfloat16:
            gd.append(DTYPE_BF16)
        elif g.dtype == torch.float32:
            gd.append(DTYPE_F32)
        else:
            raise TypeError(f"grads must be bf16 or fp32, got {g.dtype}")
    split_rows = list(split_rows) if split_rows is not None else [0] * n
    descs = _descs(params, split_rows, gd)
    hc = hyper.to_c()
    need = ctypes.c_size_t(0)
    st = LIB.muon_workspace_size(descs, n, ctypes.byref(hc), ctypes.byref(need))
    if st != MUON_OK:
        raise MuonError(st, "muon_workspace_size")
    if ws is None:
        ws = workspace(need.value, dev, stream)
    args = (
        _ptrs(params), _ptrs(grads), _ptrs(momenta), descs, n, ctypes.byref(hc),
        ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
        ctypes.c_void_p(_stream_ptr(stream)),
    )
    st = _run_traced(LIB.muon_step_batched_traced if trace else LIB.muon_step_batched, args, trace)
    count = trace.count if trace else 0
    if st != MUON_OK:
        raise MuonError(st, "muon_step_batched")
    if check_default if check is None else check:
        workspace_status(ws, stream)
    return count


def step_noalloc(
    params: Sequence[torch.Tensor],
    grads: Sequence[torch.Tensor],
    momenta: Sequence[torch.Tensor],
    hyper: Hyper | None = None,
    split_rows: Sequence[int] | None = None,
    stream=None,
) -> None:
    """One Muon step on the library's fixed device scratch
    (muon_step_batched_noalloc): no workspace, nothing allocated; the step
    may need at most 128 MiB of scratch.  Calls that overlap on one GPU
    race."""
    hyper = hyper or Hyper()
    n = len(params)
    if not (len(grads) == len(momenta) == n):
        raise ValueError("params, grads and momenta must have the same length")
    if n == 0:
        return
    dev = params[0].device
    _check(params, torch.float32, "params", dev)
    _check(momenta, torch.float32, "momenta", dev)
    _check(grads, None, "grads", dev)
    gd = []
    for p, g, m in zip(params, grads, momenta):
        if p.shape != g.shape or p.shape != m.shape:
            raise ValueError("params, grads and momenta shapes differ")
        if g.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError(f"grads must be bf16 or fp32, got {g.dtype}")
        gd.append(DTYPE_BF16 if g.dtype == torch.bfloat16 else DTYPE_F32)
    split_rows = list(split_rows) if split_rows is not None else [0] * n
    descs = _descs(params, split_rows, gd)
    hc = hyper.to_c()
    st = LIB.muon_step_batched_noalloc(
        _ptrs(params), _ptrs(grads), _ptrs(momenta), descs, n, ctypes.byref(hc),
        ctypes.c_void_p(_stream_ptr(stream)),
    )
    if st != MUON_OK:
        raise MuonError(st, "muon_step_batched_noalloc")


def newton_schulz(
    xs: Sequence[torch.Tensor],
    outs: Sequence[torch.Tensor] | None = None,
    hyper: Hyper | None = None,
    split_rows: Sequence[int] | None = None,
    stream=None,
    ws: torch.Tensor | None = None,
    trace: Trace | None = None,
    check: bool | None = None,
):
    """Hybrid Newton-Schulz only (muon_newton_schulz_batched): the unscaled
    NS output of every unit of every fp32 bank in `xs`, written to `outs`
    (new tensors when None).  `check` as for step().  Returns (outs, traced
    launch count)."""
    hyper = hyper or Hyper()
    n = len(xs)
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    if n == 0:
        return outs, 0
    dev = xs[0].device
    _check(xs, torch.float32, "xs", dev)
    _check(outs, torch.float32, "outs", dev)
    split_rows = list(split_rows) if split_rows is not None else [0] * n
    descs = _descs(xs, split_rows, [DTYPE_F32] * n)
    hc = hyper.to_c()
    need = ctypes.c_size_t(0)
    st = LIB.muon_workspace_size(descs, n, ctypes.byref(hc), ctypes.byref(need))
    if st != MUON_OK:
        raise MuonError(st, "muon_workspace_size")
    if ws is None:
        ws = workspace(need.value, dev, stream)
    args = (
        _ptrs(xs), _ptrs(outs), descs, n, ctypes.byref(hc), ctypes.c_void_p(ws.data_ptr()),
        ctypes.c_size_t(ws.numel()), ctypes.c_void_p(_stream_ptr(stream)),
    )
    st = _run_traced(
        LIB.muon_newton_schulz_batched_traced if trace else LIB.muon_newton_schulz_batched, args, trace
    )
    count = trace.count if trace else 0
    if st != MUON_OK:
        raise MuonError(st, "muon_newton_schulz_batched")
    if check_default if check is None else check:
        workspace_status(ws, stream)
    return outs, count
