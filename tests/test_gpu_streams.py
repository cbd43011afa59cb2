"""Steps on two streams at once.  The binding caches one workspace per
(device, stream), so two calls that overlap on the device never share claim
queues, completion counts or iterates; and a workgroup of a persistent launch
only waits for items claimed by running workgroups, so two such launches may
share the CUs in any proportion.  Overlapping steps must then give the
weights and momenta of the same steps run one after the other, bit for bit."""

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"

# (batch, rows, cols, split_rows).  One set per stream, of different
# workspace sizes: stacked 256-tile passes (persistent), a pass of one
# 256-tile unit, long 128-row units on chip, split heads and a one-block unit.
SETS = [
    [(4, 1024, 1024, 0), (1, 512, 768, 0), (8, 128, 1024, 0)],
    [(3, 768, 512, 0), (2, 256, 1536, 128), (1, 64, 128, 0)],
]
STEPS = 2


def _inputs(banks, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    w0 = [(torch.randn((b, r, c), generator=g) * 0.02).to(DEV) for b, r, c, _ in banks]
    grads = [[(torch.randn((b, r, c), generator=g) * 1e-3).to(DEV).to(torch.bfloat16)
              for b, r, c, _ in banks] for _ in range(STEPS)]
    return w0, grads


def test_overlapping_steps_on_two_streams_match_sequential_steps(gpu_lib):
    print(f"[streams] sets {SETS}", flush=True)
    h = gpu_lib.Hyper()
    data = [_inputs(banks, 300 + i) for i, banks in enumerate(SETS)]
    splits = [[b[3] for b in banks] for banks in SETS]

    # one after the other, on the current stream
    expect = []
    for (w0, grads), sp in zip(data, splits):
        w = [x.clone() for x in w0]
        m = [torch.zeros_like(x) for x in w0]
        for k in range(STEPS):
            gpu_lib.step(w, grads[k], m, hyper=h, split_rows=sp, check=True)
        expect.append((w, m))
    torch.cuda.synchronize()

    # both sets at once, each on a stream of its own (default priority)
    streams = [torch.cuda.Stream(device=DEV) for _ in SETS]
    state = [([x.clone() for x in w0], [torch.zeros_like(x) for x in w0]) for w0, _ in data]
    torch.cuda.synchronize()
    for k in range(STEPS):
        for (w, m), (_, grads), sp, s in zip(state, data, splits, streams):
            gpu_lib.step(w, grads[k], m, hyper=h, split_rows=sp, stream=s, check=False)
    wss = [gpu_lib.workspace(0, torch.device(DEV), s) for s in streams]
    assert wss[0].data_ptr() != wss[1].data_ptr()
    for ws, s in zip(wss, streams):
        gpu_lib.workspace_status(ws, s)
    torch.cuda.synchronize()

    for i, ((w, m), (ew, em)) in enumerate(zip(state, expect)):
        for j in range(len(SETS[i])):
            assert torch.equal(w[j], ew[j]), f"set {i}, params of bank {j}"
            assert torch.equal(m[j], em[j]), f"set {i}, momenta of bank {j}"
