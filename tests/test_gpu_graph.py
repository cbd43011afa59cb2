"""A step captured in a HIP graph and replayed.  Every kernel of a step
resets what it counts on (claim queues, completion counts, the status word)
by its own writes, and the step allocates nothing once its workspace
exists, so a captured step replays like an eager one: each replay, with
new gradients copied into the captured buffer and the stream synchronised
in between, must give the eager step's weights and momenta bit for bit."""

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"

# A stacked 256-tile pass with a single unit riding in its persistent launch
# (workspace entry), split heads of 12 column blocks (on chip, split over
# workgroups that wait on each other), and a one-block unit (one launch).
BANKS = [(3, 512, 768, 0), (1, 640, 512, 0), (2, 256, 1536, 128), (1, 64, 128, 0)]


def _inputs(seed, steps):
    g = torch.Generator(device="cpu").manual_seed(seed)
    w0 = [(torch.randn((b, r, c), generator=g) * 0.02).to(DEV) for b, r, c, _ in BANKS]
    grads = [[(torch.randn((b, r, c), generator=g) * 1e-3).to(DEV).to(torch.bfloat16)
              for b, r, c, _ in BANKS] for _ in range(steps)]
    return w0, grads


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_captured_step_replays_like_eager_steps(gpu_lib, entry):
    print(f"[graph] entry {entry}: {BANKS}", flush=True)
    steps = 3
    h = gpu_lib.Hyper()
    splits = [b[3] for b in BANKS]
    w0, grads = _inputs(77, steps)
    ws = None
    if entry == "workspace":
        ws = gpu_lib.workspace(gpu_lib.workspace_size(w0, h, splits), torch.device(DEV))

    def one(params, g, moms):
        if entry == "workspace":
            gpu_lib.step(params, g, moms, hyper=h, split_rows=splits, ws=ws, check=False)
        else:
            gpu_lib.step_noalloc(params, g, moms, hyper=h, split_rows=splits)

    # eager reference, step by step
    ref_w = [w.clone() for w in w0]
    ref_m = [torch.zeros_like(w) for w in w0]
    expect = []
    for k in range(steps):
        one(ref_w, grads[k], ref_m)
        torch.cuda.synchronize()
        expect.append(([w.clone() for w in ref_w], [m.clone() for m in ref_m]))
    if ws is not None:
        gpu_lib.workspace_status(ws)

    # captured: static weights, momenta and gradients (nothing runs while
    # capturing, so they keep their initial values)
    sw = [w.clone() for w in w0]
    sm = [torch.zeros_like(w) for w in w0]
    sg = [g.clone() for g in grads[0]]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one(sw, sg, sm)
    torch.cuda.synchronize()
    for a, b in zip(sw, w0):
        assert torch.equal(a, b)
    for k in range(steps):
        for dst, src in zip(sg, grads[k]):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(BANKS)):
            assert torch.equal(sw[i], expect[k][0][i]), f"replay {k}: params of bank {i}"
            assert torch.equal(sm[i], expect[k][1][i]), f"replay {k}: momenta of bank {i}"
    if ws is not None:
        gpu_lib.workspace_status(ws)
    del graph
