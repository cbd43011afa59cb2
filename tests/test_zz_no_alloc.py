"""muon_step_batched_noalloc (the library's fixed device scratch instead of
a workspace) against muon_step_batched on the same inputs, through the C
ABI: two calls in a row, the second on smaller banks, must give the same
weights and momenta bit for bit (both run the same tile code; the scratch
entry point runs every tiled pass as one launch per product, which the
persistent launch matches bit for bit).  A step that needs more than the
scratch is refused before anything is written."""

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _banks(specs, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    out = []
    for b, r, c, split, gdt in specs:
        w = torch.randn((b, r, c), generator=g) * 0.02
        gr = torch.randn((b, r, c), generator=g) * 1e-3
        if b > 1:
            gr[b - 1].zero_()  # one all-zero unit
        out.append((w.to(DEV), gr.to(torch.bfloat16 if gdt == "bf16" else torch.float32).to(DEV), split))
    return out


CALLS = [
    # 256 tiles (two panels per side), split heads on 128 tiles, a ragged tall
    # bank with fp32 gradients, a unit small enough for the on-chip kernel,
    # and a single 256-tile unit (with a workspace it runs inside the first
    # bank's persistent launch; the scratch entry runs it on its own)
    [(4, 512, 768, 0, "bf16"), (2, 384, 1024, 128, "bf16"), (3, 300, 200, 0, "fp32"),
     (1, 64, 128, 0, "fp32"), (1, 640, 512, 0, "bf16")],
    # smaller: fewer, smaller units
    [(2, 256, 300, 0, "bf16"), (1, 64, 128, 0, "fp32")],
]


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_noalloc_matches_the_workspace_entry_point(gpu_lib, prec):
    for k, specs in enumerate(CALLS):
        print(f"[noalloc] call {k}: {specs} products {prec}", flush=True)
        banks = _banks(specs, 40 + k)
        splits = [s for _, _, s in banks]
        res = {}
        for entry in ("workspace", "noalloc"):
            h = gpu_lib.Hyper(ns_precision=prec)
            params = [w.clone() for w, _, _ in banks]
            moms = [torch.zeros_like(w) for w, _, _ in banks]
            grads = [g for _, g, _ in banks]
            for t in range(2):  # the second step starts from a live momentum
                if entry == "workspace":
                    gpu_lib.step(params, grads, moms, hyper=h, split_rows=splits)
                else:
                    gpu_lib.step_noalloc(params, grads, moms, hyper=h, split_rows=splits)
            torch.cuda.synchronize()
            res[entry] = (params, moms)
        for i in range(len(banks)):
            assert torch.equal(res["workspace"][0][i], res["noalloc"][0][i]), f"call {k} params {i}"
            assert torch.equal(res["workspace"][1][i], res["noalloc"][1][i]), f"call {k} momenta {i}"


def test_noalloc_refuses_a_step_beyond_the_scratch(gpu_lib):
    # 40 units of 1024 x 1024 need 320 MiB of workspace on the bf16 path
    print("[noalloc] 40 x 1024^2: beyond the scratch", flush=True)
    w = torch.zeros((40, 1024, 1024), device=DEV)
    g = torch.ones((40, 1024, 1024), device=DEV, dtype=torch.bfloat16)
    m = torch.zeros_like(w)
    assert gpu_lib.workspace_size([w], gpu_lib.Hyper()) > 128 << 20
    with pytest.raises(gpu_lib.MuonError) as e:
        gpu_lib.step_noalloc([w], [g], [m])
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert torch.count_nonzero(m).item() == 0  # nothing ran
