"""The persistent schedule's stop path, driven from the host.

MUON_WAIT_LIMIT_US=0 makes every dependency wait give up at its first
unsuccessful look, so a persistent launch whose tiles must wait stops: every
workgroup leaves normally and the workspace's status reports it.  On one
4096 x 4096 unit (136 Gram tiles of K = 4096 on 256 workgroups) the
polynomial tiles are claimed while the Gram still runs, so they wait.  The
report is sticky until muon_workspace_status reads it."""

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_stop_is_reported_sticky_and_cleared(gpu_lib, monkeypatch):
    print("[status] one 4096x4096 unit, persistent schedule, zero wait limit", flush=True)
    g = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn((1, 4096, 4096), generator=g).to(DEV)
    h = gpu_lib.Hyper(schedule="persistent")
    ws = gpu_lib.workspace(gpu_lib.workspace_size([x], h), torch.device(DEV))
    out = torch.empty_like(x)

    def run(check):
        gpu_lib.newton_schulz([x], [out], hyper=h, ws=ws, check=check)

    run(False)
    gpu_lib.workspace_status(ws)  # a clean call reports nothing
    monkeypatch.setenv("MUON_WAIT_LIMIT_US", "0")
    run(False)
    with pytest.raises(gpu_lib.MuonError) as e:
        gpu_lib.workspace_status(ws)
    assert e.value.status == -9
    gpu_lib.workspace_status(ws)  # read once, then cleared
    # sticky: a stopped call followed by a clean one is still reported
    run(False)
    monkeypatch.delenv("MUON_WAIT_LIMIT_US")
    run(False)
    with pytest.raises(gpu_lib.MuonError):
        gpu_lib.workspace_status(ws)
    # the binding's check raises on a stop
    monkeypatch.setenv("MUON_WAIT_LIMIT_US", "0")
    with pytest.raises(gpu_lib.MuonError):
        run(True)
    monkeypatch.delenv("MUON_WAIT_LIMIT_US")
    # and clean calls afterwards report nothing and give the right output
    run(True)
    ref = torch.empty_like(x)
    gpu_lib.newton_schulz([x], [ref], hyper=gpu_lib.Hyper(schedule="launches"), check=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_stop_report_kept_through_a_one_launch_call(gpu_lib, monkeypatch):
    # A call whose only launch is the one-workgroup small-unit step (a
    # 64 x 128 unit, bf16 products) moves the previous call's stop flag into
    # the sticky word like any first launch of a call.
    print("[status] stop, then a one-launch 64x128 call on the same workspace", flush=True)
    g = torch.Generator(device="cpu").manual_seed(6)
    x = torch.randn((1, 4096, 4096), generator=g).to(DEV)
    small = torch.randn((64, 128), generator=g).to(DEV)
    h = gpu_lib.Hyper(schedule="persistent")
    ws = gpu_lib.workspace(gpu_lib.workspace_size([x], h), torch.device(DEV))
    hs = gpu_lib.Hyper()
    assert gpu_lib.workspace_size([small], hs) <= ws.numel()
    out, out_s = torch.empty_like(x), torch.empty_like(small)
    monkeypatch.setenv("MUON_WAIT_LIMIT_US", "0")
    gpu_lib.newton_schulz([x], [out], hyper=h, ws=ws, check=False)
    monkeypatch.delenv("MUON_WAIT_LIMIT_US")
    gpu_lib.newton_schulz([small], [out_s], hyper=hs, ws=ws, check=False)
    with pytest.raises(gpu_lib.MuonError) as e:
        gpu_lib.workspace_status(ws)
    assert e.value.status == -9
    gpu_lib.newton_schulz([small], [out_s], hyper=hs, ws=ws, check=True)


def test_split_unit_stop_is_reported_and_the_next_call_is_clean(gpu_lib, monkeypatch):
    # 12 wide 128 x 4096 units are split over 8 workgroups each, which wait
    # for each other's partial Grams once per iteration.  With a zero wait
    # limit the first group to publish gives up at once (the other seven are
    # still in their column blocks): the call reports the stop, and the
    # counters it left do not disturb the next call, which matches a clean
    # run bit for bit.
    print("[status] split units, zero wait limit", flush=True)
    g = torch.Generator(device="cpu").manual_seed(8)
    x = torch.randn((12, 128, 4096), generator=g).to(DEV)
    h = gpu_lib.Hyper()
    ws = gpu_lib.workspace(gpu_lib.workspace_size([x], h), torch.device(DEV))
    ref, out = torch.empty_like(x), torch.empty_like(x)
    gpu_lib.newton_schulz([x], [ref], hyper=h, ws=ws, check=True)
    monkeypatch.setenv("MUON_WAIT_LIMIT_US", "0")
    gpu_lib.newton_schulz([x], [out], hyper=h, ws=ws, check=False)
    monkeypatch.delenv("MUON_WAIT_LIMIT_US")
    with pytest.raises(gpu_lib.MuonError) as e:
        gpu_lib.workspace_status(ws)
    assert e.value.status == -9
    gpu_lib.newton_schulz([x], [out], hyper=h, ws=ws, check=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
