"""The largest unit the C ABI accepts, on the GPU.

A unit's padded bf16 iterate must stay under 2^31 bytes, since the K-major
operand copies address it with 32-bit offsets: 32512 x 32768 and its
transpose are the largest such units with a 32768 side.  Its Newton-Schulz output is checked on a
rectangular diagonal input, which the iteration keeps diagonal: after the
common Frobenius normalisation every diagonal entry follows the scalar
iteration on its own, so the expected entries come from the oracle run on
small diagonal blocks of the normalised entries (each block padded with one
entry that makes its Frobenius norm 1, so that the oracle's own
normalisation leaves it unchanged), and every off-diagonal entry must be
exactly zero.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL_NS, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _expected_diagonal(v):
    """Oracle NS of diag(v) for a vector v of Frobenius norm 1."""
    out = np.empty_like(v)
    block = 127
    for b in range(0, len(v), block):
        c = v[b:b + block]
        pad = math.sqrt(max(0.0, 1.0 - float(np.dot(c, c))))
        o = oracle.newton_schulz(np.diag(np.concatenate([c, [pad]])))
        out[b:b + len(c)] = np.diag(o)[:len(c)]
    return out


@pytest.mark.parametrize("rows,cols", [(32512, 32768), (32768, 32512)], ids=["wide", "tall"])
def test_largest_unit_on_a_diagonal_input(gpu_lib, rows, cols):
    # wide: the apply reads X K-major; tall: the Gram reads X K-major on both sides
    say(f"[limits] NS of one {rows}x{cols} unit (rectangular diagonal input)")
    n = min(rows, cols)
    rng = np.random.default_rng(31)
    d = rng.uniform(0.5, 1.5, n) * rng.choice([-1.0, 1.0], n)
    d32 = d.astype(np.float32)
    x = torch.zeros((1, rows, cols), dtype=torch.float32, device=DEV)
    idx = torch.arange(n, device=DEV)
    x[0, idx, idx] = torch.from_numpy(d32).to(DEV)
    outs, _ = gpu_lib.newton_schulz([x], hyper=gpu_lib.Hyper(ns_precision="bf16"))
    torch.cuda.synchronize()
    o = outs[0][0]
    diag = o[idx, idx].double().cpu().numpy()
    off = float(o.abs().sum(dtype=torch.float64)) - float(np.abs(diag).sum())
    del x, outs, o
    torch.cuda.empty_cache()
    v = d32.astype(np.float64)
    v /= np.linalg.norm(v)
    want = _expected_diagonal(v)
    e = float(np.linalg.norm(diag - want) / np.linalg.norm(want))
    say(f"   rel err of the diagonal {e:.3e}, off-diagonal mass {off:.3e}")
    assert off == 0.0
    assert e <= TOL_NS["bf16"]
