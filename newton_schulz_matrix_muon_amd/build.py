"""Compile the HIP library libmuon.so for gfx950, in-tree.

    python -m newton_schulz_matrix_muon_amd.build

hipcc cross-compiles without a GPU.  The library is written next to this
file so that it travels with the source tree.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmuon.so")
SOURCES = [os.path.join(HERE, "csrc", "muon.hip")]
DEPS = SOURCES + [
    os.path.join(HERE, "csrc", "kernels.hpp"),
    os.path.join(ROOT, "include", "muon.h"),
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    "-mcode-object-version=5",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep private arrays out of LDS (the GEMM tiles size their LDS exactly)
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wno-unused-result",
    # the LDS copy names M0 as clobbered on purpose (it sets M0 itself)
    "-Wno-inline-asm",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = True, extra: list[str] | None = None) -> str:
    """Compile libmuon.so (always; a stale library is replaced)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [
        ln
        for ln in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in ln and ln.strip()
    ]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
