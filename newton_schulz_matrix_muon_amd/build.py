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


# Host code built with AddressSanitizer and UndefinedBehaviorSanitizer (the
# device code is compiled as usual): the CPU tests run the ABI suite, which
# drives the host planner, against this build.  It loads only with the ASan
# runtime preloaded (see tests/test_sanitizers.py).
SAN_LIB = os.path.join(ROOT, "_build", "libmuon_san.so")
SAN_FLAGS = [
    "--offload-arch=gfx950",
    "-O1",
    "-g",
    "-std=c++17",
    "-shared",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Wno-unused-result",
    "-Wno-inline-asm",
    "-I", os.path.join(ROOT, "include"),
]


def build_sanitized(verbose: bool = False) -> str:
    """Compile the host-sanitized library into _build/ unless it is newer
    than every source."""
    if os.path.exists(SAN_LIB) and all(os.path.getmtime(p) <= os.path.getmtime(SAN_LIB) for p in DEPS):
        return SAN_LIB
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, *SAN_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc (sanitizer build) failed:\n" + (res.stdout + res.stderr)[-4000:])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime."""
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True)
    return out.stdout.strip()


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
