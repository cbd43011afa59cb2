"""MI355X (gfx950) Muon optimizer step: HIP kernels behind a C ABI.

`newton_schulz_matrix_muon_amd.muon` is the ctypes binding of
include/muon.h; it is imported on first use so that the build step can run
before the library exists.
"""

import importlib

__all__ = ["muon", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
