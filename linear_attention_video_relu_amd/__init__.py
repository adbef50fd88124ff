"""Block-causal ReLU linear attention with RoPE on AMD MI355X (gfx950).

The compute runs in the HIP library ``liblavr.so`` (built from ``csrc/``) behind a
C ABI declared in ``include/la_vr.h``; ``lavr`` is the thin ctypes binding to it and
``workloads`` names the benchmark shapes and draws seeded synthetic inputs.
The binding is imported on first use so that ``workloads`` works without the
built library.
"""

import importlib

__all__ = ["lavr", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
