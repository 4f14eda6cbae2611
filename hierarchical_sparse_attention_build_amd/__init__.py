"""HGA routed attention for MI355X (gfx950).

The compute path is the HIP shared library ``libhga.so`` built from ``csrc/``;
``hga`` is a thin ctypes binding over its C-ABI (argument marshalling only).
``workloads`` draws seeded synthetic inputs.  Submodules are imported on first
use, so importing the package loads no native code.
"""
import importlib

__all__ = ["hga", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
