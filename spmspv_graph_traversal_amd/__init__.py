"""DB-SpMSpV for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library ``libdbs.so`` (C ABI in
``include/dbs.h``); :mod:`spmspv_graph_traversal_amd.binding` marshals torch
tensors into it.  Attribute access on this package loads the binding and
fails with ``ImportError`` when the library has not been built; the build
helper :mod:`spmspv_graph_traversal_amd.build_lib` imports without it.
"""
import importlib

__all__ = ["binding"]

_SUBMODULES = ("binding", "build_lib")


def __getattr__(name):
    if name in _SUBMODULES:
        return importlib.import_module(f".{name}", __name__)
    if name.startswith("__"):
        raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
    binding = importlib.import_module(".binding", __name__)
    try:
        return getattr(binding, name)
    except AttributeError:
        raise AttributeError(f"module {__name__!r} has no attribute {name!r}") from None
