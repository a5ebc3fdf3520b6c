"""RotateAttention INT4 FlashAttention forward for 3D-RoPE video DiTs, on MI355X.

The compute path is the C-ABI library ``libra_attn.so`` (hand-written HIP for
gfx950, declared in ``include/ra_attn.h``).  This package is its thin Python
binding: argument marshalling only; PyTorch supplies device memory and the
stream.  Importing the package loads nothing; the native library is opened on
first use and a missing library is an error, never a fallback.
"""
from .inputs import Workload, WORKLOADS  # noqa: F401

__all__ = ["Workload", "WORKLOADS", "native", "api"]


def __getattr__(name):
    if name in ("native", "api"):
        import importlib
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
