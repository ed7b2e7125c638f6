"""Routed Mixture-of-Experts layer for MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind the C ABI
of ``include/moe.h``); ``ops`` marshals PyTorch tensors and streams into it.
Importing the package does not load the library; the first call does, and it
raises if the library has not been built.
"""

from . import bytemodel  # noqa: F401

__all__ = ["ops", "bytemodel"]
