"""Paged sliding-window two-stream KV cache and paged prefill attention for
AMD MI355X (gfx950).

The library is ``libpsw.so`` (C ABI in ``include/psw.h``): host page
bookkeeping in C++ and HIP kernels for the K/V append and the attention.
This package is its Python binding (``Cache``) and build script.
"""
from ._lib import PswError, load
from .cache import Cache

__all__ = ["Cache", "PswError", "load"]
