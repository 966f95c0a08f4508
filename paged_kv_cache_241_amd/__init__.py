"""Paged KV cache and single-token decode attention for AMD MI355X (gfx950).

The product is ``libpa.so`` (C ABI in ``include/pa.h``): a host block
allocator (allocate-on-fill, free, shared blocks with share counts,
copy-on-write) and hand-written HIP kernels for the KV append, the
copy-on-write block copy and paged decode attention.  This package is its thin
Python binding: ``capi`` declares the C functions under their own names,
``Pool`` wraps them around torch device memory and streams.
"""

from . import capi  # noqa: F401
from .pool import Pool  # noqa: F401

__all__ = ["capi", "Pool"]
