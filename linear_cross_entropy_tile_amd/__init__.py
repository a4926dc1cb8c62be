"""Fused linear cross-entropy + entropy head for MI355X (gfx950).

The compute lives in the HIP library ``libflce.so`` behind a C ABI
(``include/flce.h``); ``linear_cross_entropy_tile_amd.flce`` is the thin ctypes
binding with the same entry-point names. Importing this package loads nothing;
the library is opened on first use and a missing library is an error.
``linear_cross_entropy_tile_amd.function.linear_cross_entropy`` wraps the
forward and backward entry points as a torch autograd function.
"""
__all__ = ["flce", "function", "workloads"]
