"""Paged KV cache and PagedAttention decode for AMD Instinct MI355X (gfx950).

The work is done by libpagedkv.so (C ABI in include/pagedkv.h): a host block
pool with reference counts and copy-on-write, slot planning, and HIP kernels
for the cache write, block copies, table updates and decode attention.
``_capi`` binds every C entry point under its own name; ``driver.PagedKV``
sequences them for one decode step.
"""
from . import _capi
from ._capi import *  # noqa: F401,F403  (the C ABI names)

__all__ = list(_capi.EXPORTED) + ["PkvError", "Pool"]
