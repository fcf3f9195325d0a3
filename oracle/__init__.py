"""CPU oracle for the block-paged KV cache and PagedAttention decode.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct numpy code (fp64
for every floating-point result) that states what the GPU path must compute.
Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it; the product package never does, and this
package imports nothing from the product package (a test enforces both).

Modules and what each follows:
  pool       block pool with a LIFO free list, refcounts and copy-on-write
  slots      slot planning for appended tokens (block table growth)
  layout     element order of K and V inside a (block, kv head) tile, as the
             C ABI header defines it
  cache      the cache tensors: write through a slot mapping, block copies,
             gathering a sequence's K/V back through its table
  attention  decode attention by its textbook definition, plus the
             partition + log-sum-exp form used to pin the reduction
  sizes      byte and block counts printed on the pages
  replay     replays a synthetic workload (prefill recipe, append step)
  fp8        the OCP E4M3 codec of the FP8 cache (nearest, ties to even)
  prefix     prefix caching: block index by (parent block, tokens), LRU
  preempt    block swap to a host pool, sliding-window block release

Parity status: every function is pinned by the CPU tests (page fixtures,
closed forms, invariants, an independent library routine); none is
"parity unpinned".
"""
from . import (attention, cache, fp8, layout, pool, preempt, prefix, replay,  # noqa: F401
               sizes, slots)
