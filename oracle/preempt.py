"""Block swap to host memory, and sliding-window block release.

"PagedAttention por dentro" (blog.lo0.es):
  - "Eviccion y preemption", "Estrategia 2: swap": when the block pool is
    exhausted a running session may be preempted; with swap its blocks are
    moved to CPU memory over PCIe, which frees their VRAM, and moved back
    when the session is scheduled again, so nothing is recomputed.
  - "Sliding window attention" (under "Lo que vLLM hace hoy"): a model that
    attends only to the last W tokens needs only the blocks of the active
    window; the engine frees the older ones and the cache no longer grows
    without bound.

Readings where the pages are silent:
  - the swap space is a second block pool of the same block shape, with its
    own free list and refcounts; a swap hands each distinct block of the
    moved references one fresh block on the other side (first-seen order),
    whose refcount is the number of moved references to it, then drops those
    references on the source side;
  - a block is released when all 16 of its positions lie before the window
    start of the earliest query still to run (``attention.window_start``);
    its table entry becomes -1.
"""
from __future__ import annotations

from .attention import window_start
from .pool import BLOCK_SIZE, PoolError, PoolModel


def swap(src: PoolModel, dst: PoolModel, ids):
    """Moves the references ``ids`` held in ``src`` to fresh blocks of
    ``dst``.  Returns (new ids, one per reference; pairs (old, new), one per
    distinct block).  All-or-nothing: PoolError and both pools unchanged."""
    if src is dst:
        raise PoolError("invalid", "swap within one pool")
    ids = [int(i) for i in ids]
    distinct = []
    count = {}
    for i in ids:
        if not (0 <= i < src.num_blocks):
            raise PoolError("invalid", f"block {i} out of range")
        if i not in count:
            distinct.append(i)
            count[i] = 0
        count[i] += 1
    for i in distinct:
        if count[i] > src.refcount[i]:
            raise PoolError("invalid", f"block {i}: {count[i]} references moved, "
                                       f"{src.refcount[i]} held")
    if len(distinct) > dst.num_free():
        raise PoolError("oom", f"want {len(distinct)}, free {dst.num_free()}")
    new_of = {}
    for i in distinct:
        (n,) = dst.alloc(1)
        dst.refcount[n] = count[i]
        new_of[i] = n
    src.free(ids)
    return [new_of[i] for i in ids], [(i, new_of[i]) for i in distinct]


def releasable(L: int, window: int):
    """Table indices whose blocks hold only positions before the window start
    of a query with context length L (position L - 1)."""
    lo = window_start(L - 1, window) if L > 0 else 0
    out = []
    for i in range(-(-L // BLOCK_SIZE)):
        if all(p < lo for p in range(i * BLOCK_SIZE, (i + 1) * BLOCK_SIZE)):
            out.append(i)
    return out


def window_release(pool_: PoolModel, tables, query_lens, window: int):
    """For each sequence s, releases the blocks of ``releasable(query_lens[s],
    window)`` still in its table (entry >= 0): one reference dropped, entry set
    to -1.  ``tables`` is a list of mutable rows.  Returns the updates
    [(s, index, -1)].  All-or-nothing."""
    if window < 1:
        raise PoolError("invalid", "window < 1")
    drops, updates = [], []
    for s, row in enumerate(tables):
        L = int(query_lens[s])
        if L < 0 or L > len(row) * BLOCK_SIZE:
            raise PoolError("invalid", f"length {L}")
        for i in releasable(L, window):
            if row[i] >= 0:
                drops.append(int(row[i]))
                updates.append((s, i, -1))
    snap = pool_.snapshot()
    try:
        pool_.free(drops)
    except PoolError:
        pool_.restore(snap)
        raise
    for s, i, _ in updates:
        tables[s][i] = -1
    return updates
