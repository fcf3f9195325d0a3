"""Slot planning: where each appended token's K/V goes.

Follows "PagedAttention por dentro" (blog.lo0.es), "La tabla de paginas
(block table)": the block holding token p of a sequence is at table
position p // 16 (the page's example: token 200 -> position 12); when a
sequence produces a token, it goes into the last block if that block still
has room (the page's test "N mod 16 != 0"), otherwise a new block is taken
from the global pool, appended to the table and the token is written into
its first slot.  "Copy-on-write para sampling paralelo": a shared last
block is replaced by a private copy before the write.

Reading of the page's "N mod 16" test: N is the number of tokens already
cached, i.e. the 0-based position p of the new token; a new block is taken
exactly when p % 16 == 0.  This matches token 200 sitting at position 12
with 0-based positions.
"""
from __future__ import annotations

import numpy as np

from .pool import BLOCK_SIZE, PoolError, PoolModel


def blocks_for(num_tokens: int) -> int:
    """Blocks a sequence of num_tokens tokens occupies: ceil(n / 16)."""
    return -(-int(num_tokens) // BLOCK_SIZE)


def slot_of(table_row, p: int) -> int:
    """Flat slot (block * 16 + offset) of token position p."""
    return int(table_row[p // BLOCK_SIZE]) * BLOCK_SIZE + p % BLOCK_SIZE


def plan_append(pool: PoolModel, tables: np.ndarray, lens: np.ndarray, num_new=None):
    """Plan the cache slots of newly appended tokens, sequence by sequence.

    tables: int32 [B][max_blocks] (updated in place); lens: int32 [B]
    (updated in place); num_new: tokens appended per sequence (default 1).
    Returns (slots int64 [sum num_new], updates [(flat index, id)],
    cow_pairs [(src, dst)]).  All or nothing: on error, pool, tables and
    lens are restored and the PoolError is re-raised; "invalid" (a position
    beyond the table, a dead table entry) takes precedence over "oom"."""
    B, max_blocks = tables.shape
    if num_new is None:
        num_new = np.ones(B, dtype=np.int64)
    # Argument errors are reported before pool exhaustion: every sequence's
    # new positions must fit its table, and a partly filled last block that
    # receives tokens must be a live block.
    for s in range(B):
        add, p0 = int(num_new[s]), int(lens[s])
        if add < 0 or p0 < 0 or p0 + add > max_blocks * BLOCK_SIZE:
            raise PoolError("invalid", f"sequence {s}: positions beyond the table")
        if add > 0 and p0 % BLOCK_SIZE != 0:
            blk = int(tables[s, p0 // BLOCK_SIZE])
            if not (0 <= blk < pool.num_blocks) or pool.refcount[blk] == 0:
                raise PoolError("invalid", f"sequence {s}: table entry {blk} is not live")
    snap = pool.snapshot()
    tables_before = tables.copy()
    lens_before = lens.copy()
    slots, updates, cows = [], [], []
    try:
        for s in range(B):
            p, end = int(lens[s]), int(lens[s]) + int(num_new[s])
            # the new tokens p .. end-1, one block's run at a time
            while p < end:
                pos = p // BLOCK_SIZE
                if p % BLOCK_SIZE == 0:
                    (blk,) = pool.alloc(1)
                    tables[s, pos] = blk
                    updates.append((s * max_blocks + pos, blk))
                else:
                    old = int(tables[s, pos])
                    new, copied = pool.cow(old)
                    if copied:
                        tables[s, pos] = new
                        updates.append((s * max_blocks + pos, new))
                        cows.append((old, new))
                run = min(end, (pos + 1) * BLOCK_SIZE) - p
                slots.extend(slot_of(tables[s], q) for q in range(p, p + run))
                p += run
                lens[s] = p
    except PoolError:
        pool.restore(snap)
        tables[...] = tables_before
        lens[...] = lens_before
        raise
    return np.array(slots, dtype=np.int64), updates, cows


def waste_slots(num_tokens: int) -> int:
    """Empty slots in a sequence's last block (internal fragmentation):
    ceil(n/16)*16 - n, between 0 and 15."""
    return blocks_for(num_tokens) * BLOCK_SIZE - int(num_tokens)
