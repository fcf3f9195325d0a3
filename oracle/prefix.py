"""Prefix caching by block hash, on top of the pool model.

"Como funciona realmente vLLM" (alexanderzelada.com), "Automatic Prefix
Caching: reutilizar el contexto entre peticiones": when a request ends its
blocks are not dropped but indexed by their content, and a later request
that starts with the same tokens reuses them from VRAM instead of
recomputing them.  "PagedAttention por dentro" (blog.lo0.es), "Prefix
caching cross-session": full blocks are hashed (no radix tree).

Readings (the pages give no more detail):
  - only full blocks are indexed; a block's identity is its 16 token ids and
    the indexed block holding the previous 16 tokens -- here the key is the
    whole token prefix up to the block's end, looked up block by block from
    the first, so a block matches only as part of a matching prefix;
  - an indexed block whose references are all dropped stays indexed on a
    second free list, least recently freed first; allocation takes blocks
    holding nothing first (the pool's LIFO stack) and only then evicts the
    least recently freed indexed block, which leaves the index together with
    every block indexed below it (they keep their place on the free lists);
  - registering a sequence's blocks indexes those whose prefix is not yet
    indexed; where the same prefix is already indexed under another block,
    the chain continues through that block.
This model keys blocks by exact token tuples (no hash), so it states the
result a hash index must give when it confirms its hits.
"""
from __future__ import annotations

from collections import OrderedDict

from .pool import BLOCK_SIZE, PoolError, PoolModel


class PrefixPoolModel(PoolModel):
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, init_order=None):
        super().__init__(num_blocks, block_size, init_order)
        self._key_of = {}            # block -> token prefix tuple (indexed blocks)
        self._block_of = {}          # token prefix tuple -> block
        self._lru = OrderedDict()    # indexed free blocks, least recently freed first

    # -- free-list policy ----------------------------------------------------------
    def free_list(self):
        return list(reversed(self._free)) + list(self._lru)

    def num_free(self) -> int:
        return len(self._free) + len(self._lru)

    def stats(self) -> dict:
        st = super().stats()
        st["num_free"] = self.num_free()
        return st

    def _drop_index(self, b: int):
        """b and every block indexed below it (longer prefixes through b) leave the index."""
        key = self._key_of.get(b)
        if key is None:
            return
        below = [x for x, k in self._key_of.items() if len(k) > len(key) and k[:len(key)] == key
                 and self._block_of.get(k[:len(key)]) == b]
        for x in [b] + below:
            k = self._key_of.pop(x, None)
            if k is not None and self._block_of.get(k) == x:
                del self._block_of[k]

    def _take(self) -> int:
        if self._free:
            return self._free.pop()
        b, _ = self._lru.popitem(last=False)
        self._drop_index(b)
        return b

    def alloc(self, n: int):
        if n < 0:
            raise PoolError("invalid", "n < 0")
        if n > self.num_free():
            raise PoolError("oom", f"want {n}, free {self.num_free()}")
        ids = [self._take() for _ in range(n)]
        for i in ids:
            self.refcount[i] = 1
        return ids

    def free(self, ids):
        ids = [int(i) for i in ids]
        drops = {}
        for i in ids:
            if not (0 <= i < self.num_blocks):
                raise PoolError("invalid", f"block {i} out of range")
            drops[i] = drops.get(i, 0) + 1
        for i, k in drops.items():
            if k > self.refcount[i]:
                raise PoolError("invalid", f"block {i}: {k} drops, {self.refcount[i]} refs")
        for i in ids:
            self.refcount[i] -= 1
            if self.refcount[i] == 0:
                if i in self._key_of:
                    self._lru[i] = None
                else:
                    self._free.append(i)

    def cow(self, i: int):
        self._check_live(i)
        if self.refcount[i] == 1:
            return i, False
        if self.num_free() == 0:
            raise PoolError("oom", "no free block for copy-on-write")
        new = self._take()
        self.refcount[new] = 1
        self.refcount[i] -= 1
        return new, True

    # -- prefix caching ---------------------------------------------------------------
    def match(self, tokens, max_blocks=None):
        """Blocks holding the longest indexed prefix of ``tokens`` (full
        blocks only); one reference is taken on each."""
        tokens = tuple(int(t) for t in tokens)
        full = len(tokens) // BLOCK_SIZE
        if max_blocks is not None:
            full = min(full, max_blocks)
        out = []
        for i in range(full):
            b = self._block_of.get(tokens[:BLOCK_SIZE * (i + 1)])
            if b is None:
                break
            out.append(b)
        for b in out:
            if self.refcount[b] == 0:
                del self._lru[b]
            self.refcount[b] += 1
        return out

    def register(self, tokens, block_ids):
        tokens = tuple(int(t) for t in tokens)
        ids = [int(b) for b in block_ids]
        full = len(tokens) // BLOCK_SIZE
        if len(ids) < full:
            raise PoolError("invalid", "fewer block ids than full blocks")
        ids = ids[:full]
        for i, b in enumerate(ids):
            self._check_live(b)
            if b in ids[:i]:
                raise PoolError("invalid", f"block {b} twice")
            key = tokens[:BLOCK_SIZE * (i + 1)]
            if b in self._key_of and self._key_of[b] != key:
                raise PoolError("invalid", f"block {b} indexed with other content")
        for i, b in enumerate(ids):
            key = tokens[:BLOCK_SIZE * (i + 1)]
            if b in self._key_of or key in self._block_of:
                continue
            self._key_of[b] = key
            self._block_of[key] = b

    def cached(self):
        """(indexed blocks, indexed free blocks)."""
        return len(self._key_of), len(self._lru)

    def snapshot(self):
        return (list(self._free), list(self.refcount), dict(self._key_of), dict(self._block_of),
                OrderedDict(self._lru))

    def restore(self, snap):
        (self._free, self.refcount, self._key_of, self._block_of, self._lru) = (
            list(snap[0]), list(snap[1]), dict(snap[2]), dict(snap[3]), OrderedDict(snap[4]))

    def check_invariants(self, tables=None):
        free_set = set(self._free) | set(self._lru)
        assert len(free_set) == len(self._free) + len(self._lru), "id twice on the free lists"
        for i in range(self.num_blocks):
            assert (i in free_set) == (self.refcount[i] == 0), f"block {i}"
        for b, k in self._key_of.items():
            assert self._block_of.get(k) == b
            if len(k) > BLOCK_SIZE:
                assert k[:-BLOCK_SIZE] in self._block_of, "indexed block without indexed parent"
        if tables is not None:
            counts = [0] * self.num_blocks
            for row in tables:
                for i in row:
                    counts[int(i)] += 1
            assert counts == self.refcount
