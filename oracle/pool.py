"""Block pool model (free list + reference counts + copy-on-write).

Follows "PagedAttention por dentro" (blog.lo0.es):
  - "El pool de bloques": a single global pool of fixed 16-token blocks,
    sized once; taking a block is O(1);
  - the figure in "La tabla de paginas (block table)": a finished session's
    blocks go back to the pool and another session takes them next step;
  - "Copy-on-write para sampling paralelo": several sequences point at the
    same physical blocks; a shared block is copied only when one of them
    is about to modify it, like fork().
The free-list discipline (LIFO) and the all-or-nothing error rules are this
library's reading; the pages do not fix them.
"""
from __future__ import annotations

BLOCK_SIZE = 16


class PoolError(Exception):
    """kind is one of "invalid", "oom", "unsupported"."""

    def __init__(self, kind: str, msg: str = ""):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, init_order=None):
        if block_size != BLOCK_SIZE:
            raise PoolError("unsupported", f"block_size {block_size}")
        if num_blocks < 1:
            raise PoolError("invalid", "num_blocks < 1")
        order = list(range(num_blocks)) if init_order is None else [int(x) for x in init_order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError("invalid", "init_order is not a permutation")
        self.num_blocks = num_blocks
        # Python list as a stack: the top is the end, so order[0] is popped first.
        self._free = list(reversed(order))
        self.refcount = [0] * num_blocks

    # -- queries ---------------------------------------------------------------
    def free_list(self):
        """Free ids, the next one to be allocated first."""
        return list(reversed(self._free))

    def num_free(self) -> int:
        return len(self._free)

    def stats(self) -> dict:
        used = sum(1 for r in self.refcount if r > 0)
        return {
            "num_blocks": self.num_blocks,
            "num_free": len(self._free),
            "num_used": used,
            "num_shared": sum(1 for r in self.refcount if r > 1),
            "num_refs": sum(self.refcount),
            "usage_percent": 100.0 * used / self.num_blocks,
        }

    def _check_live(self, i: int):
        if not (0 <= i < self.num_blocks) or self.refcount[i] == 0:
            raise PoolError("invalid", f"block {i} is not a live block")

    # -- operations --------------------------------------------------------------
    def alloc(self, n: int):
        if n < 0:
            raise PoolError("invalid", "n < 0")
        if n > len(self._free):
            raise PoolError("oom", f"want {n}, free {len(self._free)}")
        ids = [self._free.pop() for _ in range(n)]
        for i in ids:
            self.refcount[i] = 1
        return ids

    def share(self, ids):
        ids = [int(i) for i in ids]
        for i in ids:
            self._check_live(i)
        for i in ids:
            self.refcount[i] += 1

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
                self._free.append(i)

    def cow(self, i: int):
        """Returns (id to write into, whether the caller must copy i -> it)."""
        self._check_live(i)
        if self.refcount[i] == 1:
            return i, False
        if not self._free:
            raise PoolError("oom", "no free block for copy-on-write")
        new = self._free.pop()
        self.refcount[new] = 1
        self.refcount[i] -= 1
        return new, True

    # -- snapshots (for all-or-nothing callers) --------------------------------------
    def snapshot(self):
        return (list(self._free), list(self.refcount))

    def restore(self, snap):
        self._free, self.refcount = list(snap[0]), list(snap[1])

    def check_invariants(self, tables=None):
        """Raises AssertionError if the pool is inconsistent.  With ``tables``
        (iterable of block-id lists), every refcount must equal the number of
        table entries pointing at that block."""
        free_set = set(self._free)
        assert len(free_set) == len(self._free), "id twice on the free list"
        for i in range(self.num_blocks):
            on_free = i in free_set
            assert on_free == (self.refcount[i] == 0), f"block {i}: refcount {self.refcount[i]}"
        used = sum(1 for r in self.refcount if r > 0)
        assert used + len(self._free) == self.num_blocks
        if tables is not None:
            counts = [0] * self.num_blocks
            for row in tables:
                for i in row:
                    counts[int(i)] += 1
            assert counts == self.refcount, "refcounts differ from table references"
