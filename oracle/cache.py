"""The cache tensors on the host: write, block copy, gather.

"KV cache: la memoria de trabajo ..." (blog.lo0.es), "El mecanismo en si":
the cache keeps the K and V of every token already processed, in every
layer.  "PagedAttention por dentro", "La tabla de paginas": a token is
found through its sequence's block table; "Copy-on-write para sampling
paralelo": a whole block is copied when a shared block diverges.
"Como funciona realmente vLLM", "PagedAttention: ...": the kernel reads the
scattered blocks through the table without copying them into a contiguous
buffer -- the gather below exists only to state the result, it is not a
step of the GPU path.

Values are kept exactly as stored (float32, bf16 as raw uint16 bits, or
FP8 E4M3 codes as uint8 with one scale per tensor); gathers widen them
exactly to float64 (FP8: the code's value times the tensor's scale).
"""
from __future__ import annotations

import numpy as np

from . import fp8 as fp8codec
from .layout import BLOCK_SIZE, offset_tables


def widen(stored: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Stored values -> float64, exactly (bf16 bits shift into float32; FP8
    codes decode to their value times ``scale``)."""
    if dtype == "fp8":
        return fp8codec.decode(stored) * float(np.float32(scale))
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        f = (np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
        return f.astype(np.float64)
    raise ValueError(dtype)


class CacheModel:
    """k, v: arrays [num_blocks][num_kv_heads][16 * D] of stored elements."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
                 fill=None, k_scale: float = 1.0, v_scale: float = 1.0):
        self.num_blocks, self.num_kv_heads, self.head_dim, self.dtype = (
            num_blocks, num_kv_heads, head_dim, dtype)
        self.k_scale, self.v_scale = k_scale, v_scale
        store = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]
        shape = (num_blocks, num_kv_heads, BLOCK_SIZE * head_dim)
        self.k = np.full(shape, 0 if fill is None else fill, dtype=store)
        self.v = np.full(shape, 0 if fill is None else fill, dtype=store)
        self.koff, self.voff = offset_tables(head_dim, fp8=(dtype == "fp8"))

    def write(self, k_new: np.ndarray, v_new: np.ndarray, slots: np.ndarray):
        """k_new, v_new [T][Hkv][D] stored values; slots int64 [T].  A slot
        outside [0, num_blocks * 16) is skipped (negative = padding)."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = (slots >= 0) & (slots < self.num_blocks * BLOCK_SIZE)
        idx = np.nonzero(keep)[0]
        blk = slots[idx] // BLOCK_SIZE
        t = slots[idx] % BLOCK_SIZE
        tile = BLOCK_SIZE * self.head_dim
        kf = self.k.reshape(-1)
        vf = self.v.reshape(-1)
        for h in range(self.num_kv_heads):
            # element (blk, h, off[t, d]) <- row i, head h, channel d
            base = (blk * self.num_kv_heads + h) * tile
            kf[base[:, None] + self.koff[t]] = k_new[idx, h, :]
            vf[base[:, None] + self.voff[t]] = v_new[idx, h, :]

    def copy_blocks(self, pairs):
        """Copy whole blocks (every head and slot, K and V), src -> dst, in order."""
        for src, dst in pairs:
            if 0 <= src < self.num_blocks and 0 <= dst < self.num_blocks:
                self.k[dst] = self.k[src]
                self.v[dst] = self.v[src]

    def gather(self, table_row, length: int, kv_head: int, start: int = 0):
        """K and V of tokens start..length-1 of one sequence and kv head, as
        float64 [length - start][D], read block by block through the table
        (entries before token start's block are not read)."""
        t = np.arange(start, length)
        blk = np.asarray(table_row, dtype=np.int64)[t // BLOCK_SIZE]
        slot = t % BLOCK_SIZE
        k = self.k[blk[:, None], kv_head, self.koff[slot]]
        v = self.v[blk[:, None], kv_head, self.voff[slot]]
        return widen(k, self.dtype, self.k_scale), widen(v, self.dtype, self.v_scale)

    def copy_blocks_to(self, other: "CacheModel", pairs):
        """Block swap: copy whole blocks of this cache into another cache of the
        same block shape (every head and slot, K and V), src -> dst."""
        for src, dst in pairs:
            other.k[dst] = self.k[src]
            other.v[dst] = self.v[src]

    def stored_bytes(self):
        return self.k.tobytes(), self.v.tobytes()
