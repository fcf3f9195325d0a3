"""Element order inside one (block, kv head) tile of the cache.

The pages say only that a block holds the K and V of 16 consecutive tokens
of one sequence in one layer ("PagedAttention por dentro", "El modelo de
bloques"); the order of elements inside a block is this library's choice
and is fixed by the C ABI header (include/pagedkv.h, "Cache layout").
Written here again, independently, from that definition:

  tile (block b, kv head h) starts at element (b * Hkv + h) * 16 * D
  K element (t, d): (d // 8) * 128 + t * 8 + d % 8
  V element (t, d): (d // 32) * 512 + (t // 4) * 128 + (d % 16) * 8
                    + ((d // 16) % 2) * 4 + t % 4
  FP8 tiles (one byte per element), with W = D / 4 bytes per lane:
  K byte (t, d): W * (16 * ((d // 8) % 4) + t) + 8 * (d // 32) + d % 8
  V byte (t, d): W * (16 * (t // 4) + d % 16) + 8 * (d // 32)
                 + ((d // 16) % 2) * 4 + t % 4
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


def k_offset(t: int, d: int) -> int:
    return (d // 8) * 128 + t * 8 + d % 8


def v_offset(t: int, d: int) -> int:
    return (d // 32) * 512 + (t // 4) * 128 + (d % 16) * 8 + ((d // 16) % 2) * 4 + t % 4


def k8_offset(t: int, d: int, head_dim: int) -> int:
    w = head_dim // 4
    return w * (16 * ((d // 8) % 4) + t) + 8 * (d // 32) + d % 8


def v8_offset(t: int, d: int, head_dim: int) -> int:
    w = head_dim // 4
    return w * (16 * (t // 4) + d % 16) + 8 * (d // 32) + ((d // 16) % 2) * 4 + t % 4


def tile_base(block: int, kv_head: int, num_kv_heads: int, head_dim: int) -> int:
    return (block * num_kv_heads + kv_head) * BLOCK_SIZE * head_dim


def offset_tables(head_dim: int, fp8: bool = False):
    """(K, V) int64 arrays [16][D] of in-tile offsets, from the scalar rules."""
    if head_dim % 32:
        raise ValueError("head_dim must be a multiple of 32")
    if fp8:
        kt = np.array([[k8_offset(t, d, head_dim) for d in range(head_dim)]
                       for t in range(BLOCK_SIZE)], dtype=np.int64)
        vt = np.array([[v8_offset(t, d, head_dim) for d in range(head_dim)]
                       for t in range(BLOCK_SIZE)], dtype=np.int64)
        return kt, vt
    kt = np.array([[k_offset(t, d) for d in range(head_dim)] for t in range(BLOCK_SIZE)],
                  dtype=np.int64)
    vt = np.array([[v_offset(t, d) for d in range(head_dim)] for t in range(BLOCK_SIZE)],
                  dtype=np.int64)
    return kt, vt
