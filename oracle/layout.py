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
  FP8 tiles (one byte per element): the codes of lane l's bf16 piece j
  (8 channels or 2 x 4 tokens) form an 8-byte piece; pieces 2i and 2i + 1 of
  every lane make up bytes [1024 i, 1024 i + 1024) as 64 lanes x 16 bytes,
  and a last piece without a partner (D / 32 odd) takes 64 lanes x 8 bytes:
  piece(l, j) = 1024 * (j // 2) + (16 if paired else 8) * l + 8 * (j % 2)
  K byte (t, d): piece(16 * ((d // 8) % 4) + t, d // 32) + d % 8
  V byte (t, d): piece(16 * (t // 4) + d % 16, d // 32)
                 + ((d // 16) % 2) * 4 + t % 4
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


def k_offset(t: int, d: int) -> int:
    return (d // 8) * 128 + t * 8 + d % 8


def v_offset(t: int, d: int) -> int:
    return (d // 32) * 512 + (t // 4) * 128 + (d % 16) * 8 + ((d // 16) % 2) * 4 + t % 4


def _f8_piece(lane: int, piece: int, head_dim: int) -> int:
    paired = 2 * (piece // 2) + 1 < head_dim // 32
    return 1024 * (piece // 2) + (16 if paired else 8) * lane + 8 * (piece % 2)


def k8_offset(t: int, d: int, head_dim: int) -> int:
    return _f8_piece(16 * ((d // 8) % 4) + t, d // 32, head_dim) + d % 8


def v8_offset(t: int, d: int, head_dim: int) -> int:
    return _f8_piece(16 * (t // 4) + d % 16, d // 32, head_dim) + ((d // 16) % 2) * 4 + t % 4


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
