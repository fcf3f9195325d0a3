"""Replays a synthetic workload on the oracle's pool, tables and cache.

The prefill recipe (the workload module documents it): an optional shared
prefix appended by sequence 0 and then shared by every other sequence
("PagedAttention por dentro", "Copy-on-write para sampling paralelo": the
sequences share the prefix's physical blocks through their tables), then
each sequence appends its own tokens.  The append step adds
``append_counts[b]`` tokens to sequence b; shared blocks about to be
written are copied first, then the new K/V are written.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import fp8
from .cache import CacheModel, widen
from .pool import PoolModel
from .slots import blocks_for, plan_append


@dataclass
class OracleState:
    pool: PoolModel
    tables: np.ndarray   # int32 [B][max_blocks]; unused entries -1
    lens: np.ndarray     # int32 [B]
    cache: CacheModel


def _rows(x, w, kv8, which):
    """Rows as the cache stores them: as given, or (FP8 cache) quantised from
    their float32 values with the tensor's scale."""
    if kv8 is None:
        return x
    return fp8.quantize(widen(x, w.spec.dtype).astype(np.float32), kv8[which])


def prefill(w, fill=None, kv8=None) -> OracleState:
    """kv8 = (k_scale, v_scale): the cache holds FP8 E4M3 codes of the
    workload's rows instead of the rows themselves."""
    s = w.spec
    B = s.num_seqs
    pool = PoolModel(w.num_blocks, 16, w.pool_order)
    tables = np.full((B, w.max_blocks_per_seq), -1, dtype=np.int32)
    lens = np.zeros(B, dtype=np.int32)
    if kv8 is None:
        cache = CacheModel(w.num_blocks, s.num_kv_heads, s.head_dim, s.dtype, fill)
    else:
        cache = CacheModel(w.num_blocks, s.num_kv_heads, s.head_dim, "fp8", fp8.NAN_CODE,
                           k_scale=kv8[0], v_scale=kv8[1])
    row = 0
    if s.prefix_len > 0:
        first = np.zeros(B, dtype=np.int64)
        first[0] = s.prefix_len
        slots, _, cows = plan_append(pool, tables, lens, first)
        assert not cows
        cache.write(_rows(w.k_rows[:s.prefix_len], w, kv8, 0),
                    _rows(w.v_rows[:s.prefix_len], w, kv8, 1), slots)
        row = s.prefix_len
        nb = blocks_for(s.prefix_len)
        for b in range(1, B):
            pool.share(tables[0, :nb])
            tables[b, :nb] = tables[0, :nb]
            lens[b] = s.prefix_len
    slots, _, cows = plan_append(pool, tables, lens, w.own_lens)
    cache.copy_blocks(cows)
    cache.write(_rows(w.k_rows[row:], w, kv8, 0), _rows(w.v_rows[row:], w, kv8, 1), slots)
    return OracleState(pool, tables, lens, cache)


def append_step(state: OracleState, w):
    """Appends w.append_counts tokens per sequence; returns (slots, updates, cows)."""
    slots, updates, cows = plan_append(state.pool, state.tables, state.lens, w.append_counts)
    state.cache.copy_blocks(cows)
    kv8 = (state.cache.k_scale, state.cache.v_scale) if state.cache.dtype == "fp8" else None
    state.cache.write(_rows(w.k_app, w, kv8, 0), _rows(w.v_app, w, kv8, 1), slots)
    return slots, updates, cows


def live_tables(state: OracleState):
    """Per sequence, the table entries that hold tokens."""
    return [list(state.tables[b, :blocks_for(int(state.lens[b]))]) for b in range(len(state.lens))]
