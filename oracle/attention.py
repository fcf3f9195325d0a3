"""Decode attention, by its definition, in float64.

"Como funciona realmente vLLM" (alexanderzelada.com), "Que es el mecanismo
de atencion": the current token's query is compared with the keys of the
previous tokens, a softmax turns the affinities into weights that add up to
100 %, and the output is the weighted sum of the value vectors.  "KV cache:
la memoria de trabajo ...", "El mecanismo en si": to predict token N only
the new Q and the cached K, V of the earlier tokens are needed.  "Trucos
para que el cuaderno sea mas fino": with grouped-query attention the query
heads share K, V in groups (Llama 3 8B: 32 query heads in groups of 4).
"PagedAttention: ..." (same lesson): paging changes how the cache is
addressed, not the mathematics of attention.

Readings where the pages are silent: the softmax is scaled by ``scale``
(1/sqrt(head_dim) in every workload) and stabilised by subtracting the
maximum (equal in exact arithmetic); query head h uses kv head
h // (num_q_heads // num_kv_heads); there is no mask beyond the context
length and no positional term; an empty context gives a zero row.  With an
FP8 cache the queries are bf16 and K, V are the codes' values times their
tensor scales (see ``fp8``).
"""
from __future__ import annotations

import numpy as np

from .cache import CacheModel, widen


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One query vector q [D] over keys k [L][D] and values v [L][D], float64."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64)
    s = scale * (k @ q)
    e = np.exp(s - s.max())
    w = e / e.sum()
    return w @ v


def window_start(p: int, window: int) -> int:
    """First position seen by the query at position p.

    "PagedAttention por dentro" (blog.lo0.es), "Sliding window attention"
    (under "Lo que vLLM hace hoy"): models such as Mistral 7B attend only to
    the most recent W tokens (W = 4096 there).  Reading: the W most recent
    positions including the query's own, p - W + 1 .. p; window 0 means no
    window (the whole prefix 0 .. p)."""
    return max(0, p - window + 1) if window > 0 else 0


def decode(q_stored: np.ndarray, cache: CacheModel, tables: np.ndarray, lens: np.ndarray,
           num_q_heads: int, num_kv_heads: int, scale: float, seqs=None,
           window: int = 0) -> np.ndarray:
    """out [B][Hq][D] float64 for the sequences in ``seqs`` (default all;
    rows of other sequences stay zero).  Each sequence's K/V are gathered
    block by block through its table; with a sliding window only positions
    window_start(L - 1, window) .. L - 1 are gathered (table entries before
    that block are never looked at)."""
    B = q_stored.shape[0]
    D = q_stored.shape[2]
    group = num_q_heads // num_kv_heads
    q = widen(q_stored, "bf16" if cache.dtype == "fp8" else cache.dtype)
    out = np.zeros((B, num_q_heads, D), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(lens[b])
        lo = window_start(L - 1, window) if L > 0 else 0
        for kvh in range(num_kv_heads):
            k, v = cache.gather(tables[b], L, kvh, start=lo)
            for h in range(kvh * group, (kvh + 1) * group):
                out[b, h] = attend(q[b, h], k, v, scale)
    return out


def partial_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Partial softmax state of one chunk of tokens: (m, l, o) with
    m = max score, l = sum exp(score - m), o = sum exp(score - m) * v."""
    s = scale * (k @ q)
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ v


def merge_states(states):
    """Log-sum-exp merge of partial states into the normalised output:
    m = max m_p, l = sum l_p e^(m_p - m), out = sum o_p e^(m_p - m) / l."""
    m = max(st[0] for st in states)
    l = sum(st[1] * np.exp(st[0] - m) for st in states)
    o = sum(st[2] * np.exp(st[0] - m) for st in states)
    return o / l


def attend_partitioned(q, k, v, scale, partition_tokens: int) -> np.ndarray:
    """Same result as ``attend`` computed as independent partitions of
    ``partition_tokens`` tokens merged by ``merge_states``."""
    L = k.shape[0]
    if L == 0:
        return np.zeros(v.shape[1], dtype=np.float64)
    states = [partial_state(q, k[a:a + partition_tokens], v[a:a + partition_tokens], scale)
              for a in range(0, L, partition_tokens)]
    return merge_states(states)


def prefill(q_stored: np.ndarray, cache: CacheModel, tables: np.ndarray, lens: np.ndarray,
            query_start: np.ndarray, num_q_heads: int, num_kv_heads: int,
            scale: float, window: int = 0) -> np.ndarray:
    """Multi-query attention over the paged cache (chunked prefill).

    "PagedAttention por dentro" (blog.lo0.es), "Chunked prefill integrado con
    paged KV": prefill split into chunks runs in the same step as decode, on
    the same paged cache.  Reading (the page gives no formula): sequence b's
    chunk holds rows query_start[b] .. query_start[b+1]-1 of ``q_stored``
    [T][Hq][D]; they are the last n_b of its L_b cached tokens, so chunk row
    i is the token at position p = L_b - n_b + i and attends to positions
    0..p only (the causal rule of a language model, applied inside the
    chunk).  With a sliding window the row sees window_start(p, window) ..
    p.  With n_b = 1 this is ``decode``.  Returns out [T][Hq][D] float64."""
    T, _, D = q_stored.shape
    group = num_q_heads // num_kv_heads
    q = widen(q_stored, "bf16" if cache.dtype == "fp8" else cache.dtype)
    out = np.zeros((T, num_q_heads, D), dtype=np.float64)
    for b in range(len(lens)):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        n, L = r1 - r0, int(lens[b])
        if n == 0:
            continue
        first = window_start(L - n, window)  # the earliest position any row sees
        for kvh in range(num_kv_heads):
            k, v = cache.gather(tables[b], L, kvh, start=first)
            for i in range(n):
                p = L - n + i
                lo = window_start(p, window) - first
                for h in range(kvh * group, (kvh + 1) * group):
                    out[r0 + i, h] = attend(q[r0 + i, h], k[lo:p + 1 - first],
                                            v[lo:p + 1 - first], scale)
    return out
