"""Seeded synthetic workloads for paged decode attention.

Five workloads follow the shapes of the decode step described on the pages
(one query token per sequence attending over a block-paged context):

  tiny-fp32        4 sequences, lengths {17,33,64,100}, 4 q heads = 4 kv heads,
                   head_dim 64, fp32, a pool of 64 blocks
  mha-7b-bf16      64 sequences, 32 q heads = 32 kv heads, head_dim 128,
                   lengths uniform in [128, 4096]
  gqa-8b-bf16      256 sequences, 32 q heads / 8 kv heads, head_dim 128,
                   lengths log-normal (median 1000, sigma 1), clipped to
                   [16, 8192], sequence 0 fixed at 273 tokens
  long-70b-bf16    8 sequences of 32768 tokens, 64 q heads / 8 kv heads
  shared-prefix    128 sequences sharing a 2048-token prefix (128 blocks),
                   each followed by 0..512 own tokens
  shared-prefix-cow  the same, but the shared prefix is 2040 tokens so its
                   last block is only half full; the append step then adds
                   s_b + 1 tokens per sequence, which forces copy-on-write
  gqa-8b-bf16-b512 the gqa-8b shape and length law with 512 sequences

Draw order (fixed): one numpy PCG64 generator seeded 1000 + workload number
draws the lengths, the own-suffix lengths, the pool permutation and Q, in
that order.  The bulk rows (K rows, V rows, appended K rows, appended V rows:
tags 1, 2, 3, 4) are drawn in chunks of 4096 rows, chunk c of tag k from
PCG64(SeedSequence([seed, k, c])), so chunks can be drawn in parallel and
the result does not depend on the number of threads.  Values are N(0, 1)
float32; bf16 workloads round them to bf16 (round to nearest even) and keep
the raw 16-bit patterns.

Prefill recipe that both sides replay with their own allocator:
  1. if ``prefix_len > 0``: sequence 0 appends ``prefix_len`` tokens, and
     every other sequence takes the same physical blocks by sharing them;
  2. each sequence b then appends ``own_lens[b]`` tokens, in order of b.
Token rows in ``k_rows``/``v_rows`` are in exactly this append order.  The
decode-step append then adds ``append_counts[b]`` tokens to sequence b,
rows in ``k_app``/``v_app`` in order of b.

The pool's free list starts in the order ``pool_order`` (a seeded
permutation), so blocks end up scattered over the pool.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16


@dataclass(frozen=True)
class WorkloadSpec:
    key: str
    number: int          # seed = 1000 + number
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str           # "f32" or "bf16"
    lengths: str         # "fixed" | "uniform" | "lognormal" | "shared"
    fixed_lens: tuple = ()
    uniform_range: tuple = ()
    lognormal: tuple = ()      # (median, sigma, lo, hi)
    pinned: tuple = ()         # ((index, length), ...)
    prefix_len: int = 0
    suffix_range: tuple = ()
    cow_append: bool = False   # append s_b + 1 tokens after a shared prefix
    fixed_pool: int = 0        # explicit pool size (0: 1.25x the need)
    partition_tokens: int = 512

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


SPECS = {
    "tiny-fp32": WorkloadSpec("tiny-fp32", 1, 4, 4, 4, 64, "f32", "fixed",
                              fixed_lens=(17, 33, 64, 100), fixed_pool=64),
    "mha-7b-bf16": WorkloadSpec("mha-7b-bf16", 2, 64, 32, 32, 128, "bf16", "uniform",
                                uniform_range=(128, 4096)),
    "gqa-8b-bf16": WorkloadSpec("gqa-8b-bf16", 3, 256, 32, 8, 128, "bf16", "lognormal",
                                lognormal=(1000.0, 1.0, 16, 8192), pinned=((0, 273),)),
    "long-70b-bf16": WorkloadSpec("long-70b-bf16", 4, 8, 64, 8, 128, "bf16", "fixed",
                                  fixed_lens=(32768,) * 8),
    "shared-prefix-bf16": WorkloadSpec("shared-prefix-bf16", 5, 128, 32, 8, 128, "bf16", "shared",
                                       prefix_len=2048, suffix_range=(0, 512)),
    "shared-prefix-cow-bf16": WorkloadSpec("shared-prefix-cow-bf16", 5, 128, 32, 8, 128, "bf16",
                                           "shared", prefix_len=2040, suffix_range=(0, 512),
                                           cow_append=True),
    # the gqa-8b shape with twice the batch (a larger serving step)
    "gqa-8b-bf16-b512": WorkloadSpec("gqa-8b-bf16-b512", 13, 512, 32, 8, 128, "bf16",
                                     "lognormal", lognormal=(1000.0, 1.0, 16, 8192),
                                     pinned=((0, 273),)),
}


def spec(key: str) -> WorkloadSpec:
    return SPECS[key]


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite normal draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the float32 values they encode (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    spec: WorkloadSpec
    lens: np.ndarray            # int32 [B], context length after prefill
    own_lens: np.ndarray        # int32 [B], tokens each sequence appends itself in prefill
    suffix_lens: np.ndarray     # int32 [B] (shared workloads; zeros otherwise)
    append_counts: np.ndarray   # int32 [B], tokens appended by the decode-step append
    num_blocks: int
    max_blocks_per_seq: int
    pool_order: np.ndarray      # int32 [num_blocks], initial free-list order
    q: np.ndarray | None        # [B][Hq][D] (uint16 bf16 bits or float32)
    k_rows: np.ndarray | None   # [T][Hkv][D]
    v_rows: np.ndarray | None
    k_app: np.ndarray | None    # [sum(append_counts)][Hkv][D]
    v_app: np.ndarray | None
    extra_tokens: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def prefix_len(self) -> int:
        return self.spec.prefix_len

    @property
    def total_rows(self) -> int:
        return int(self.prefix_len + self.own_lens.sum())

    @property
    def final_lens(self) -> np.ndarray:
        return (self.lens + self.append_counts).astype(np.int32)


def _ceil_div(a, b):
    return -(-a // b)


def _draw_values(rng: np.random.Generator, shape, dtype: str, chunk_rows: int = 1 << 14):
    """N(0,1) float32 draws from ``rng``, stored as float32 or bf16 bits,
    drawn row-chunk by row-chunk (same stream as one draw of the array)."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    flat = out.reshape(rows, inner)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0) * inner, dtype=np.float32).reshape(r1 - r0, inner)
        flat[r0:r1] = x if dtype == "f32" else round_bf16_bits(x)
    return out


BULK_CHUNK = 4096


def _draw_rows(seed: int, tag: int, shape, dtype: str, threads: int | None = None):
    """Bulk rows: chunk c of BULK_CHUNK rows from PCG64(SeedSequence([seed,
    tag, c])); chunks are independent, so they are drawn on a thread pool."""
    from concurrent.futures import ThreadPoolExecutor
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    flat = out.reshape(rows, inner)

    def fill(c):
        r0, r1 = c * BULK_CHUNK, min(rows, (c + 1) * BULK_CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, c])))
        x = g.standard_normal((r1 - r0) * inner, dtype=np.float32).reshape(r1 - r0, inner)
        flat[r0:r1] = x if dtype == "f32" else round_bf16_bits(x)

    nchunks = -(-rows // BULK_CHUNK)
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if nchunks <= 1 or threads <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def generate(key: str, *, values: bool = True, extra_tokens: int = 0) -> Workload:
    """Build the seeded workload ``key``.

    ``values=False`` skips drawing Q/K/V (shapes and tables only).
    ``extra_tokens`` reserves pool and table room for that many further
    single-token appends per sequence (used when benchmarking many steps)."""
    s = SPECS[key]
    rng = np.random.Generator(np.random.PCG64(s.seed))
    B = s.num_seqs
    # 1. lengths
    if s.lengths == "fixed":
        lens = np.array(s.fixed_lens, dtype=np.int64)
    elif s.lengths == "uniform":
        lo, hi = s.uniform_range
        lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    elif s.lengths == "lognormal":
        med, sigma, lo, hi = s.lognormal
        z = rng.standard_normal(B)
        lens = np.clip(np.rint(np.exp(np.log(med) + sigma * z)), lo, hi).astype(np.int64)
    elif s.lengths == "shared":
        lens = np.full(B, s.prefix_len, dtype=np.int64)
    else:
        raise ValueError(s.lengths)
    for idx, val in s.pinned:
        lens[idx] = val
    # 2. own suffix lengths (shared-prefix workloads)
    if s.lengths == "shared":
        lo, hi = s.suffix_range
        suffix = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    else:
        suffix = np.zeros(B, dtype=np.int64)
    if s.lengths == "shared":
        if s.cow_append:
            own = np.zeros(B, dtype=np.int64)
            append = suffix + 1
        else:
            own = suffix.copy()
            lens = lens + suffix
            append = np.ones(B, dtype=np.int64)
        # sequence 0's own appends come after the shared prefix
    else:
        own = lens.copy()
        append = np.ones(B, dtype=np.int64)
    # pool size: 1.25x the blocks needed through the append step (+ bench room)
    grow = append + extra_tokens
    if s.fixed_pool:
        nb = s.fixed_pool
    elif s.lengths == "shared":
        full_prefix = s.prefix_len // BLOCK_SIZE
        need = _ceil_div(s.prefix_len, BLOCK_SIZE) + int(
            np.sum(_ceil_div(lens + grow, BLOCK_SIZE) - full_prefix))
        nb = int(math.ceil(1.25 * need))
    else:
        need = int(np.sum(_ceil_div(lens + grow, BLOCK_SIZE)))
        nb = int(math.ceil(1.25 * need))
    max_blocks = int(np.max(_ceil_div(lens + grow, BLOCK_SIZE)))
    # 3. pool permutation
    order = rng.permutation(nb).astype(np.int32)
    total_rows = int(s.prefix_len + own.sum()) if s.lengths == "shared" else int(own.sum())
    q = k_rows = v_rows = k_app = v_app = None
    if values:
        H, Hkv, D = s.num_q_heads, s.num_kv_heads, s.head_dim
        q = _draw_values(rng, (B, H, D), s.dtype)                      # 4. Q
        k_rows = _draw_rows(s.seed, 1, (total_rows, Hkv, D), s.dtype)   # 5. K rows
        v_rows = _draw_rows(s.seed, 2, (total_rows, Hkv, D), s.dtype)   # 6. V rows
        n_app = int(append.sum())
        k_app = _draw_rows(s.seed, 3, (n_app, Hkv, D), s.dtype)         # 7. appended K, V
        v_app = _draw_rows(s.seed, 4, (n_app, Hkv, D), s.dtype)
    return Workload(spec=s, lens=lens.astype(np.int32), own_lens=own.astype(np.int32),
                    suffix_lens=suffix.astype(np.int32), append_counts=append.astype(np.int32),
                    num_blocks=nb, max_blocks_per_seq=max_blocks, pool_order=order,
                    q=q, k_rows=k_rows, v_rows=v_rows, k_app=k_app, v_app=v_app,
                    extra_tokens=extra_tokens)


def small_random(seed: int, *, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, dtype: str, max_len: int, num_blocks: int | None = None,
                 min_len: int = 0, append: int = 1, fixed=None) -> Workload:
    """A small random workload for edge-case tests (not one of the named ones).

    Lengths uniform in [min_len, max_len], the first ones replaced by
    ``fixed`` if given; the pool holds 1.25x the need."""
    s = WorkloadSpec(f"random-{seed}", 0, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     dtype, "fixed")
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(min_len, max_len, size=num_seqs, endpoint=True).astype(np.int64)
    if fixed is not None:
        lens[:len(fixed)] = fixed
    append_c = np.full(num_seqs, append, dtype=np.int64)
    need = int(np.sum(_ceil_div(lens + append_c, BLOCK_SIZE)))
    nb = num_blocks if num_blocks is not None else max(1, int(math.ceil(1.25 * need)))
    max_blocks = max(1, int(np.max(_ceil_div(lens + append_c, BLOCK_SIZE))))
    order = rng.permutation(nb).astype(np.int32)
    q = _draw_values(rng, (num_seqs, num_q_heads, head_dim), dtype)
    T = int(lens.sum())
    k_rows = _draw_rows(seed, 1, (T, num_kv_heads, head_dim), dtype)
    v_rows = _draw_rows(seed, 2, (T, num_kv_heads, head_dim), dtype)
    n_app = int(append_c.sum())
    k_app = _draw_rows(seed, 3, (n_app, num_kv_heads, head_dim), dtype)
    v_app = _draw_rows(seed, 4, (n_app, num_kv_heads, head_dim), dtype)
    return Workload(spec=s, lens=lens.astype(np.int32), own_lens=lens.astype(np.int32),
                    suffix_lens=np.zeros(num_seqs, np.int32), append_counts=append_c.astype(np.int32),
                    num_blocks=nb, max_blocks_per_seq=max_blocks, pool_order=order,
                    q=q, k_rows=k_rows, v_rows=v_rows, k_app=k_app, v_app=v_app)


def subset(w: Workload, seqs, seed: int = 0) -> Workload:
    """The sequences ``seqs`` of workload ``w`` as a workload of their own
    (a bounded sample with the same lengths, prefix sharing and values): the
    rows of each chosen sequence in the same append order, a pool of 1.25x
    their need (shared prefix blocks counted once), drawn in a seeded order.
    Used to time a fixed share of a large workload on the CPU."""
    s = w.spec
    idx = np.asarray(sorted(int(b) for b in seqs), dtype=np.int64)
    sub = WorkloadSpec(f"{s.key}[{len(idx)} of {s.num_seqs}]", s.number, len(idx), s.num_q_heads,
                       s.num_kv_heads, s.head_dim, s.dtype, s.lengths, s.fixed_lens,
                       s.uniform_range, s.lognormal, (), s.prefix_len, s.suffix_range,
                       s.cow_append, 0, s.partition_tokens)
    own = w.own_lens.astype(np.int64)
    starts = s.prefix_len + np.concatenate([[0], np.cumsum(own)[:-1]])
    rows = [np.arange(s.prefix_len)] if s.prefix_len else []
    rows += [np.arange(starts[b], starts[b] + own[b]) for b in idx]
    rows = np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)
    app = w.append_counts.astype(np.int64)
    app_starts = np.concatenate([[0], np.cumsum(app)[:-1]])
    app_rows = np.concatenate([np.arange(app_starts[b], app_starts[b] + app[b]) for b in idx])
    lens = w.lens[idx].astype(np.int64)
    grow = app[idx] + w.extra_tokens
    if s.prefix_len:
        full_prefix = s.prefix_len // BLOCK_SIZE
        need = _ceil_div(s.prefix_len, BLOCK_SIZE) + int(
            np.sum(_ceil_div(lens + grow, BLOCK_SIZE) - full_prefix))
    else:
        need = int(np.sum(_ceil_div(lens + grow, BLOCK_SIZE)))
    nb = max(1, int(math.ceil(1.25 * need)))
    order = np.random.Generator(np.random.PCG64(seed)).permutation(nb).astype(np.int32)
    pick = lambda a, r: None if a is None else a[r]
    return Workload(spec=sub, lens=w.lens[idx].copy(), own_lens=w.own_lens[idx].copy(),
                    suffix_lens=w.suffix_lens[idx].copy(),
                    append_counts=w.append_counts[idx].copy(), num_blocks=nb,
                    max_blocks_per_seq=int(np.max(_ceil_div(lens + grow, BLOCK_SIZE))),
                    pool_order=order, q=pick(w.q, idx), k_rows=pick(w.k_rows, rows),
                    v_rows=pick(w.v_rows, rows), k_app=pick(w.k_app, app_rows),
                    v_app=pick(w.v_app, app_rows), extra_tokens=w.extra_tokens)
