"""Host driver for one layer's paged KV cache on one GPU.

Holds the device cache tensors, the device-resident block tables and
lengths (with their host mirrors), the host pool and a decode workspace, and
sequences the C-ABI calls of one decode step:

  1. plan the appended tokens' slots on the host (paged_kv_append_slots);
  2. stage slots, table and length deltas and copy-on-write pairs in pinned
     host memory, which the kernels read in place;
  3. copy shared blocks that are about to be written (paged_kv_copy_blocks,
     only when there are such blocks);
  4. write the new K/V and apply the deltas (paged_kv_append, one launch;
     an FP8 cache: paged_block_table_update, then paged_kv_write_fp8);
  5. attend (paged_attention_decode).

decode_step does 4 and 5 in one launch (paged_kv_append_decode): the new
tokens are attended from their rows and stored at the end of the launch;
the device lengths alternate between two buffers, one read and one written
per step.

With a sliding window, blocks wholly before every upcoming query's window
are released before step 1 (pkv_window_release), so the same step can reuse
them.  A swap space in pinned host memory takes whole sequences out of the
device cache and brings them back (kv_block_swap + paged_kv_swap_blocks).

Every step runs in libpagedkv; this module only moves arguments.
"""
from __future__ import annotations

import time

import numpy as np
import torch

from . import _capi as capi

BLOCK = capi.BLOCK_SIZE


class _Staging:
    """A ring of pinned host buffers for each step's small inputs (slots,
    table and length deltas, block pairs).  The kernels read them in place
    over the host link (system-scope loads), so a step needs no copy launch
    and no second stream.  A buffer is refilled only once an event recorded
    behind its last reader has completed.  Recording an event puts a marker
    with a system-wide release between two kernels (several microseconds),
    so one event is recorded per ``every`` releases and covers all buffers
    released since the previous one (the stream runs in order)."""

    def __init__(self, nbytes: int, depth: int = 16, every: int = 8):
        assert 0 < every < depth
        self.bufs = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(depth)]
        # each buffer seen as int64 and int32 (pieces start at multiples of 8 bytes),
        # and as numpy bytes, made once
        self._typed = [{np.dtype(np.int64): b.view(torch.int64), np.dtype(np.int32): b.view(torch.int32)}
                       for b in self.bufs]
        self._host = [b.numpy() for b in self.bufs]
        self.events = [None] * depth
        self.every = every
        self.pending = []      # released buffers no event covers yet
        self.stream = None     # stream of the last release
        self.i = 0
        self.cur = None
        self.wait_s = 0.0      # host time spent waiting for a buffer's readers

    def _cover(self):
        ev = torch.cuda.Event()
        ev.record(self.stream)
        for k in self.pending:
            self.events[k] = ev
        self.pending = []

    def put(self, arrays):
        """Packs numpy arrays (8-byte aligned pieces) into the next pinned
        buffer and returns pinned tensor views of them; ``release`` must
        follow once their readers are enqueued."""
        k = self.i
        self.i = (k + 1) % len(self.bufs)
        if k in self.pending:
            self._cover()
        if self.events[k] is not None:
            t = time.perf_counter()
            self.events[k].synchronize()
            self.wait_s += time.perf_counter() - t
            self.events[k] = None
        host, typed = self._host[k], self._typed[k]
        views, off = [], 0
        for a in arrays:
            n = a.nbytes
            host[off:off + n] = np.ascontiguousarray(a).view(np.uint8).ravel()
            isz = a.dtype.itemsize
            t = typed[a.dtype][off // isz:(off + n) // isz]
            views.append(t.view(*a.shape) if a.ndim > 1 and a.size else t)
            off += (n + 7) & ~7
        self.cur = k
        return views

    def release(self, stream):
        """The last ``put`` buffer is free once ``stream`` passes this point."""
        if self.stream is not None and stream != self.stream and self.pending:
            self._cover()
        self.stream = stream
        self.pending.append(self.cur)
        if len(self.pending) >= self.every:
            self._cover()

    def drain(self):
        if self.pending:
            self._cover()
        for ev in self.events:
            if ev is not None:
                ev.synchronize()


class PagedKV:
    def __init__(self, *, num_blocks: int, num_seqs: int, max_blocks_per_seq: int,
                 num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                 device="cuda", init_order=None, fill=None, partition_size: int = 0,
                 k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0):
        """dtype "f32", "bf16" or "fp8" (E4M3 codes with tensor scales k_scale,
        v_scale; appended rows are bf16 or fp32 and quantised on write).
        window > 0: sliding-window attention over the last ``window`` tokens,
        with the blocks before it released as the sequences grow."""
        self.num_blocks, self.num_seqs, self.max_blocks = num_blocks, num_seqs, max_blocks_per_seq
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.dtype = dtype
        self.k_scale, self.v_scale = k_scale, v_scale
        self.device = torch.device(device)
        self.partition_size = partition_size
        self.pool = capi.pkv_pool_create(num_blocks, BLOCK, init_order)
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]
        n = num_blocks * num_kv_heads * BLOCK * head_dim
        self.k_cache = torch.empty(n, dtype=tdt, device=self.device)
        self.v_cache = torch.empty(n, dtype=tdt, device=self.device)
        if fill is None:
            self.k_cache.zero_()
            self.v_cache.zero_()
        elif dtype == "fp8":
            self.k_cache.fill_(0x7F)   # the NaN code
            self.v_cache.fill_(0x7F)
        else:
            self.k_cache.fill_(fill)
            self.v_cache.fill_(fill)
        self.tables = np.full((num_seqs, max_blocks_per_seq), -1, dtype=np.int32)
        self.lens = np.zeros(num_seqs, dtype=np.int32)
        # the slot planner, bound to these two arrays (changed only in place)
        self._plan = capi.AppendPlanner(self.pool, self.tables, self.lens)
        # device tables and lengths share one int32 buffer, so that a step's
        # length changes travel as table deltas at flat index S*mb + s; the
        # lengths have two copies, the current one and the one a fused step
        # (decode_step) writes
        nt = num_seqs * max_blocks_per_seq
        if nt + 2 * num_seqs >= 2 ** 31:
            raise ValueError("num_seqs * (max_blocks_per_seq + 2) must be < 2^31")
        self.state_d = torch.empty(nt + 2 * num_seqs, dtype=torch.int32, device=self.device)
        self.tables_d = self.state_d[:nt].view(num_seqs, max_blocks_per_seq)
        self._cur = 0
        self._lens_views = [self.state_d[nt + c * num_seqs:nt + (c + 1) * num_seqs] for c in (0, 1)]
        self.tables_d.copy_(torch.from_numpy(self.tables))
        self.lens_d.copy_(torch.from_numpy(self.lens))
        ws = capi.paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_blocks_per_seq * BLOCK, partition_size)
        self.workspace = torch.empty(max(ws // 4, 1), dtype=torch.float32, device=self.device)
        self._staging = None
        self.window = window
        self.host_pool = None
        self.swapped = {}   # sequence -> (host table row, length)

    @property
    def lens_d(self):
        """The device context lengths currently in use (int32 [num_seqs])."""
        return self._lens_views[self._cur]

    # ------------------------------------------------------------------ host helpers
    def _stage(self, arrays):
        need = sum((a.nbytes + 7) & ~7 for a in arrays) + 8
        if self._staging is None or self._staging.bufs[0].numel() < need:
            if self._staging is not None:
                self._staging.drain()  # pending kernels may still read the old ring
            self._staging = _Staging(max(need, 1 << 16))
        return self._staging.put(arrays)

    def share_prefix(self, src: int, dsts, num_blocks: int):
        """Sequences ``dsts`` take the first ``num_blocks`` blocks of ``src``
        by reference (refcount + 1 each) and the same length."""
        ids = self.tables[src, :num_blocks].copy()
        for d in dsts:
            capi.kv_block_share(self.pool, ids)
            self.tables[d, :num_blocks] = ids
            self.lens[d] = self.lens[src]
        self.tables_d.copy_(torch.from_numpy(self.tables))
        self.lens_d.copy_(torch.from_numpy(self.lens))

    # ------------------------------------------------------------------ a step
    def append(self, k_new, v_new, num_new=None, stream=None):
        """Appends tokens (k_new, v_new device [T][Hkv][D], rows in order of
        sequence) and returns (slots, table updates, cow pairs) as numpy."""
        stream = stream or torch.cuda.current_stream(self.device)
        nn = np.ones_like(self.lens) if num_new is None else np.asarray(num_new, np.int32)
        rel = None
        if self.window > 0:
            # the earliest query still to run sees context length lens + 1
            # (a sequence with nothing to append: its current length)
            ctx = self.lens + (nn > 0).astype(np.int32)
            rel = capi.pkv_window_release(self.pool, self.tables, ctx, self.window)
        slots, upd, cows = self._plan(num_new)
        if rel is not None and len(rel):
            upd = np.concatenate([rel, upd]) if len(upd) else rel
        # new lengths of the sequences that grew, as deltas into the state buffer
        grown = np.flatnonzero(nn)
        lupd = np.empty((len(grown), 2), dtype=np.int32)
        lupd[:, 0] = self.tables.size + self._cur * self.num_seqs + grown
        lupd[:, 1] = self.lens[grown]
        h_slots, h_upd, h_cows = self._stage([slots, np.concatenate([upd, lupd]), cows])
        s = stream.cuda_stream
        try:
            capi.paged_kv_copy_blocks(self.k_cache, self.v_cache, h_cows, self.num_kv_heads,
                                      self.head_dim, self.num_blocks, s)
            if self.dtype == "fp8":
                capi.paged_block_table_update(self.state_d, h_upd, s)
                capi.paged_kv_write_fp8(k_new, v_new, h_slots, self.k_cache, self.v_cache,
                                        self.num_kv_heads, self.head_dim, self.num_blocks,
                                        self.k_scale, self.v_scale, s)
            else:
                capi.paged_kv_append(k_new, v_new, h_slots, self.k_cache, self.v_cache,
                                     self.num_kv_heads, self.head_dim, self.num_blocks,
                                     self.state_d, h_upd, s)
        finally:
            self._staging.release(stream)
        return slots, upd, cows

    def decode_step(self, q, k_new, v_new, scale: float, out=None, stream=None):
        """One decode step in one launch (paged_kv_append_decode): every
        sequence with a context gains one token (row s of k_new / v_new,
        device [num_seqs][Hkv][D], bf16) and attends over its grown context.
        The host plans the slots and any copy-on-write first, as in append."""
        stream = stream or torch.cuda.current_stream(self.device)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        live = self.lens > 0
        nn = live.astype(np.int32)
        rel = None
        if self.window > 0:
            rel = capi.pkv_window_release(self.pool, self.tables, self.lens + nn, self.window)
        slots, upd, cows = self._plan(nn)
        if rel is not None and len(rel):
            upd = np.concatenate([rel, upd]) if len(upd) else rel
        slot_seq = np.full(self.num_seqs, -1, dtype=np.int64)
        slot_seq[live] = slots
        h_slots, h_upd, h_cows = self._stage([slot_seq, np.ascontiguousarray(upd, np.int32),
                                              np.ascontiguousarray(cows, np.int32)])
        s = stream.cuda_stream
        max_ctx = int(self.lens.max()) if self.lens.size else 0
        ws = self.workspace
        need = capi.paged_attention_workspace_size(self.num_seqs, self.num_q_heads,
                                                   self.num_kv_heads, self.head_dim, max_ctx, 0)
        if need > ws.numel() * 4:
            ws = self.workspace = torch.empty(need // 4, dtype=torch.float32, device=self.device)
        lens_in = self.lens_d
        self._cur ^= 1
        lens_out = self.lens_d
        try:
            capi.paged_kv_copy_blocks(self.k_cache, self.v_cache, h_cows, self.num_kv_heads,
                                      self.head_dim, self.num_blocks, s)
            capi.paged_kv_append_decode(q, k_new, v_new, h_slots, self.k_cache, self.v_cache,
                                        self.tables_d, lens_in, lens_out, h_upd, out,
                                        num_kv_heads=self.num_kv_heads, num_blocks=self.num_blocks,
                                        max_context_len=max_ctx, scale=scale, window=self.window,
                                        workspace=ws, stream=s)
        except Exception:
            self._cur ^= 1
            raise
        finally:
            self._staging.release(stream)
        return out

    def decode(self, q, scale: float, out=None, stream=None, partition_size=None):
        stream = stream or torch.cuda.current_stream(self.device)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        ps = self.partition_size if partition_size is None else partition_size
        max_ctx = int(self.lens.max()) if self.lens.size else 0
        ws = self.workspace
        need = capi.paged_attention_workspace_size(self.num_seqs, self.num_q_heads,
                                                   self.num_kv_heads, self.head_dim,
                                                   max_ctx, ps)
        if need > ws.numel() * 4:
            ws = self.workspace = torch.empty(need // 4, dtype=torch.float32, device=self.device)
        if self.window > 0:
            capi.paged_attention_decode_window(
                q, self.k_cache, self.v_cache, self.tables_d, self.lens_d, out,
                num_kv_heads=self.num_kv_heads, num_blocks=self.num_blocks,
                max_context_len=max_ctx, scale=scale, window=self.window,
                partition_size=0 if self.dtype == "fp8" else ps, k_scale=self.k_scale,
                v_scale=self.v_scale, workspace=ws, stream=stream.cuda_stream)
            return out
        if self.dtype == "fp8":
            capi.paged_attention_decode_fp8(q, self.k_cache, self.v_cache, self.tables_d,
                                            self.lens_d, out, num_kv_heads=self.num_kv_heads,
                                            num_blocks=self.num_blocks, max_context_len=max_ctx,
                                            scale=scale, k_scale=self.k_scale,
                                            v_scale=self.v_scale, workspace=ws,
                                            stream=stream.cuda_stream)
            return out
        capi.paged_attention_decode(q, self.k_cache, self.v_cache, self.tables_d, self.lens_d, out,
                                    num_kv_heads=self.num_kv_heads, num_blocks=self.num_blocks,
                                    max_context_len=max_ctx, scale=scale, partition_size=ps,
                                    workspace=ws, stream=stream.cuda_stream)
        return out

    def prefill_attention(self, q, query_start, scale: float, out=None, stream=None,
                          max_query_len=None):
        """Multi-query attention for chunk rows q [T][Hq][D] (their K/V already
        appended); query_start int32 [B + 1]: numpy (uploaded here), or a
        device tensor that stays resident (then max_query_len is required)."""
        stream = stream or torch.cuda.current_stream(self.device)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        if isinstance(query_start, torch.Tensor):
            if max_query_len is None:
                raise ValueError("max_query_len is required with a device query_start")
            qs_d, max_q = query_start, int(max_query_len)
        else:
            qs = np.ascontiguousarray(query_start, dtype=np.int32)
            qs_d = torch.from_numpy(qs).to(self.device)
            max_q = int(np.max(np.diff(qs))) if qs.size > 1 else 0
        max_ctx = int(self.lens.max()) if self.lens.size else 0
        if self.dtype == "fp8":
            capi.paged_attention_prefill_fp8(q, self.k_cache, self.v_cache, self.tables_d,
                                             self.lens_d, qs_d, out, num_kv_heads=self.num_kv_heads,
                                             num_blocks=self.num_blocks, max_context_len=max_ctx,
                                             max_query_len=max_q, scale=scale,
                                             k_scale=self.k_scale, v_scale=self.v_scale,
                                             window=self.window, stream=stream.cuda_stream)
            return out
        capi.paged_attention_prefill(q, self.k_cache, self.v_cache, self.tables_d, self.lens_d, qs_d,
                                     out, num_kv_heads=self.num_kv_heads, num_blocks=self.num_blocks,
                                     max_context_len=max_ctx, max_query_len=max_q, scale=scale,
                                     window=self.window, stream=stream.cuda_stream)
        return out

    # ------------------------------------------------------------------ prefix caching
    def enable_prefix_cache(self):
        capi.pkv_prefix_cache_enable(self.pool)

    def match_prefix(self, s: int, tokens) -> int:
        """Sequence s (empty) takes the cached blocks holding the longest
        indexed prefix of ``tokens``; returns the number of tokens covered."""
        assert self.lens[s] == 0
        ids = capi.pkv_prefix_match(self.pool, tokens, self.max_blocks)
        k = len(ids)
        if k:
            self.tables[s, :k] = ids
            self.lens[s] = k * BLOCK
            self.tables_d[s, :k] = torch.from_numpy(ids.astype(np.int32)).to(self.device)
            self.lens_d[s] = int(self.lens[s])
        return k * BLOCK

    def register_prefix(self, s: int, tokens):
        """Indexes the full blocks of sequence s, whose first tokens are ``tokens``."""
        n = min(len(tokens), int(self.lens[s]))
        full = n // BLOCK  # only full blocks are indexed
        capi.pkv_prefix_register(self.pool, np.asarray(tokens[:full * BLOCK], np.int32),
                                 self.tables[s, :full])

    # ------------------------------------------------------------------ swap
    def enable_swap(self, num_host_blocks: int):
        """A swap space of ``num_host_blocks`` blocks in pinned host memory."""
        self.host_pool = capi.pkv_pool_create(num_host_blocks, BLOCK)
        self.num_host_blocks = num_host_blocks
        n = num_host_blocks * self.num_kv_heads * BLOCK * self.head_dim
        self.k_host = torch.empty(n, dtype=self.k_cache.dtype, pin_memory=True)
        self.v_host = torch.empty(n, dtype=self.v_cache.dtype, pin_memory=True)

    def swap_out(self, seqs, stream=None):
        """Moves the blocks of sequences ``seqs`` to the swap space and frees
        their device blocks; the sequences leave the batch (length 0) until
        swap_in.  Blocks shared among ``seqs`` are moved once."""
        stream = stream or torch.cuda.current_stream(self.device)
        seqs = [int(s) for s in seqs]
        rows = [self.tables[s, :-(-int(self.lens[s]) // BLOCK)] for s in seqs]
        ids = np.concatenate([r[r >= 0] for r in rows]) if rows else np.zeros(0, np.int32)
        new, pairs = capi.kv_block_swap(self.pool, self.host_pool, ids)
        k = 0
        for s, r in zip(seqs, rows):
            h = np.full(self.max_blocks, -1, np.int32)
            live = np.nonzero(r >= 0)[0]
            h[live] = new[k:k + len(live)]
            k += len(live)
            self.swapped[s] = (h, int(self.lens[s]))
            self.tables[s, :] = -1
            self.lens[s] = 0
        self._swap_copy(pairs, self.k_cache, self.v_cache, self.num_blocks, self.k_host,
                        self.v_host, self.num_host_blocks, stream)
        self.tables_d.copy_(torch.from_numpy(self.tables), non_blocking=False)
        self.lens_d.copy_(torch.from_numpy(self.lens), non_blocking=False)
        return pairs

    def swap_in(self, seqs, stream=None):
        """Brings swapped-out sequences back into fresh device blocks."""
        stream = stream or torch.cuda.current_stream(self.device)
        seqs = [int(s) for s in seqs]
        rows = [self.swapped[s][0] for s in seqs]
        ids = np.concatenate([r[r >= 0] for r in rows]) if rows else np.zeros(0, np.int32)
        new, pairs = capi.kv_block_swap(self.host_pool, self.pool, ids)
        k = 0
        for s, r in zip(seqs, rows):
            live = np.nonzero(r >= 0)[0]
            self.tables[s, :] = -1
            self.tables[s, live] = new[k:k + len(live)]
            k += len(live)
            self.lens[s] = self.swapped.pop(s)[1]
        self._swap_copy(pairs, self.k_host, self.v_host, self.num_host_blocks, self.k_cache,
                        self.v_cache, self.num_blocks, stream)
        self.tables_d.copy_(torch.from_numpy(self.tables), non_blocking=False)
        self.lens_d.copy_(torch.from_numpy(self.lens), non_blocking=False)
        return pairs

    def _swap_copy(self, pairs, sk, sv, snb, dk, dv, dnb, stream):
        if len(pairs) == 0:
            return
        (h_pairs,) = self._stage([np.ascontiguousarray(pairs, np.int32)])
        try:
            capi.paged_kv_swap_blocks(sk, sv, dk, dv, h_pairs, self.num_kv_heads, self.head_dim,
                                      snb, dnb, stream.cuda_stream)
        finally:
            self._staging.release(stream)

    def free_sequence(self, s: int):
        """Returns sequence s's blocks to the pool (one reference each)."""
        n = -(-int(self.lens[s]) // BLOCK)
        row = self.tables[s, :n]
        capi.kv_block_free(self.pool, row[row >= 0])
        self.tables[s, :] = -1
        self.lens[s] = 0
        self.tables_d[s].fill_(-1)
        self.lens_d[s] = 0


def replay_prefill(kv: PagedKV, w, to_device):
    """Builds the prefill state of a synthetic workload ``w`` (attributes as
    in workloads.synth.Workload): optional shared prefix appended by sequence
    0 and shared by the others, then every sequence's own tokens.
    ``to_device`` turns a host row array into a device tensor of the cache
    dtype."""
    s = w.spec
    row = 0
    if s.prefix_len > 0:
        first = np.zeros(s.num_seqs, dtype=np.int32)
        first[0] = s.prefix_len
        kv.append(to_device(w.k_rows[:s.prefix_len]), to_device(w.v_rows[:s.prefix_len]), first)
        row = s.prefix_len
        kv.share_prefix(0, range(1, s.num_seqs), -(-s.prefix_len // BLOCK))
    if int(w.own_lens.sum()) > 0:
        kv.append(to_device(w.k_rows[row:]), to_device(w.v_rows[row:]), w.own_lens)
