"""Plants plausible mistakes in the oracle (on the CPU, by monkeypatching)
and checks that at least one pin in test_oracle_pins fails for each."""
import math

import numpy as np
import pytest

from oracle import attention, layout, pool, slots
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, Exception):
        return True
    return False


def test_mutation_gqa_head_map(monkeypatch):
    def bad_decode(q_stored, cache, tables, lens, num_q_heads, num_kv_heads, scale, seqs=None):
        B, D = q_stored.shape[0], q_stored.shape[2]
        q = attention.widen(q_stored, cache.dtype)
        out = np.zeros((B, num_q_heads, D))
        for b in range(B):
            for h in range(num_q_heads):
                k, v = cache.gather(tables[b], int(lens[b]), h % num_kv_heads)   # wrong map
                out[b, h] = attention.attend(q[b, h], k, v, scale)
        return out
    monkeypatch.setattr(attention, "decode", bad_decode)
    assert _fails(pins.test_paged_equals_contiguous_sdpa, 8, 2, "f32")


def test_mutation_dropped_scale(monkeypatch):
    orig = attention.attend
    monkeypatch.setattr(attention, "attend", lambda q, k, v, scale: orig(q, k, v, 1.0))
    assert _fails(pins.test_paged_equals_contiguous_sdpa, 4, 4, "f32")
    assert _fails(pins.test_closed_forms)


def test_mutation_unnormalised_weights(monkeypatch):
    def bad(q, k, v, scale):
        if k.shape[0] == 0:
            return np.zeros(v.shape[1])
        s = scale * (k @ q)
        return np.exp(s - s.max()) @ v
    monkeypatch.setattr(attention, "attend", bad)
    assert _fails(pins.test_closed_forms)


def test_mutation_lse_merge(monkeypatch):
    def bad_merge(states):
        m = max(st[0] for st in states)
        l = sum(st[1] * np.exp(st[0] - m) for st in states)
        o = sum(st[2] for st in states)                # forgot the rescale
        return o / l
    monkeypatch.setattr(attention, "merge_states", bad_merge)
    assert _fails(pins.test_partitioned_lse_equals_single_pass, 2000, 512)


def test_mutation_layout_transposed(monkeypatch):
    monkeypatch.setattr(layout, "k_offset", lambda t, d: t * 128 + d)
    assert _fails(pins.test_layout_golden_offsets)


def test_mutation_layout_v_swapped_halves(monkeypatch):
    monkeypatch.setattr(layout, "v_offset", lambda t, d: (d // 32) * 512 + (t // 4) * 128
                        + (d % 16) * 8 + ((d // 16) % 2) + (t % 4) * 2)
    assert _fails(pins.test_layout_golden_offsets)


def test_mutation_slot_off_by_one(monkeypatch):
    monkeypatch.setattr(slots, "slot_of", lambda row, p: int(row[p // 16]) * 16 + (p + 1) % 16)
    assert _fails(pins.test_token_200_position_12)


def test_mutation_alloc_on_wrong_boundary(monkeypatch):
    orig = slots.plan_append

    def bad_plan(pool_, tables, lens, num_new=None):
        # allocates one token late: p % 16 == 1 instead of 0
        lens[...] = lens - 0
        B = tables.shape[0]
        num_new = np.ones(B, np.int64) if num_new is None else num_new
        out = []
        for s in range(B):
            for _ in range(int(num_new[s])):
                p = int(lens[s])
                if p % 16 == 1 or p == 0:
                    (blk,) = pool_.alloc(1)
                    tables[s, (p + 15) // 16 if p else 0] = blk
                out.append(0)
                lens[s] = p + 1
        return np.array(out), [], []
    monkeypatch.setattr(slots, "plan_append", bad_plan)
    assert _fails(pins.test_session_273_blocks)
    monkeypatch.setattr(slots, "plan_append", orig)


def test_mutation_fifo_free_list(monkeypatch):
    orig_free = pool.PoolModel.free

    def fifo_free(self, ids):
        orig_free(self, ids)
        # move freed ids to the bottom of the stack (FIFO reuse)
        freed = [i for i in ids if self.refcount[i] == 0]
        self._free = freed + [i for i in self._free if i not in freed]
    monkeypatch.setattr(pool.PoolModel, "free", fifo_free)
    assert _fails(pins.test_figure_pool_and_reuse)


def test_mutation_cow_copies_always(monkeypatch):
    def bad_cow(self, i):
        self._check_live(i)
        new = self._free.pop()
        self.refcount[new] = 1
        self.refcount[i] -= 1
        return new, True
    monkeypatch.setattr(pool.PoolModel, "cow", bad_cow)
    assert _fails(pins.test_cow_beam_fork)


@pytest.mark.parametrize("shift", [-1, 1])
def test_mutation_prefill_causal_off_by_one(monkeypatch, shift):
    """A causal limit one position early or late is caught."""
    def bad_prefill(q_stored, cache, tables, lens, query_start, num_q_heads, num_kv_heads, scale):
        T, _, D = q_stored.shape
        g = num_q_heads // num_kv_heads
        q = attention.widen(q_stored, cache.dtype)
        out = np.zeros((T, num_q_heads, D))
        for b in range(len(lens)):
            r0, r1 = int(query_start[b]), int(query_start[b + 1])
            n, L = r1 - r0, int(lens[b])
            for kvh in range(num_kv_heads):
                k, v = cache.gather(tables[b], L, kvh)
                for i in range(n):
                    p = max(0, min(L - 1, L - n + i + shift))
                    for h in range(kvh * g, (kvh + 1) * g):
                        out[r0 + i, h] = attention.attend(q[r0 + i, h], k[:p + 1], v[:p + 1], scale)
        return out
    monkeypatch.setattr(attention, "prefill", bad_prefill)
    assert _fails(pins.test_prefill_equals_causal_sdpa, 8, 2, "f32")


def test_mutation_prefill_query_rows(monkeypatch):
    """Chunk rows read as the first n positions (not the last n) is caught."""
    orig = attention.prefill

    def bad_prefill(q_stored, cache, tables, lens, query_start, num_q_heads, num_kv_heads, scale):
        n = np.diff(np.asarray(query_start))
        return orig(q_stored, cache, tables, np.minimum(np.asarray(lens), n + 0) * 0 + n,
                    query_start, num_q_heads, num_kv_heads, scale)
    monkeypatch.setattr(attention, "prefill", bad_prefill)
    assert _fails(pins.test_prefill_equals_causal_sdpa, 4, 4, "bf16")


def test_mutation_fp8_bias_8(monkeypatch):
    """An E4M3 decode with exponent bias 8 (another FP8 variant) is caught."""
    from oracle import fp8
    orig = fp8.decode
    monkeypatch.setattr(fp8, "decode", lambda c: orig(c) / 2)
    assert _fails(pins.test_fp8_decode_matches_torch_all_codes)


def test_mutation_fp8_ties_away(monkeypatch):
    """Rounding ties away from zero instead of to even is caught."""
    from oracle import fp8
    vals = fp8.decode(np.arange(0x7F, dtype=np.uint8))

    def bad_encode(y):
        y = np.asarray(y, dtype=np.float32)
        a = np.minimum(np.abs(y.astype(np.float64)).ravel(), 448.0)
        codes = np.array([int(np.argmin(np.abs(vals - v) - 1e-30 * np.arange(len(vals))))
                          for v in a], dtype=np.uint8)
        return (codes | (np.signbit(y.ravel()).astype(np.uint8) << 7)).reshape(y.shape)
    monkeypatch.setattr(fp8, "encode_f32", bad_encode)
    assert _fails(pins.test_fp8_worked_values)


def test_mutation_fp8_scale_inverted(monkeypatch):
    """Quantising with x * scale instead of x / scale is caught."""
    from oracle import fp8
    monkeypatch.setattr(fp8, "quantize",
                        lambda x, scale: fp8.encode_f32(np.asarray(x, np.float32) * np.float32(scale)))
    assert _fails(pins.test_fp8_worked_values)


def test_mutation_prefix_match_without_chain(monkeypatch):
    """Matching blocks by their own 16 tokens only (not the whole prefix) is caught."""
    from oracle import prefix
    from tests import test_prefix_cache as pc

    def bad_match(self, tokens, max_blocks=None):
        tokens = tuple(int(t) for t in tokens)
        out = []
        for i in range(len(tokens) // 16):
            blk = tokens[16 * i:16 * (i + 1)]
            hit = next((b for k, b in self._block_of.items() if k[-16:] == blk), None)
            if hit is None:
                break
            out.append(hit)
        for b in out:
            if self.refcount[b] == 0:
                del self._lru[b]
            self.refcount[b] += 1
        return out
    monkeypatch.setattr(prefix.PrefixPoolModel, "match", bad_match)
    assert _fails(pc.test_block_reused_only_under_its_own_prefix)


def test_mutation_prefix_evicts_most_recent(monkeypatch):
    """Evicting the most recently freed indexed block first is caught."""
    from oracle import prefix
    from tests import test_prefix_cache as pc

    def bad_take(self):
        if self._free:
            return self._free.pop()
        b, _ = self._lru.popitem(last=True)
        self._drop_index(b)
        return b
    monkeypatch.setattr(prefix.PrefixPoolModel, "_take", bad_take)
    assert _fails(pc.test_eviction_order_and_descendants)


# ---------------------------------------------------------------- sliding window and swap
from oracle import preempt  # noqa: E402
from tests import test_window_swap as wpins  # noqa: E402


@pytest.mark.parametrize("bad", [lambda p, w: max(0, p - w) if w > 0 else 0,
                                 lambda p, w: max(0, p - w + 2) if w > 0 else 0])
def test_mutation_window_off_by_one(monkeypatch, bad):
    monkeypatch.setattr(attention, "window_start", bad)
    assert _fails(wpins.test_window_decode_equals_banded_sdpa, 17, "f32")
    assert _fails(wpins.test_prefill_window_equals_banded_causal_sdpa, 7)


def test_mutation_window_ignored_in_prefill(monkeypatch):
    orig = attention.prefill
    monkeypatch.setattr(attention, "prefill",
                        lambda *a, window=0, **k: orig(*a, **k))
    assert _fails(wpins.test_prefill_window_equals_banded_causal_sdpa, 20)


def test_mutation_release_one_block_too_many(monkeypatch):
    def bad(L, window):
        lo = attention.window_start(L - 1, window) if L > 0 else 0
        return [i for i in range(-(-L // 16)) if 16 * i < lo]   # frees the block holding lo
    monkeypatch.setattr(preempt, "releasable", bad)
    assert _fails(wpins.test_window_release_frees_only_unneeded_blocks, 17)


def test_mutation_swap_unshares(monkeypatch):
    def bad(src, dst, ids):
        ids = [int(i) for i in ids]
        if len(ids) > dst.num_free():
            raise preempt.PoolError("oom", "")
        new = dst.alloc(len(ids))                # one host block per reference
        src.free(ids)
        return new, list(zip(ids, new))
    monkeypatch.setattr(preempt, "swap", bad)
    assert _fails(wpins.test_swap_round_trip_bit_exact)
