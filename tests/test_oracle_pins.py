"""Pins the CPU oracle to things other than itself: values printed on the
pages (tests/golden/*.json, each with its source), closed forms of softmax
attention, invariants, an independent library routine
(torch.nn.functional.scaled_dot_product_attention in float64 on the CPU) and
brute force on tiny pools."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, cache, layout, pool, replay, sizes, slots
from oracle.pool import PoolError, PoolModel
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- page fixtures: blocks
def test_session_273_blocks():
    g = load("pages_blocks.json")["session_273"]
    assert slots.blocks_for(g["tokens"]) == g["blocks"]
    assert sizes.blocks_for(g["tokens"]) == g["blocks"]
    p = PoolModel(64)
    tables = np.full((1, 32), -1, np.int32)
    lens = np.zeros(1, np.int32)
    sl, upd, cows = slots.plan_append(p, tables, lens, [g["tokens"]])
    assert len(upd) == g["blocks"] and not cows
    assert p.stats()["num_used"] == g["blocks"]
    # at most 15 empty slots; exactly 15 here (18*16 - 273)
    assert slots.waste_slots(g["tokens"]) == 15
    assert all(slots.waste_slots(n) <= 15 for n in range(1, 2000))


def test_token_200_position_12():
    g = load("pages_blocks.json")["token_200"]
    order = list(np.random.default_rng(7).permutation(40))
    p = PoolModel(40, init_order=order)
    tables = np.full((1, 16), -1, np.int32)
    lens = np.zeros(1, np.int32)
    sl, _, _ = slots.plan_append(p, tables, lens, [g["token"] + 1])
    assert g["token"] // 16 == g["table_position"]
    assert sl[g["token"]] == tables[0, g["table_position"]] * 16 + g["token"] % 16
    # the 13th allocation (table position 12) returned the 13th id of the order
    assert tables[0, 12] == order[12]


def test_session_blocks_per_layer():
    g = load("pages_blocks.json")["session_128_layers_32"]
    assert sizes.session_blocks(g["tokens"], g["layers"]) == g["blocks"]


def test_worst_case_reservation_example():
    g = load("pages_blocks.json")["worst_case_reservation"]
    used, reserved = g["tokens_used"], g["tokens_reserved"]
    # paged: 15 of 288 allocated slots empty; static: 32 495 of 32 768 empty
    assert sizes.paged_waste_fraction([used]) == pytest.approx(15 / 288)
    assert sizes.static_waste_fraction([used], reserved) == pytest.approx((reserved - used) / reserved)
    # paged allocation is 288 slots = 0.88 % of the contiguous reservation
    assert slots.blocks_for(used) * 16 / reserved == pytest.approx(288 / 32768)


def test_figure_pool_and_reuse():
    g = load("pages_blocks.json")["figure_pool"]
    X, Y, Z, free = g["session_X"], g["session_Y"], g["session_Z"], g["free"]
    order = X + Y + Z + free
    p = PoolModel(g["num_blocks"], init_order=order)
    assert p.alloc(len(X)) == X
    assert p.alloc(len(Y)) == Y
    assert p.alloc(len(Z)) == Z
    assert sorted(p.free_list()) == sorted(free)
    p.check_invariants([X, Y, Z])
    # tokens 0..15 in X's block #7, 16..31 in #2, 32..47 in #11 (the kernel
    # section of the same page walks X's table this way)
    assert [slots.slot_of(X, t) // 16 for t in (0, 15, 16, 31, 32, 47)] == [7, 7, 2, 2, 11, 11]
    # X ends: its blocks return to the pool and the next session gets them
    p.free(X)
    assert p.num_free() == len(free) + len(X)
    nxt = p.alloc(len(X))
    assert sorted(nxt) == sorted(X)
    p.check_invariants([nxt, Y, Z])


def test_lesson_table_entries():
    g = load("pages_blocks.json")["lesson_table"]
    phys = [ph for _, ph in g["logical_to_physical"]]
    rest = [i for i in range(16) if i not in phys]
    p = PoolModel(16, init_order=phys + rest)
    tables = np.full((1, 4), -1, np.int32)
    lens = np.zeros(1, np.int32)
    slots.plan_append(p, tables, lens, [40])
    for logical, physical in g["logical_to_physical"]:
        assert tables[0, logical] == physical
    # the last entry holds 40 - 32 = 8 tokens, the others 16
    assert [min(16, 40 - 16 * i) for i in range(3)] == [16, 16, 8]


# ---------------------------------------------------------------- page fixtures: sizes
def test_bytes_per_token_table():
    g = load("pages_sizes.json")["bytes_per_token"]
    for r in g["rows"]:
        bpt = sizes.kv_bytes_per_token(r["n_layers"], r["n_kv_heads"], r["head_dim"], g["elem_bytes"])
        assert bpt == r["bytes_per_token"], r["model"]
        for ctx, key in ((8192, "gb_8k"), (32768, "gb_32k"), (131072, "gb_128k")):
            gib = sizes.kv_bytes(r["n_layers"], r["n_kv_heads"], r["head_dim"], ctx, g["elem_bytes"]) / 2**30
            assert round(gib, 2) == pytest.approx(r[key], abs=0.006), (r["model"], key)


def test_kv_transfer_70b():
    g = load("pages_sizes.json")["kv_transfer_70b"]
    bpt = sizes.kv_bytes_per_token(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["elem_bytes"])
    assert bpt == g["bytes_per_token"]
    total = sizes.kv_bytes(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["tokens"], g["elem_bytes"])
    assert round(total / 1e9, 2) == g["gb_decimal"]


def test_quadratic_cost_table():
    for n, without, with_cache, ratio in load("pages_sizes.json")["quadratic_cost"]["rows"]:
        assert sizes.attention_ops_without_cache(n) == without
        assert with_cache == n
        assert round(without / with_cache) == pytest.approx(ratio, rel=0.01)
    g = load("pages_sizes.json")["lesson_100_tokens"]
    # about 5 000 redundant recomputations at 100 tokens, ~half a million at 1 000
    assert sizes.attention_ops_without_cache(g["n"] - 1) == pytest.approx(g["approx_ops"], rel=0.02)
    assert sizes.attention_ops_without_cache(g["n2"] - 1) == pytest.approx(g["approx_ops2"], rel=0.01)


def test_pool_example():
    g = load("pages_sizes.json")["pool_example"]
    bb = sizes.all_layer_block_bytes(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["elem_bytes"],
                                     g["block_tokens"])
    assert bb == g["block_bytes"]
    assert g["blocks_approx"] * g["block_tokens"] == g["tokens_total"]
    # 5.5 GiB over 2 MiB blocks is 2816, the page's "~2800" (within 1 %);
    # mixing decimal GB with binary MB would give 2622
    assert sizes.pool_blocks(int(5.5 * 2**30), bb) == 2816
    assert sizes.pool_blocks(int(5.5 * 2**30), bb) == pytest.approx(g["blocks_approx"], rel=0.01)
    # the per-layer block of the same model is 1/32 of it: 16*2*8*128*2 = 64 KiB
    assert sizes.all_layer_block_bytes(1, 8, 128, 2) * 32 == bb


# ---------------------------------------------------------------- pool: brute force + CoW
def _all_ops(nb, seqs):
    ops = [("alloc", 1), ("alloc", 2)]
    for s in range(len(seqs)):
        ops += [("share", s), ("free", s), ("cow", s)]
    return ops


def _apply(p, seqs, op):
    kind, arg = op
    if kind == "alloc":
        seqs.append(p.alloc(arg))
    elif kind == "share":
        p.share(seqs[arg])
        seqs.append(list(seqs[arg]))
    elif kind == "free":
        p.free(seqs[arg])
        seqs.pop(arg)
    elif kind == "cow":
        new, copied = p.cow(seqs[arg][-1])
        assert copied == (new != seqs[arg][-1])
        seqs[arg][-1] = new


@pytest.mark.parametrize("nb", [1, 2, 3])
def test_pool_brute_force_invariants(nb):
    """Every sequence of up to 4 operations on a tiny pool keeps the
    invariants; a failing operation leaves the pool exactly as it was."""
    count = 0

    def rec(p, seqs, depth):
        nonlocal count
        p.check_invariants(seqs)
        if depth == 0:
            return
        for op in _all_ops(nb, seqs):
            q = PoolModel(nb)
            q.restore(p.snapshot())
            s2 = [list(x) for x in seqs]
            before = q.snapshot()
            try:
                _apply(q, s2, op)
            except PoolError as e:
                assert e.kind in ("oom", "invalid")
                assert q.snapshot() == before
                continue
            count += 1
            rec(q, s2, depth - 1)

    rec(PoolModel(nb), [], 4)
    assert count > 0


def test_pool_errors():
    p = PoolModel(4)
    with pytest.raises(PoolError) as e:
        p.alloc(5)
    assert e.value.kind == "oom" and p.num_free() == 4
    a = p.alloc(2)
    with pytest.raises(PoolError):
        p.free([a[0], a[0]])                 # two drops, one reference
    assert p.refcount[a[0]] == 1
    with pytest.raises(PoolError):
        p.share([3])                         # free block
    with pytest.raises(PoolError):
        p.free([4])                          # out of range
    with pytest.raises(PoolError) as e:
        PoolModel(4, block_size=32)
    assert e.value.kind == "unsupported"


def test_cow_beam_fork():
    """Four beams share a 40-token prefix (3 blocks, the last one partial);
    each appends a token: the first three get private copies of the last
    block only, the fourth writes in place."""
    p = PoolModel(32)
    tables = np.full((4, 8), -1, np.int32)
    lens = np.zeros(4, np.int32)
    slots.plan_append(p, tables, lens, [40, 0, 0, 0])
    for b in range(1, 4):
        p.share(tables[0, :3])
        tables[b, :3] = tables[0, :3]
        lens[b] = 40
    shared_last = int(tables[0, 2])
    assert p.refcount[shared_last] == 4
    sl, upd, cows = slots.plan_append(p, tables, lens, None)
    assert [c[0] for c in cows] == [shared_last] * 3
    assert tables[3, 2] == shared_last and p.refcount[shared_last] == 1
    assert all(p.refcount[int(tables[b, 0])] == 4 for b in range(4))   # full blocks stay shared
    assert sorted(set(int(tables[b, 2]) for b in range(4))) == sorted(
        [shared_last] + [c[1] for c in cows])
    p.check_invariants([list(tables[b, :3]) for b in range(4)])
    assert list(sl % 16) == [8, 8, 8, 8]


def test_plan_append_all_or_nothing():
    p = PoolModel(3)
    tables = np.full((2, 4), -1, np.int32)
    lens = np.zeros(2, np.int32)
    slots.plan_append(p, tables, lens, [16, 16])      # 2 blocks
    snap, t0, l0 = p.snapshot(), tables.copy(), lens.copy()
    with pytest.raises(PoolError) as e:
        slots.plan_append(p, tables, lens, [1, 1])     # needs 2, 1 free
    assert e.value.kind == "oom"
    assert p.snapshot() == snap and (tables == t0).all() and (lens == l0).all()
    p = PoolModel(16)
    tables = np.full((2, 4), -1, np.int32)
    lens = np.zeros(2, np.int32)
    slots.plan_append(p, tables, lens, [16, 16])
    snap, t0, l0 = p.snapshot(), tables.copy(), lens.copy()
    with pytest.raises(PoolError) as e:
        slots.plan_append(p, tables, lens, [5, 49])    # beyond 4 table entries
    assert e.value.kind == "invalid"
    assert p.snapshot() == snap and (tables == t0).all() and (lens == l0).all()


# ---------------------------------------------------------------- layout
def test_layout_golden_offsets():
    g = load("layout_offsets.json")
    for D, rows in g["cases"].items():
        for t, d, ko, vo in rows:
            assert layout.k_offset(t, d) == ko, (D, t, d)
            assert layout.v_offset(t, d) == vo, (D, t, d)
    for D, rows in g["fp8_cases"].items():
        for t, d, ko, vo in rows:
            assert layout.k8_offset(t, d, int(D)) == ko, (D, t, d)
            assert layout.v8_offset(t, d, int(D)) == vo, (D, t, d)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_layout_is_bijective(D):
    kt, vt = layout.offset_tables(D)
    assert sorted(kt.ravel()) == list(range(16 * D))
    assert sorted(vt.ravel()) == list(range(16 * D))


# ---------------------------------------------------------------- cache
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_then_gather_roundtrip(dtype):
    rng = np.random.default_rng(3)
    NB, H, D = 6, 2, 64
    fill = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    c = cache.CacheModel(NB, H, D, dtype, fill=fill)
    rows = rng.standard_normal((20, H, D)).astype(np.float32)
    stored = rows if dtype == "f32" else synth.round_bf16_bits(rows)
    sl = rng.permutation(NB * 16)[:20]
    sl[3] = -1                                             # padding row
    c.write(stored, stored, sl)
    for i, s in enumerate(sl):
        if s < 0:
            continue
        blk, t = divmod(int(s), 16)
        for h in range(H):
            tile_k = c.k[blk, h]
            got = np.array([tile_k[layout.k_offset(t, d)] for d in range(D)])
            assert got.tobytes() == np.asarray(stored[i, h]).tobytes()
            tile_v = c.v[blk, h]
            got = np.array([tile_v[layout.v_offset(t, d)] for d in range(D)])
            assert got.tobytes() == np.asarray(stored[i, h]).tobytes()
    # everything else still holds the fill pattern
    written = {int(s) for s in sl if s >= 0}
    for blk in range(NB):
        for t in range(16):
            if blk * 16 + t in written:
                continue
            for h in range(H):
                ks = c.k[blk, h][[layout.k_offset(t, d) for d in range(D)]]
                assert np.asarray(ks).view(np.uint32 if dtype == "f32" else np.uint16).tolist() == \
                    [np.asarray(fill).view(np.uint32 if dtype == "f32" else np.uint16).item()] * D


def test_copy_blocks():
    c = cache.CacheModel(4, 2, 32, "bf16")
    c.k[1] = 5
    c.v[1] = 7
    c.copy_blocks([(1, 3), (9, 0)])                        # second pair out of range: skipped
    assert (c.k[3] == 5).all() and (c.v[3] == 7).all() and (c.k[0] == 0).all()


# ---------------------------------------------------------------- attention
def _paged_vs_contiguous(rng, B, Hq, Hkv, D, dtype, max_len, NB):
    lens = rng.integers(1, max_len + 1, size=B)
    need = sum(-(-int(n) // 16) for n in lens)
    assert need <= NB
    p = PoolModel(NB, init_order=rng.permutation(NB))
    mb = max(-(-int(n) // 16) for n in lens)
    tables = np.full((B, mb), -1, np.int32)
    cur = np.zeros(B, np.int32)
    sl, _, _ = slots.plan_append(p, tables, cur, lens)
    T = int(lens.sum())
    kf = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    vf = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    qf = rng.standard_normal((B, Hq, D)).astype(np.float32)
    if dtype == "bf16":
        kf, vf, qf = (synth.bf16_bits_to_f32(synth.round_bf16_bits(x)) for x in (kf, vf, qf))
        ks, vs, qs = (synth.round_bf16_bits(x) for x in (kf, vf, qf))
    else:
        ks, vs, qs = kf, vf, qf
    c = cache.CacheModel(NB, Hkv, D, dtype, fill=np.uint16(0x7FC0) if dtype == "bf16" else np.nan)
    c.write(ks, vs, sl)
    scale = 1 / math.sqrt(D)
    out = attention.decode(qs, c, tables, cur, Hq, Hkv, scale)
    # independent: torch SDPA in float64 on contiguous per-sequence K/V
    start = np.concatenate([[0], np.cumsum(lens)])
    for b in range(B):
        k = torch.from_numpy(kf[start[b]:start[b + 1]].astype(np.float64)).permute(1, 0, 2)
        v = torch.from_numpy(vf[start[b]:start[b + 1]].astype(np.float64)).permute(1, 0, 2)
        k = k.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        v = v.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        q = torch.from_numpy(qf[b].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)
    return out


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (16, 2), (6, 3)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_equals_contiguous_sdpa(Hq, Hkv, dtype):
    rng = np.random.default_rng(Hq * 100 + Hkv)
    _paged_vs_contiguous(rng, B=5, Hq=Hq, Hkv=Hkv, D=64, dtype=dtype, max_len=70, NB=40)


def test_paged_result_independent_of_block_placement():
    """Same tokens, two different scatterings of blocks: identical outputs."""
    outs = []
    for seed in (1, 2):
        rng = np.random.default_rng(11)
        vals = rng.standard_normal((50, 1, 32)).astype(np.float32)
        q = rng.standard_normal((1, 2, 32)).astype(np.float32)
        p = PoolModel(8, init_order=np.random.default_rng(seed).permutation(8))
        tables = np.full((1, 4), -1, np.int32)
        lens = np.zeros(1, np.int32)
        sl, _, _ = slots.plan_append(p, tables, lens, [50])
        c = cache.CacheModel(8, 1, 32, "f32", fill=np.nan)
        c.write(vals, vals[::-1].copy(), sl)
        outs.append((tables.copy(), attention.decode(q, c, tables, lens, 2, 1, 0.3)))
    assert not (outs[0][0] == outs[1][0]).all()
    assert np.array_equal(outs[0][1], outs[1][1])


def test_closed_forms():
    rng = np.random.default_rng(5)
    D = 16
    v = rng.standard_normal((7, D))
    k = rng.standard_normal((7, D))
    q = rng.standard_normal(D)
    # one token: the output is that token's value
    np.testing.assert_array_equal(attention.attend(q, k[:1], v[:1], 0.5), v[0])
    # weights add up to one: with every value = 1 the output is 1
    np.testing.assert_allclose(attention.attend(q, k, np.ones((7, D)), 0.25), 1.0, atol=1e-15)
    # zero query, or identical keys: plain mean of the values
    np.testing.assert_allclose(attention.attend(np.zeros(D), k, v, 1.0), v.mean(0), atol=1e-15)
    np.testing.assert_allclose(attention.attend(q, np.tile(k[:1], (7, 1)), v, 1.0), v.mean(0),
                               atol=1e-15)
    # two tokens: w0 = sigmoid(s0 - s1)
    s0, s1 = 0.5 * k[0] @ q, 0.5 * k[1] @ q
    w0 = 1 / (1 + math.exp(-(s0 - s1)))
    np.testing.assert_allclose(attention.attend(q, k[:2], v[:2], 0.5), w0 * v[0] + (1 - w0) * v[1],
                               atol=1e-14)
    # hand example: q=(1,0), keys e1, e2, scale 1 -> weights e/(e+1), 1/(e+1)
    out = attention.attend(np.array([1.0, 0.0]), np.eye(2), np.eye(2), 1.0)
    np.testing.assert_allclose(out, [0.7310585786300049, 0.2689414213699951], atol=1e-15)
    # the page's illustration: affinities giving 70 % / 20 % / 10 % weights
    w = np.array([0.7, 0.2, 0.1])
    keys = np.log(w)[:, None]
    np.testing.assert_allclose(attention.attend(np.array([1.0]), keys, np.eye(3), 1.0), w, atol=1e-15)
    # the order of tokens does not matter (same permutation of keys and values)
    perm = rng.permutation(7)
    np.testing.assert_allclose(attention.attend(q, k[perm], v[perm], 0.7),
                               attention.attend(q, k, v, 0.7), atol=1e-14)
    # empty context: zero row
    assert not attention.attend(q, k[:0], v[:0], 1.0).any()


@pytest.mark.parametrize("L,P", [(1, 512), (511, 512), (513, 512), (2000, 512), (777, 32)])
def test_partitioned_lse_equals_single_pass(L, P):
    rng = np.random.default_rng(L)
    k = rng.standard_normal((L, 64)) * 3
    v = rng.standard_normal((L, 64))
    q = rng.standard_normal(64)
    np.testing.assert_allclose(attention.attend_partitioned(q, k, v, 0.125, P),
                               attention.attend(q, k, v, 0.125), rtol=0, atol=1e-12)


def test_large_scores_stable():
    """Scores of +-1000 would overflow a naive exp; the result stays finite
    and matches the single surviving token."""
    k = np.array([[1000.0], [-1000.0], [999.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    out = attention.attend(np.array([1.0]), k, v, 1.0)
    w = np.array([1.0, 0.0, math.exp(-1.0)])
    np.testing.assert_allclose(out, (w @ v) / w.sum(), atol=1e-15)


# ---------------------------------------------------------------- replay of the named workloads
def test_replay_tiny_workload():
    w = synth.generate("tiny-fp32")
    st = replay.prefill(w, fill=np.float32(np.nan))
    assert list(st.lens) == [17, 33, 64, 100]
    used = sum(slots.blocks_for(int(n)) for n in st.lens)
    assert st.pool.stats()["num_used"] == used == 16
    st.pool.check_invariants(replay.live_tables(st))
    sl, upd, cows = replay.append_step(st, w)
    # only the 64-token sequence crosses into a new block (position 64 % 16 == 0)
    assert [u[0] // w.max_blocks_per_seq for u in upd] == [2] and not cows
    assert list(st.lens) == [18, 34, 65, 101]
    # the appended tokens are found where the slots say
    for b in range(4):
        p = int(st.lens[b]) - 1
        assert sl[b] == st.tables[b, p // 16] * 16 + p % 16


def test_replay_shared_prefix_cow():
    w = synth.generate("shared-prefix-cow-bf16", values=False)
    # a light copy: no values needed to check the tables
    B = w.spec.num_seqs
    p = PoolModel(w.num_blocks, init_order=w.pool_order)
    tables = np.full((B, w.max_blocks_per_seq), -1, np.int32)
    lens = np.zeros(B, np.int32)
    first = np.zeros(B, np.int64)
    first[0] = w.spec.prefix_len
    slots.plan_append(p, tables, lens, first)
    for b in range(1, B):
        p.share(tables[0, :128])
        tables[b, :128] = tables[0, :128]
        lens[b] = w.spec.prefix_len
    last = int(tables[0, 127])
    assert p.refcount[last] == B
    sl, upd, cows = slots.plan_append(p, tables, lens, w.append_counts)
    assert len(cows) == B - 1 and all(c[0] == last for c in cows)
    assert p.refcount[last] == 1
    assert list(lens) == list(w.spec.prefix_len + w.suffix_lens + 1)
    p.check_invariants([list(tables[b, :slots.blocks_for(int(lens[b]))]) for b in range(B)])


# ---------------------------------------------------------------- multi-query (chunked prefill)
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 3)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_equals_causal_sdpa(Hq, Hkv, dtype):
    """oracle.attention.prefill against torch SDPA (fp64, CPU) with an
    explicit causal mask on contiguous K/V: chunk row i of sequence b is
    position L_b - n_b + i and sees positions 0..that."""
    rng = np.random.default_rng(Hq * 10 + Hkv + (dtype == "bf16"))
    B, D, NB = 5, 32, 40
    lens = np.array([1, 17, 40, 64, 70])
    chunks = np.array([1, 0, 40, 5, 33])           # a decode row, an idle sequence, a full prefill
    p = PoolModel(NB, init_order=rng.permutation(NB))
    mb = max(-(-int(n) // 16) for n in lens)
    tables = np.full((B, mb), -1, np.int32)
    cur = np.zeros(B, np.int32)
    sl, _, _ = slots.plan_append(p, tables, cur, lens)
    T = int(lens.sum())
    kf = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    vf = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    Q = int(chunks.sum())
    qf = rng.standard_normal((Q, Hq, D)).astype(np.float32)
    if dtype == "bf16":
        kf, vf, qf = (synth.bf16_bits_to_f32(synth.round_bf16_bits(x)) for x in (kf, vf, qf))
        ks, vs, qs = (synth.round_bf16_bits(x) for x in (kf, vf, qf))
    else:
        ks, vs, qs = kf, vf, qf
    c = cache.CacheModel(NB, Hkv, D, dtype, fill=np.uint16(0x7FC0) if dtype == "bf16" else np.nan)
    c.write(ks, vs, sl)
    qstart = np.concatenate([[0], np.cumsum(chunks)])
    scale = 1 / math.sqrt(D)
    out = attention.prefill(qs, c, tables, cur, qstart, Hq, Hkv, scale)
    start = np.concatenate([[0], np.cumsum(lens)])
    for b in range(B):
        n, L = int(chunks[b]), int(lens[b])
        if n == 0:
            continue
        k = torch.from_numpy(kf[start[b]:start[b + 1]].astype(np.float64)).permute(1, 0, 2)
        v = torch.from_numpy(vf[start[b]:start[b + 1]].astype(np.float64)).permute(1, 0, 2)
        k = k.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        v = v.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        q = torch.from_numpy(qf[qstart[b]:qstart[b + 1]].astype(np.float64)).permute(1, 0, 2)
        pos = torch.arange(L - n, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos             # [n][L], True = attend
        ref = torch.nn.functional.scaled_dot_product_attention(q.contiguous(), k, v,
                                                               attn_mask=mask, scale=scale)
        np.testing.assert_allclose(out[qstart[b]:qstart[b + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_prefill_closed_forms():
    """Chunk row at position 0 sees only token 0: its output is v_0; a
    one-row chunk at the end of the context is a decode step."""
    rng = np.random.default_rng(3)
    D, L = 32, 20
    p = PoolModel(4, init_order=np.arange(4))
    tables = np.full((1, 2), -1, np.int32)
    cur = np.zeros(1, np.int32)
    sl, _, _ = slots.plan_append(p, tables, cur, [L])
    kv = rng.standard_normal((L, 1, D)).astype(np.float32)
    vv = rng.standard_normal((L, 1, D)).astype(np.float32)
    c = cache.CacheModel(4, 1, D, "f32", fill=np.nan)
    c.write(kv, vv, sl)
    q = rng.standard_normal((L, 2, D)).astype(np.float32)
    out = attention.prefill(q, c, tables, cur, np.array([0, L]), 2, 1, 0.25)
    np.testing.assert_array_equal(out[0, 0], vv[0, 0].astype(np.float64))
    np.testing.assert_array_equal(out[0, 1], vv[0, 0].astype(np.float64))
    # the last chunk row equals plain attention over the whole context
    ref = attention.attend(q[L - 1, 1].astype(np.float64), kv[:, 0].astype(np.float64),
                           vv[:, 0].astype(np.float64), 0.25)
    np.testing.assert_allclose(out[L - 1, 1], ref, atol=1e-15)


# ---------------------------------------------------------------- FP8 E4M3 cache
from oracle import fp8 as ofp8  # noqa: E402


def test_fp8_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ofp8.decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.standard_normal(5000) * 1e-3,
                        ofp8.decode(np.arange(0x7F, dtype=np.uint8)),           # exact values
                        (ofp8.decode(np.arange(0x7E, dtype=np.uint8)) +          # midpoints: ties
                         ofp8.decode(np.arange(1, 0x7F, dtype=np.uint8))) / 2]).astype(np.float32)
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ofp8.encode_f32(x), ref)


def test_fp8_worked_values():
    """Values fixed by the OCP E4M3 definition, and the library's clamp at 448."""
    cases = [(448.0, 0x7E), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (1.0, 0x38), (-2.0, 0xC0),
             (0.0, 0x00), (-0.0, 0x80), (1 + 1 / 16, 0x38), (1 + 3 / 16, 0x3A), (1e6, 0x7E),
             (-1e6, 0xFE), (464.0, 0x7E), (3 * 2.0 ** -10, 0x02), (2.0 ** -10, 0x00)]
    for v, c in cases:
        assert int(ofp8.encode_f32(np.float32(v))) == c, (v, c)
    assert int(ofp8.encode_f32(np.float32(np.nan))) == 0x7F
    assert ofp8.decode(np.uint8(0x7E)) == 448.0 and np.isnan(ofp8.decode(np.uint8(0xFF)))
    # quantize: one float32 multiply by float32(1/scale), then the code
    assert int(ofp8.quantize(np.float32(3.0), 0.5)) == int(ofp8.encode_f32(np.float32(6.0)))


@pytest.mark.parametrize("D", [32, 64, 96, 128])
def test_fp8_layout_is_the_bf16_operand_order(D):
    """Every byte of an FP8 tile is used once, and (t, d) sits at the same
    (lane, piece, position) as in the bf16 tile: bf16 16-byte piece j of lane
    l starts at element 512 j + 8 l; FP8 pieces 2i, 2i + 1 of lane l are the
    16 bytes at 1024 i + 16 l, so one load instruction reads 1 KiB in order
    (a last unpaired piece: the 8 bytes at 1024 i + 8 l)."""
    pieces = D // 32
    for k8, k16 in ((layout.k8_offset, layout.k_offset), (layout.v8_offset, layout.v_offset)):
        seen = set()
        for t in range(16):
            for d in range(D):
                o8, o16 = k8(t, d, D), k16(t, d)
                seen.add(o8)
                j, l, w = o16 // 512, (o16 % 512) // 8, o16 % 8
                if j // 2 * 2 + 1 < pieces:
                    assert o8 == 1024 * (j // 2) + 16 * l + 8 * (j % 2) + w
                else:
                    assert o8 == 1024 * (j // 2) + 8 * l + w
        assert seen == set(range(16 * D))


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_fp8_paged_equals_contiguous_sdpa(Hq, Hkv):
    """Decode over an FP8 cache equals torch SDPA (fp64) on the dequantised
    values, gathered contiguously."""
    rng = np.random.default_rng(80 + Hq)
    B, D, NB = 4, 64, 24
    lens = rng.integers(1, 80, size=B)
    p = PoolModel(NB, init_order=rng.permutation(NB))
    mb = max(-(-int(n) // 16) for n in lens)
    tables = np.full((B, mb), -1, np.int32)
    cur = np.zeros(B, np.int32)
    sl, _, _ = slots.plan_append(p, tables, cur, lens)
    T = int(lens.sum())
    ks_, vs_ = 0.05, 0.02
    kx = rng.standard_normal((T, Hkv, D)).astype(np.float32) * 3
    vx = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    kc, vc = ofp8.quantize(kx, ks_), ofp8.quantize(vx, vs_)
    qf = synth.bf16_bits_to_f32(synth.round_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32)))
    qs = synth.round_bf16_bits(qf)
    c = cache.CacheModel(NB, Hkv, D, "fp8", fill=np.uint8(0x7F), k_scale=ks_, v_scale=vs_)
    c.write(kc, vc, sl)
    out = attention.decode(qs, c, tables, cur, Hq, Hkv, 1 / math.sqrt(D))
    kd = ofp8.decode(kc) * float(np.float32(ks_))
    vd = ofp8.decode(vc) * float(np.float32(vs_))
    start = np.concatenate([[0], np.cumsum(lens)])
    for b in range(B):
        k = torch.from_numpy(kd[start[b]:start[b + 1]]).permute(1, 0, 2)
        v = torch.from_numpy(vd[start[b]:start[b + 1]]).permute(1, 0, 2)
        k = k.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        v = v.repeat_interleave(Hq // Hkv, dim=0).contiguous()
        q = torch.from_numpy(qf[b].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=1 / math.sqrt(D))
        np.testing.assert_allclose(out[b], ref[:, 0, :].numpy(), rtol=0, atol=1e-12)
