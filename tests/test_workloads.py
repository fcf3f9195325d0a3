"""The seeded input module: shapes, draw order, bf16 rounding, recipe sizes."""
import numpy as np
import torch

from workloads import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 3.0e38]   # ties and a large value
    ours = synth.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_chunked_draws_equal_one_draw():
    a = synth._draw_values(np.random.Generator(np.random.PCG64(9)), (37, 3, 8), "f32", chunk_rows=5)
    b = np.random.Generator(np.random.PCG64(9)).standard_normal(37 * 3 * 8, dtype=np.float32)
    assert np.array_equal(a.ravel(), b)


def test_named_workload_shapes():
    w = synth.generate("tiny-fp32")
    assert list(w.lens) == [17, 33, 64, 100] and w.num_blocks == 64
    assert w.q.shape == (4, 4, 64) and w.k_rows.shape == (214, 4, 64) and w.q.dtype == np.float32
    w3 = synth.generate("gqa-8b-bf16", values=False)
    assert w3.lens[0] == 273 and w3.lens.min() >= 16 and w3.lens.max() <= 8192
    assert 900 <= np.median(w3.lens) <= 1100
    assert sorted(w3.pool_order) == list(range(w3.num_blocks))
    need = int(np.sum(-(-(w3.lens + 1) // 16)))
    assert w3.num_blocks == int(np.ceil(1.25 * need))
    w4 = synth.generate("long-70b-bf16", values=False)
    assert (w4.lens == 32768).all() and w4.max_blocks_per_seq == 2049
    w5 = synth.generate("shared-prefix-bf16", values=False)
    assert (w5.lens == 2048 + w5.suffix_lens).all() and w5.suffix_lens.max() <= 512
    w5c = synth.generate("shared-prefix-cow-bf16", values=False)
    assert (w5c.lens == 2040).all() and (w5c.append_counts == w5c.suffix_lens + 1).all()
    # the two shared-prefix workloads draw the same suffix lengths (same seed, same order)
    assert np.array_equal(w5.suffix_lens, w5c.suffix_lens)


def test_values_deterministic():
    a = synth.generate("tiny-fp32")
    b = synth.generate("tiny-fp32")
    assert np.array_equal(a.k_rows, b.k_rows) and np.array_equal(a.pool_order, b.pool_order)


def test_subset_keeps_each_sequence():
    """A bounded sample (synth.subset) holds exactly the chosen sequences:
    the same lengths and rows, so the oracle gives the same outputs for
    them as on the whole workload (with and without a shared prefix)."""
    from oracle import attention, replay
    for w, pick in ((synth.small_random(21, num_seqs=9, num_q_heads=4, num_kv_heads=2,
                                        head_dim=64, dtype="bf16", max_len=90), [1, 4, 8]),
                    (synth.generate("shared-prefix-bf16"), [0, 77, 127])):
        s = w.spec
        sub = synth.subset(w, pick, seed=3)
        assert list(sub.lens) == [int(w.lens[b]) for b in pick]
        assert sorted(sub.pool_order) == list(range(sub.num_blocks))
        full, part = replay.prefill(w), replay.prefill(sub)
        exp = attention.decode(w.q, full.cache, full.tables, full.lens, s.num_q_heads,
                               s.num_kv_heads, s.scale, seqs=pick)
        got = attention.decode(sub.q, part.cache, part.tables, part.lens, s.num_q_heads,
                               s.num_kv_heads, s.scale)
        assert np.array_equal(got, exp[pick])
        replay.append_step(full, w)
        replay.append_step(part, sub)
        assert list(part.lens) == [int(full.lens[b]) for b in pick]
