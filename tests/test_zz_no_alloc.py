"""The allocation-free decode entry point (paged_attention_decode_noalloc)
against the entry point it is a variant of (paged_attention_decode /
paged_attention_decode_window / _fp8, with a workspace), through the C ABI:
two calls in a row on one GPU, the second with a smaller input, so the
static scratch still holds the first call's partial states and arrival
counters.  Every output row is also held to the oracle's tolerance."""
import numpy as np
import pytest
import torch

from workloads import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _noalloc(kv, q, scale, window=0):
    from paged_kv_cache_102_amd import _capi as capi
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    capi.paged_attention_decode_noalloc(q, kv.k_cache, kv.v_cache, kv.tables_d, kv.lens_d, out,
                                        num_kv_heads=kv.num_kv_heads, num_blocks=kv.num_blocks,
                                        max_context_len=int(kv.lens.max()), scale=scale,
                                        window=window, k_scale=kv.k_scale, v_scale=kv.v_scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_pair(p, window=0):
    """No-alloc output vs the workspace entry point's and vs the oracle."""
    from tests.gpu_parity import TOL, compare
    s = p.w.spec
    p.kv.window = window
    ref = p.kv.decode(p.q, s.scale).cpu().numpy()
    p.kv.window = 0
    got = _noalloc(p.kv, p.q, s.scale, window)
    # same kernel and split; only the order of the in-CU merges may differ
    d = compare(got, ref, 1e-4)
    e = compare(got, p.oracle_out(window=window), TOL[s.dtype])
    print(f"[noalloc] {s.key} window={window}: vs entry point {d:.2e}, vs oracle {e:.2e}",
          flush=True)


def test_noalloc_two_calls_bf16():
    """The gqa-8b batch (256 sequences), then a 9-sequence batch with empty,
    one-token and block-edge contexts, then the first again."""
    from tests.gpu_parity import Pair
    print("[noalloc] bf16 gqa-8b", flush=True)
    big = Pair(synth.generate("gqa-8b-bf16"))
    _check_pair(big)
    small = Pair(synth.small_random(4711, num_seqs=9, num_q_heads=8, num_kv_heads=2,
                                    head_dim=128, dtype="bf16", max_len=3000,
                                    fixed=[0, 1, 16, 17]))
    _check_pair(small)
    _check_pair(big, window=1024)


def test_noalloc_two_calls_fp8_and_shapes():
    """FP8 cache (the gqa shape, 64 sequences), then a smaller FP8 batch with
    head_dim 64 and 16 query heads per kv head (partial states beyond LDS),
    then bf16 at group 16."""
    from tests.gpu_parity import Pair, TOL, compare, oracle_decode, to_device
    from tests.test_gpu_parity import _fp8_pair
    for w, tag in ((synth.small_random(4712, num_seqs=64, num_q_heads=32, num_kv_heads=8,
                                       head_dim=128, dtype="bf16", max_len=4000), "fp8 D128"),
                   (synth.small_random(4713, num_seqs=5, num_q_heads=16, num_kv_heads=1,
                                       head_dim=64, dtype="bf16", max_len=700), "fp8 D64 g16")):
        s = w.spec
        ora, kv = _fp8_pair(w, 6.0 / 448, 6.0 / 448)
        q = to_device(w.q)
        ref = kv.decode(q, s.scale).cpu().numpy()
        got = _noalloc(kv, q, s.scale)
        d = compare(got, ref, 1e-4)
        e = compare(got, oracle_decode(w.q, ora.cache, ora.tables, ora.lens, s.num_q_heads,
                                       s.num_kv_heads, s.scale), TOL["bf16"])
        print(f"[noalloc] {tag}: vs entry point {d:.2e}, vs oracle {e:.2e}", flush=True)
    g16 = Pair(synth.small_random(4714, num_seqs=300, num_q_heads=16, num_kv_heads=1,
                                  head_dim=128, dtype="bf16", max_len=900))
    _check_pair(g16)


def test_noalloc_rejects_what_it_cannot_hold():
    """Shapes beyond the static scratch, fp32 caches and partitions are
    refused before any launch; nothing is written."""
    from paged_kv_cache_102_amd import _capi as capi
    q = torch.zeros((1, 1, 128), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(16 * 128, dtype=torch.bfloat16, device="cuda")
    t = torch.zeros((16384, 1), dtype=torch.int32, device="cuda")
    out = torch.full((64,), 7.0, dtype=torch.float32, device="cuda")   # never written
    lib = capi._lib
    # 16384 sequences x 128 kv heads: the arrival counters alone fill 16 MiB
    st = lib.paged_attention_decode_noalloc(q.data_ptr(), c.data_ptr(), c.data_ptr(),
                                            t.data_ptr(), t.data_ptr(), 16384, 128, 128, 128,
                                            1, 1, 16, 1.0, 0, capi.PKV_BF16, 1.0, 1.0,
                                            out.data_ptr(), None)
    assert st == capi.PKV_ERR_UNSUPPORTED
    st = lib.paged_attention_decode_noalloc(q.data_ptr(), c.data_ptr(), c.data_ptr(),
                                            t.data_ptr(), t.data_ptr(), 16385, 1, 1, 128,
                                            1, 1, 16, 1.0, 0, capi.PKV_BF16, 1.0, 1.0,
                                            out.data_ptr(), None)
    assert st == capi.PKV_ERR_UNSUPPORTED
    st = lib.paged_attention_decode_noalloc(q.data_ptr(), c.data_ptr(), c.data_ptr(),
                                            t.data_ptr(), t.data_ptr(), 1, 1, 1, 128,
                                            1, 1, 16, 1.0, 0, capi.PKV_F32, 1.0, 1.0,
                                            out.data_ptr(), None)
    assert st == capi.PKV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
