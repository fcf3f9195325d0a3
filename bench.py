"""Benchmark of the paged decode step on one MI355X.

A step is one pass of the whole hot path for a batch of sequences, each
gaining one token:
  host slot planning + block allocation (C++), one pinned host-to-device
  upload, block-table deltas, copy-on-write copies (when a shared block is
  hit), the K/V write, and decode attention (split-K partitions + LSE
  merge).
Contexts grow by one token per step, exactly as in serving.

Workload: gqa-8b-bf16 -- 256 sequences, 32 query / 8 kv heads, head_dim 128,
bf16 cache, log-normal lengths (median 1000, sigma 1, clipped to [16, 8192],
one sequence at 273), scattered 16-token blocks.

Prints ONE JSON line.  value = effective KV GB/s of the whole step (K+V
bytes the decode reads / step time); roofline = the decode main kernel's
own average duration (HIP events recorded by the library on the kernel's
stream) against 8 TB/s; cpu_baseline = the CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "gqa-8b-bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bf16_cu_gqa-8b_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    src = os.path.join(ROOT, "paged_kv_cache_102_amd", "csrc", "kernels.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def committed_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def kernel_name(partition: int) -> str:
    """The decode main kernel the library launches for the headline workload."""
    if partition != 0:
        return "decode_bf16_kernel<128,3,2> + lse_reduce_kernel"
    if os.environ.get("PKV_DECODE_SPLIT") == "wave":
        return "decode_bf16_balanced_kernel<128,2,2> (per-wave split, merge inside)"
    return "decode_bf16_cu_kernel<128,2,2> (per-CU split, LDS fold, merge inside)"


def all_configs(path: str, dev):
    """Decode alone (back to back, after warm-up) on every bf16 workload at
    its full size; written to ``path`` as JSON."""
    import numpy as np
    import torch
    from paged_kv_cache_102_amd.driver import PagedKV, replay_prefill
    from workloads import synth
    res = {}
    for key in ("mha-7b-bf16", "gqa-8b-bf16", "long-70b-bf16", "shared-prefix-bf16"):
        w = synth.generate(key)
        s = w.spec

        def to_dev(rows):
            return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(
                torch.bfloat16)
        kv = PagedKV(num_blocks=w.num_blocks, num_seqs=s.num_seqs,
                     max_blocks_per_seq=w.max_blocks_per_seq, num_q_heads=s.num_q_heads,
                     num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype=s.dtype, device=dev,
                     init_order=w.pool_order)
        replay_prefill(kv, w, to_dev)
        q = to_dev(w.q)
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        for _ in range(20):
            kv.decode(q, s.scale, out=out)
        torch.cuda.synchronize()
        n = 100
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            kv.decode(q, s.scale, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        logical = kv_bytes(kv.lens, s.num_kv_heads, s.head_dim)
        blocks = -(-kv.lens.astype(np.int64) // 16)
        unique = (int(blocks.sum()) if s.prefix_len == 0 else
                  int(blocks.sum()) - (s.num_seqs - 1) * (s.prefix_len // 16)) * 16 \
            * 2 * s.num_kv_heads * s.head_dim * 2
        res[key] = {"ms": round(ms, 4), "seqs_per_s": round(s.num_seqs / ms * 1e3, 1),
                    "logical_kv_bytes": logical, "unique_kv_bytes": unique,
                    "effective_kv_gb_per_s": round(logical / ms / 1e6, 1),
                    "frac_of_hbm_peak_unique": round(unique / ms / 1e6 / HBM_PEAK_GBS, 4)}
        log(f"[bench] {key}: {res[key]}")
        del kv, q, out
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump(res, f, indent=1)


BF16_MFMA_PEAK_TFLOPS = 2500.0


def prefill_measure(dev, reps: int = 20):
    """Multi-query (chunked prefill) attention: 8 sequences of the gqa-8b
    shape with 1024..2048 cached tokens each take a 512-token chunk, causal
    inside the chunk.  Returns the kernel time and its rate against the bf16
    matrix-core peak (4 * D flops per (query row, attended token))."""
    import numpy as np
    import torch
    from paged_kv_cache_102_amd.driver import PagedKV, replay_prefill
    from workloads import synth
    n = 512
    w = synth.small_random(4242, num_seqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           dtype="bf16", max_len=2048, min_len=1024, append=n)
    s = w.spec

    def to_dev(rows):
        return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(torch.bfloat16)
    kv = PagedKV(num_blocks=w.num_blocks, num_seqs=s.num_seqs,
                 max_blocks_per_seq=w.max_blocks_per_seq, num_q_heads=s.num_q_heads,
                 num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype=s.dtype, device=dev,
                 init_order=w.pool_order)
    replay_prefill(kv, w, to_dev)
    kv.append(to_dev(w.k_app), to_dev(w.v_app), w.append_counts)
    T = n * s.num_seqs
    q = torch.randn((T, s.num_q_heads, s.head_dim), device=dev).to(torch.bfloat16)
    qstart = np.arange(0, T + 1, n, dtype=np.int32)
    out = torch.empty((T, s.num_q_heads, s.head_dim), dtype=torch.float32, device=dev)
    for _ in range(3):
        kv.prefill_attention(q, qstart, s.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kv.prefill_attention(q, qstart, s.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    lens = kv.lens.astype(np.int64)
    attended = int(sum(int(L) * n - n * (n - 1) // 2 for L in lens))   # sum over rows of (p + 1)
    flops = 4.0 * s.head_dim * s.num_q_heads * attended
    kv_unique = int(lens.sum()) * 2 * s.num_kv_heads * s.head_dim * 2
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": "8 sequences x 512-token chunks on 1024..2048 cached tokens, 32 q / 8 kv heads, "
                        "head_dim 128, bf16",
            "kernel": "prefill_bf16_kernel<128,2,2>", "ms": round(ms, 4),
            "tflops": round(tflops, 2), "bound": "mfma", "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
            "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "unique_kv_gb_per_s": round(kv_unique / ms / 1e6, 1)}


def fp8_measure(dev, w, reps: int = 50):
    """Decode alone over an FP8 E4M3 copy of the headline workload's cache
    (same lengths, same block placement, rows quantised with per-tensor
    scales on the GPU): time per call and rate of its FP8 bytes."""
    import numpy as np
    import torch
    from paged_kv_cache_102_amd.driver import PagedKV, replay_prefill
    s = w.spec

    def to_dev(rows):
        return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(torch.bfloat16)
    kv = PagedKV(num_blocks=w.num_blocks, num_seqs=s.num_seqs,
                 max_blocks_per_seq=w.max_blocks_per_seq, num_q_heads=s.num_q_heads,
                 num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype="fp8", device=dev,
                 init_order=w.pool_order, k_scale=6.0 / 448, v_scale=6.0 / 448)
    replay_prefill(kv, w, to_dev)
    q = to_dev(w.q)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    for _ in range(10):
        kv.decode(q, s.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kv.decode(q, s.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    b = kv_bytes(kv.lens, s.num_kv_heads, s.head_dim, elem=1)
    res = {"workload": f"{WORKLOAD} at its prefill lengths, FP8 E4M3 cache", "ms": round(ms, 4),
           "kv_bytes": b, "kv_gb_per_s": round(b / ms / 1e6, 1),
           "frac_of_hbm_peak": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
           "seqs_per_s": round(s.num_seqs / ms * 1e3, 1)}
    del kv
    torch.cuda.empty_cache()
    return res


def kv_bytes(lens, num_kv_heads, head_dim, elem=2) -> int:
    return int(lens.astype("int64").sum()) * 2 * num_kv_heads * head_dim * elem


def cpu_baseline(w, seconds: float = 12.0):
    """The oracle, as it stands, on this host: decode over the whole batch,
    repeated until ``seconds`` of CPU work, single-threaded BLAS."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention, replay
    st = replay.prefill(w)
    s = w.spec
    reps, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            attention.decode(w.q, st.cache, st.tables, st.lens, s.num_q_heads, s.num_kv_heads,
                             s.scale)
            reps += 1
            if time.perf_counter() - t0 >= seconds or reps >= 4:
                break
    dt = time.perf_counter() - t0
    gbs = kv_bytes(st.lens, s.num_kv_heads, s.head_dim) * reps / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seqs_per_s": round(s.num_seqs * reps / dt, 2),
            "sample": f"full {s.num_seqs}-sequence batch at its prefill lengths, {reps} pass(es), "
                      f"{dt:.1f} s, numpy float64, 1 thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition", type=int, default=0, help="tokens per partition (0 = default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only-steps", type=int, default=50)
    ap.add_argument("--no-read-ceiling", dest="read_ceiling", action="store_false",
                    help="skip the streaming-read ceiling measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--no-contiguous", dest="contiguous", action="store_false",
                    help="skip the paged-vs-contiguous comparison")
    ap.add_argument("--no-fp8", dest="fp8", action="store_false",
                    help="skip the FP8 cache decode measurement")
    ap.add_argument("--no-prefill", dest="prefill", action="store_false",
                    help="skip the multi-query (chunked prefill) measurement")
    ap.add_argument("--all-configs", metavar="PATH", default=None,
                    help="also time decode alone on every workload and write them to PATH (JSON)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path "
              "is single-GPU in this build.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from paged_kv_cache_102_amd import _capi as capi
    from paged_kv_cache_102_amd.driver import PagedKV, replay_prefill
    from workloads import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n} bytes read, {n} bytes written")
        del src, dst
    steps, warm = args.steps, args.warmup
    w = synth.generate(WORKLOAD, extra_tokens=steps + warm + args.decode_only_steps + 1)
    s = w.spec
    log(f"[bench] {WORKLOAD}: B={s.num_seqs} Hq={s.num_q_heads} Hkv={s.num_kv_heads} "
        f"D={s.head_dim} pool={w.num_blocks} blocks, {int(w.lens.sum())} tokens")

    def to_dev(rows):
        return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(torch.bfloat16)

    kv = PagedKV(num_blocks=w.num_blocks, num_seqs=s.num_seqs,
                 max_blocks_per_seq=w.max_blocks_per_seq, num_q_heads=s.num_q_heads,
                 num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype=s.dtype, device=dev,
                 init_order=w.pool_order, partition_size=args.partition)
    replay_prefill(kv, w, to_dev)
    q = to_dev(w.q)
    k_new, v_new = to_dev(w.k_app), to_dev(w.v_app)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # paged vs contiguous: the same lengths and values with the blocks of
    # each sequence consecutive in the pool (identity free-list order), decode
    # alone, back to back
    paged_vs_contig = None
    if args.contiguous and args.decode_only_steps > 0:
        kc = PagedKV(num_blocks=w.num_blocks, num_seqs=s.num_seqs,
                     max_blocks_per_seq=w.max_blocks_per_seq, num_q_heads=s.num_q_heads,
                     num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype=s.dtype, device=dev,
                     init_order=None, partition_size=args.partition)
        replay_prefill(kc, w, to_dev)
        kv.decode(q, s.scale, out=out)
        kc.decode(q, s.scale, out=out)
        times = {}
        for name, obj in (("paged", kv), ("contiguous", kc)):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.decode_only_steps):
                obj.decode(q, s.scale, out=out)
            e1.record()
            torch.cuda.synchronize()
            times[name] = e0.elapsed_time(e1) / args.decode_only_steps
        paged_vs_contig = {"paged_ms": round(times["paged"], 4),
                           "contiguous_ms": round(times["contiguous"], 4),
                           "paged_overhead_pct": round(100 * (times["paged"] / times["contiguous"] - 1),
                                                       2),
                           "note": "after prefill, same lengths and values; contiguous = each "
                                   "sequence's blocks consecutive in the pool"}
        del kc
        torch.cuda.empty_cache()


    def step():
        kv.append(k_new, v_new)
        kv.decode(q, s.scale, out=out)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    # timed region: K whole steps
    bytes_total = 0
    capi.pkv_profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
        bytes_total += kv_bytes(kv.lens, s.num_kv_heads, s.head_dim)
    t_issued = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nlaunch, kern_ms = capi.pkv_profile_end()
    dt = t1 - t0
    ms_per_step = dt * 1e3 / steps
    value = bytes_total / dt / 1e9
    bytes_per_launch = bytes_total / steps
    avg_kernel_ms = kern_ms / max(nlaunch, 1)
    achieved = bytes_per_launch / (avg_kernel_ms * 1e-3) / 1e9

    # decode alone, back to back (no appends), for context
    dec = {}
    if args.decode_only_steps > 0:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.decode_only_steps):
            kv.decode(q, s.scale, out=out)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.decode_only_steps
        db = kv_bytes(kv.lens, s.num_kv_heads, s.head_dim)
        dec = {"ms": round(dms, 4), "kv_gb_per_s": round(db / dms / 1e6, 1),
               "frac_of_peak": round(db / dms / 1e6 / HBM_PEAK_GBS, 4)}

    # measured streaming-read ceiling on this GPU (2 GiB, 16-byte loads)
    ceiling = None
    if args.read_ceiling:
        buf = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
        capi.pkv_stream_read(buf, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            capi.pkv_stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        ceiling = buf.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del buf, sink

    fp8 = fp8_measure(dev, w) if args.fp8 else None
    prefill = None
    if args.prefill:
        torch.cuda.synchronize()
        prefill = prefill_measure(dev)

    traffic = committed_traffic()
    stats = capi.kv_pool_stats(kv.pool)
    waste = float(np.sum(-(-kv.lens // 16) * 16 - kv.lens) / np.sum(-(-kv.lens // 16) * 16))
    result = {
        "metric": "paged decode attn: effective KV GB/s & % of HBM peak; sequences/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "num_seqs": s.num_seqs, "num_q_heads": s.num_q_heads,
                   "num_kv_heads": s.num_kv_heads, "head_dim": s.head_dim, "block_size": 16,
                   "mean_context": round(float(kv.lens.mean()), 1),
                   "split": "balanced" if args.partition == 0 else f"{args.partition}-token partitions",
                   "parallelism": "single-gpu"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(s.num_seqs * steps / dt, 1),
        "decode_only": dec,
        "host_issue_ms_per_step": round((t_issued - t0) * 1e3 / steps, 4),
        "kv_waste_fraction": round(waste, 5),
        "pool_usage_percent": round(stats["usage_percent"], 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": kernel_name(args.partition),
                     "avg_launch_ms": round(avg_kernel_ms, 5), "launches": nlaunch,
                     "algorithmic_bytes_per_launch": int(bytes_per_launch)},
        "paged_vs_contiguous": paged_vs_contig,
        "prefill_chunked": prefill,
        "fp8_decode": fp8,
        "hbm_read_ceiling_gbs": round(ceiling, 1) if ceiling else None,
        "decode_frac_of_read_ceiling": round(achieved / ceiling, 4) if ceiling else None,
    }
    if args.all_configs:
        del kv
        torch.cuda.empty_cache()
        all_configs(args.all_configs, dev)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(w)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
