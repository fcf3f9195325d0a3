"""Benchmark of the paged decode step on one MI355X.

A step is one pass of the whole hot path for a batch of sequences, each
gaining one token:
  host slot planning + block allocation (C++), the step's small inputs
  (slots, table and length deltas, copy-on-write pairs) staged in pinned
  host memory and read in place by the kernels, block-table deltas,
  copy-on-write copies (when a shared block is hit), the K/V write, and
  decode attention (balanced split + log-sum-exp merges inside the launch).
Contexts grow by one token per step, exactly as in serving.

Headline workload: gqa-8b-bf16 -- 256 sequences, 32 query / 8 kv heads,
head_dim 128, bf16 cache, log-normal lengths (median 1000, sigma 1, clipped
to [16, 8192], one sequence at 273), scattered 16-token blocks.

Prints ONE JSON line.  value = effective KV GB/s of the whole step (K+V
bytes the decode reads / step time); roofline = the decode main kernel's
own average duration (HIP events recorded by the library on the kernel's
stream) against 8 TB/s; configs = every workload of the configs table at
full size (decode with cold caches, decode back to back, whole steps);
cpu_baseline = the CPU oracle timed on this host, on one core and on all
cores, per workload (a bounded sample of each).
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
FUSED_WARM = 3      # untimed one-launch steps before they are timed
PROFILE_EVERY = 5   # decode launches timed with events: one in five of the timed steps
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_bf16_cu_gqa-8b_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(names=("kernels.hip", "device_common.h")) -> str:
    """Hash of the code kernels are built from (by default the decode
    kernels'; the prefill's are prefill.hip and device_common.h): the sources
    with comments removed and whitespace runs collapsed (a change of wording
    in a comment leaves the kernels, and their counters, as they were)."""
    h = hashlib.sha256()
    for name in names:
        text = open(os.path.join(ROOT, "paged_kv_cache_102_amd", "csrc", name)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


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


# The five workloads of the configs table, each measured at full size in the
# default run; gqa-8b-bf16 is also the headline step above.
CONFIG_KEYS = ("tiny-fp32", "mha-7b-bf16", "gqa-8b-bf16", "long-70b-bf16", "shared-prefix-bf16")
# bounded CPU samples of each workload: every k-th sequence (all of tiny)
CPU_SAMPLE_STRIDE = {"tiny-fp32": 1, "mha-7b-bf16": 4, "gqa-8b-bf16": 4, "long-70b-bf16": 2,
                     "shared-prefix-bf16": 4}
FLUSH_BYTES = 1 << 30   # written between cold launches: more than L2 + the 256 MB MALL


def unique_kv_bytes(w, lens, elem) -> int:
    """K+V bytes of distinct cached tokens: a shared prefix counts once."""
    s = w.spec
    toks = int(lens.astype("int64").sum())
    if s.prefix_len:
        toks -= (s.num_seqs - 1) * s.prefix_len
    return toks * 2 * s.num_kv_heads * s.head_dim * elem


def config_measure(dev, key: str, flush, cold: int = 30, b2b: int = 50, steps: int = 30,
                   warm: int = 5, partition: int = 0):
    """One workload at full size, three ways:
      decode_cold  -- median of ``cold`` single decode calls, each timed by
                      the library's events on the call's stream, with a
                      1 GiB buffer written before each (L2 and MALL evicted);
      decode_b2b   -- mean of ``b2b`` decode calls back to back;
      step         -- mean of ``steps`` whole steps (append one token per
                      sequence, then decode), timed on the host clock with
                      synchronizations around the loop, as the headline.
    Bytes: logical = every sequence's K+V; unique = distinct blocks' tokens
    (a shared prefix once), the bytes HBM has to deliver."""
    import numpy as np
    import torch
    from paged_kv_cache_102_amd import _capi as capi
    from paged_kv_cache_102_amd.driver import PagedKV, replay_prefill
    from workloads import synth
    w = synth.generate(key, extra_tokens=steps + warm + 2)
    s = w.spec
    elem = 4 if s.dtype == "f32" else 2

    def to_dev(rows):
        if s.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(rows)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(
            torch.bfloat16)
    kv = PagedKV(num_blocks=w.num_blocks, num_seqs=s.num_seqs,
                 max_blocks_per_seq=w.max_blocks_per_seq, num_q_heads=s.num_q_heads,
                 num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype=s.dtype, device=dev,
                 init_order=w.pool_order, partition_size=partition)
    replay_prefill(kv, w, to_dev)
    q = to_dev(w.q)
    ones = np.ones(s.num_seqs, np.int32)
    k1, v1 = to_dev(w.k_app[:s.num_seqs]), to_dev(w.v_app[:s.num_seqs])
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    for _ in range(3):
        kv.decode(q, s.scale, out=out)
    torch.cuda.synchronize()
    logical = kv_bytes(kv.lens, s.num_kv_heads, s.head_dim, elem)
    unique = unique_kv_bytes(w, kv.lens, elem)
    # cold single calls
    capi.pkv_profile_begin(1)
    for i in range(cold):
        flush.fill_(float(i & 7))
        kv.decode(q, s.scale, out=out)
    each = capi.pkv_profile_durations()
    capi.pkv_profile_end()
    cold_ms = float(np.median(each))
    # back to back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(b2b):
        kv.decode(q, s.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    b2b_ms = e0.elapsed_time(e1) / b2b

    # whole steps (the contexts grow by one token per step)
    def step():
        kv.append(k1, v1, ones)
        kv.decode(q, s.scale, out=out)
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    step_bytes = 0
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
        step_bytes += kv_bytes(kv.lens, s.num_kv_heads, s.head_dim, elem)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_logical = step_bytes / steps
    step_unique = step_logical - (logical - unique)
    gbs = lambda b, ms: round(b / ms / 1e6, 1)
    frac = lambda b, ms: round(b / ms / 1e6 / HBM_PEAK_GBS, 4)
    res = {"num_seqs": s.num_seqs, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
           "head_dim": s.head_dim, "kv_dtype": s.dtype,
           "mean_context": round(float(kv.lens.mean()) - steps - warm, 1),
           "split": (f"{partition}-token partitions + log-sum-exp reduce" if partition else
                     "512-token partitions + reduce (fp32 default)" if s.dtype == "f32" else
                     "balanced per-CU"),
           "logical_kv_bytes": logical, "unique_kv_bytes": unique,
           "decode_cold_ms": round(cold_ms, 4), "decode_b2b_ms": round(b2b_ms, 4),
           "step_ms": round(step_ms, 4),
           "decode_cold_gb_per_s": gbs(logical, cold_ms),
           "decode_cold_frac_of_hbm_peak": frac(unique, cold_ms),
           "decode_b2b_gb_per_s": gbs(logical, b2b_ms),
           "decode_b2b_frac_of_hbm_peak": frac(unique, b2b_ms),
           "step_gb_per_s": gbs(step_logical, step_ms),
           "step_frac_of_hbm_peak": frac(step_unique, step_ms),
           "decode_seqs_per_s": round(s.num_seqs / cold_ms * 1e3, 1),
           "step_seqs_per_s": round(s.num_seqs / step_ms * 1e3, 1)}
    if s.dtype == "f32":
        res["decode_cold_latency_us"] = round(cold_ms * 1e3, 2)
        res["step_latency_us"] = round(step_ms * 1e3, 2)
        res["note"] = "launch- and latency-bound at this size; the rates are context only"
    if s.prefix_len:
        res["note"] = ("logical bytes read the shared prefix once per sequence (served from "
                       "L2 / MALL after the first reads); frac_of_hbm_peak counts unique bytes")
    del kv, q, out
    torch.cuda.empty_cache()
    return res


def configs_measure(dev):
    """Every workload of the configs table at full size (config_measure),
    plus the long-context one with the split it is specified with."""
    import torch
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    res = {}
    for key in CONFIG_KEYS:
        log(f"[bench] config {key} ...")
        res[key] = config_measure(dev, key, flush)
        log(f"[bench] {key}: {res[key]}")
    log("[bench] gqa-8b shape at 512 sequences ...")
    res["gqa-8b-bf16-b512"] = config_measure(dev, "gqa-8b-bf16-b512", flush)
    log("[bench] config long-70b-bf16, 512-token partitions ...")
    res["long-70b-bf16/partitions-512"] = config_measure(dev, "long-70b-bf16", flush,
                                                         partition=512)
    del flush
    torch.cuda.empty_cache()
    return res


_CPU_STATE = None   # the oracle state the forked workers of cpu_child read


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    global _CPU_LIMIT
    _CPU_LIMIT = threadpool_limits(1)   # one BLAS thread per worker process


def _cpu_worker(seqs):
    from oracle import attention
    w, st = _CPU_STATE
    s = w.spec
    out = attention.decode(w.q, st.cache, st.tables, st.lens, s.num_q_heads, s.num_kv_heads,
                           s.scale, seqs=seqs)
    return seqs, out[seqs]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_child(seconds: float):
    """The oracle, as it stands, on this host's cores: for every workload, a
    bounded sample (every k-th sequence, CPU_SAMPLE_STRIDE) replayed on the
    oracle, then its decode timed (a) on one core (BLAS limited to one
    thread) and (b) on all cores of this process's affinity (at most 16, the
    host share of one GPU): a fork pool of that many single-threaded
    workers, each decoding a share of the sequences.  Runs in a process of
    its own that never touches the GPU.  Prints one JSON line."""
    import multiprocessing
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention, replay
    from workloads import synth
    global _CPU_STATE
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    res = {}
    for key in CONFIG_KEYS:
        w = synth.generate(key)
        k = CPU_SAMPLE_STRIDE[key]
        sub = synth.subset(w, range(0, w.spec.num_seqs, k), seed=77) if k > 1 else w
        del w
        st = replay.prefill(sub)
        s = sub.spec
        elem = 4 if s.dtype == "f32" else 2
        nbytes = kv_bytes(st.lens, s.num_kv_heads, s.head_dim, elem)
        B = s.num_seqs
        with threadpool_limits(1):
            reps, t0 = 0, time.perf_counter()
            while True:
                attention.decode(sub.q, st.cache, st.tables, st.lens, s.num_q_heads,
                                 s.num_kv_heads, s.scale)
                reps += 1
                if time.perf_counter() - t0 >= seconds or reps >= 200:
                    break
            one = time.perf_counter() - t0
        _CPU_STATE = (sub, st)
        n = min(cores, B)
        parts = [list(range(i, B, n)) for i in range(n)]
        with multiprocessing.get_context("fork").Pool(n, initializer=_cpu_worker_init) as pool:
            pool.map(_cpu_worker, parts)          # warm the workers
            reps_all, t0 = 0, time.perf_counter()
            while True:
                pool.map(_cpu_worker, parts)
                reps_all += 1
                if time.perf_counter() - t0 >= seconds or reps_all >= 400:
                    break
            allc = time.perf_counter() - t0
        _CPU_STATE = None
        res[key] = {"sample": f"{B} of {B * k} sequences (one in {k})"
                              if k > 1 else f"all {B} sequences",
                    "kv_bytes": nbytes,
                    "one_core": {"gb_per_s": round(nbytes * reps / one / 1e9, 4),
                                 "seqs_per_s": round(B * reps / one, 2), "passes": reps,
                                 "seconds": round(one, 2)},
                    "all_cores": {"cores": n, "gb_per_s": round(nbytes * reps_all / allc / 1e9, 4),
                                  "seqs_per_s": round(B * reps_all / allc, 2),
                                  "passes": reps_all, "seconds": round(allc, 2)}}
        log(f"[cpu] {key}: {res[key]}")
        del sub, st
    print(json.dumps({"cores": cores, "cpu_model": cpu_model(), "configs": res}), flush=True)


def cpu_baseline(seconds: float = 3.0):
    """Runs cpu_child in a fresh interpreter (this process has the GPU open)
    and shapes its result: value = the headline workload on all cores."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child",
                        str(seconds)], capture_output=True, text=True)
    sys.stderr.write(r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"CPU baseline child failed ({r.returncode})")
    d = json.loads(r.stdout.strip().splitlines()[-1])
    head = d["configs"][WORKLOAD]
    return {"value": head["all_cores"]["gb_per_s"], "unit": "GB/s",
            "cores": head["all_cores"]["cores"], "kind": "oracle",
            "sample": f"{WORKLOAD}: {head['sample']} at their prefill lengths, numpy float64 "
                      f"decode, {head['all_cores']['passes']} passes over "
                      f"{head['all_cores']['seconds']} s on a pool of "
                      f"{head['all_cores']['cores']} single-threaded processes",
            "seqs_per_s": head["all_cores"]["seqs_per_s"],
            "one_core": head["one_core"], "cpu_model": d["cpu_model"],
            "host_cores_available": d["cores"], "per_config": d["configs"]}


BF16_MFMA_PEAK_TFLOPS = 2500.0


def prefill_measure(dev, reps: int = 20, cache: str = "bf16"):
    """Multi-query (chunked prefill) attention: 8 sequences of the gqa-8b
    shape with 1024..2048 cached tokens each take a 512-token chunk, causal
    inside the chunk, over a bf16 or an FP8 (E4M3, tensor scales) cache.
    Returns the kernel time and its rate against the bf16 matrix-core peak
    (4 * D flops per (query row, attended token); Q.K^T runs on bf16 and
    P.V on f16 operands, 16-bit products priced at the same peak)."""
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
                 num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype=cache, device=dev,
                 init_order=w.pool_order, k_scale=6.0 / 448, v_scale=6.0 / 448)
    replay_prefill(kv, w, to_dev)
    kv.append(to_dev(w.k_app), to_dev(w.v_app), w.append_counts)
    T = n * s.num_seqs
    q = torch.randn((T, s.num_q_heads, s.head_dim), device=dev).to(torch.bfloat16)
    # chunk row offsets uploaded once: the timed calls are the kernel alone
    qstart = torch.arange(0, T + 1, n, dtype=torch.int32, device=dev)
    out = torch.empty((T, s.num_q_heads, s.head_dim), dtype=torch.float32, device=dev)
    for _ in range(3):
        kv.prefill_attention(q, qstart, s.scale, out=out, max_query_len=n)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kv.prefill_attention(q, qstart, s.scale, out=out, max_query_len=n)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    lens = kv.lens.astype(np.int64)
    attended = int(sum(int(L) * n - n * (n - 1) // 2 for L in lens))   # sum over rows of (p + 1)
    flops = 4.0 * s.head_dim * s.num_q_heads * attended
    kv_unique = int(lens.sum()) * 2 * s.num_kv_heads * s.head_dim * (1 if cache == "fp8" else 2)
    tflops = flops / (ms * 1e-3) / 1e12
    f8 = cache == "fp8"
    return {"workload": "8 sequences x 512-token chunks on 1024..2048 cached tokens, 32 q / 8 kv heads, "
                        "head_dim 128, " + ("FP8 E4M3 cache" if f8 else "bf16"),
            "kernel": f"prefill_bf16_kernel<128,false,4{',F8' if f8 else ''}> (8 wavefronts, 256 score "
                      "columns, 4-block K/V stages in three LDS buffers, the next stage's scores issued "
                      "among this stage's exponentials, P.V on f16" + (", codes expanded on the way in)"
                                                            if f8 else ")"),
            "ms": round(ms, 4),
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


def window_measure(dev, kv, q, scale, windows=(4096, 1024), reps: int = 30):
    """Sliding-window decode on the headline batch: for each window W, time
    decode alone (kernel reads only positions max(0, L - W) .. L - 1 of each
    sequence, from the block holding the window start), then release the
    blocks wholly before every window and count them.  Windows go from wide
    to narrow, so each release only adds to the previous one."""
    import numpy as np
    import torch
    from paged_kv_cache_102_amd import _capi as capi
    s_kv, D = kv.num_kv_heads, kv.head_dim
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    used0 = capi.kv_pool_stats(kv.pool)["num_used"]
    res = []
    for W in windows:
        kv.window = W
        for _ in range(5):
            kv.decode(q, scale, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            kv.decode(q, scale, out=out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        lens = kv.lens.astype(np.int64)
        lo = np.maximum(lens - W, 0)
        tile_lo = lo // 16 * 16                      # the kernel streams whole blocks
        attended = int((lens - lo).sum()) * 2 * s_kv * D * 2
        streamed = int((lens - tile_lo).sum()) * 2 * s_kv * D * 2
        upd = capi.pkv_window_release(kv.pool, kv.tables, kv.lens, W)
        if len(upd):
            capi.paged_block_table_update(kv.tables_d, torch.from_numpy(upd).to(dev))
        used = capi.kv_pool_stats(kv.pool)["num_used"]
        res.append({"window": W, "ms": round(ms, 4), "attended_kv_bytes": attended,
                    "kv_gb_per_s": round(streamed / ms / 1e6, 1),
                    "frac_of_hbm_peak": round(streamed / ms / 1e6 / HBM_PEAK_GBS, 4),
                    "blocks_in_use_after_release": int(used),
                    "blocks_released_frac": round(1 - used / used0, 4)})
    kv.window = 0
    return {"workload": f"{WORKLOAD} batch after the timed steps; kv_gb_per_s counts the "
                        "window's blocks (from the one holding the window start)",
            "results": res}


def swap_measure(dev, kv, frac: float = 0.5, reps: int = 5):
    """Block swap of about ``frac`` of the batch's blocks: the copy kernel
    (paged_kv_swap_blocks) device -> pinned host and back, each timed with
    events on its stream, beside a plain DMA copy of the same byte count
    between the same kinds of memory (torch copy_, one contiguous run)."""
    import numpy as np
    import torch
    from paged_kv_cache_102_amd import _capi as capi
    order = np.argsort(-kv.lens)
    n_tot = int(np.sum(-(-kv.lens // 16)))
    pick, nb = [], 0
    for b in order:
        if nb >= frac * n_tot:
            break
        pick.append(int(b))
        nb += -(-int(kv.lens[b]) // 16)
    ids = np.concatenate([kv.tables[b, :-(-int(kv.lens[b]) // 16)] for b in pick])
    ids = ids[ids >= 0]
    NH = len(ids)
    per_block = kv.num_kv_heads * 16 * kv.head_dim
    hk = torch.empty(NH * per_block, dtype=kv.k_cache.dtype, pin_memory=True)
    hv = torch.empty(NH * per_block, dtype=kv.v_cache.dtype, pin_memory=True)
    # host planning cost, on a pool pair of the same sizes (the batch's own
    # pool keeps its state: the copies below move its blocks' data to host
    # slots 0..NH-1 and back onto the same blocks)
    gp, hpool = capi.pkv_pool_create(kv.num_blocks, 16), capi.pkv_pool_create(NH, 16)
    held = capi.kv_block_alloc(gp, NH)
    t0 = time.perf_counter()
    capi.kv_block_swap(gp, hpool, held)
    plan_ms = (time.perf_counter() - t0) * 1e3
    pairs = np.stack([ids, np.arange(NH)], axis=1).astype(np.int32)
    d_pairs = torch.from_numpy(pairs).to(dev)
    back_pairs = torch.from_numpy(np.ascontiguousarray(pairs[:, ::-1])).to(dev)
    st = torch.cuda.current_stream(dev)
    nbytes = 2 * len(pairs) * per_block * kv.k_cache.element_size()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out_ms = timed(lambda: capi.paged_kv_swap_blocks(kv.k_cache, kv.v_cache, hk, hv, d_pairs,
                                                     kv.num_kv_heads, kv.head_dim, kv.num_blocks,
                                                     NH, st.cuda_stream))
    in_ms = timed(lambda: capi.paged_kv_swap_blocks(hk, hv, kv.k_cache, kv.v_cache, back_pairs,
                                                    kv.num_kv_heads, kv.head_dim, NH,
                                                    kv.num_blocks, st.cuda_stream))
    # DMA of the same bytes: device <-> pinned host, one run each way
    dsrc = kv.k_cache[:nbytes // 2 // kv.k_cache.element_size()]
    hdst = hk[:dsrc.numel()]
    d2h_ms = timed(lambda: (hdst.copy_(dsrc, non_blocking=True), hv[:dsrc.numel()].copy_(
        kv.v_cache[:dsrc.numel()], non_blocking=True)))
    kscratch = torch.empty_like(dsrc)
    vscratch = torch.empty_like(dsrc)
    h2d_ms = timed(lambda: (kscratch.copy_(hdst, non_blocking=True),
                            vscratch.copy_(hv[:dsrc.numel()], non_blocking=True)))
    del hk, hv, kscratch, vscratch
    gbs = lambda ms: round(nbytes / ms / 1e6, 1)
    return {"workload": f"{len(pick)} longest sequences of the {WORKLOAD} batch, "
                        f"{len(pairs)} blocks, K and V",
            "bytes": nbytes, "plan_ms": round(plan_ms, 3),
            "swap_out_ms": round(out_ms, 3), "swap_out_gb_per_s": gbs(out_ms),
            "swap_in_ms": round(in_ms, 3), "swap_in_gb_per_s": gbs(in_ms),
            "dma_d2h_gb_per_s": gbs(d2h_ms), "dma_h2d_gb_per_s": gbs(h2d_ms),
            "out_frac_of_dma": round(d2h_ms / out_ms, 3), "in_frac_of_dma": round(h2d_ms / in_ms, 3),
            "round_trip_ms_per_4gb": round((out_ms + in_ms) * 4e9 / nbytes, 1)}


def prefix_measure(num_requests: int = 128, prefix_tokens: int = 2048, suffix_max: int = 256):
    """Prefix caching on the host: requests sharing a 2048-token system
    prompt, each with its own suffix.  The first request's blocks are
    registered; every later one matches them (longest indexed prefix), takes
    fresh blocks for the rest and registers its own.  Reports the host cost
    per request and the share of blocks (and KV writes) that reuse saves."""
    import numpy as np
    from paged_kv_cache_102_amd import _capi as capi
    rng = np.random.default_rng(55)
    system = rng.integers(0, 32000, size=prefix_tokens).astype(np.int32)
    reqs = [np.concatenate([system, rng.integers(0, 32000, size=int(rng.integers(1, suffix_max)))])
            .astype(np.int32) for _ in range(num_requests)]
    need = sum(-(-len(r) // 16) for r in reqs)
    pool = capi.pkv_pool_create(need, 16)
    capi.pkv_prefix_cache_enable(pool)
    t_match = t_reg = 0.0
    reused = 0
    for r in reqs:
        t0 = time.perf_counter()
        got = capi.pkv_prefix_match(pool, r)
        t1 = time.perf_counter()
        fresh = capi.kv_block_alloc(pool, -(-len(r) // 16) - len(got))
        t2 = time.perf_counter()
        capi.pkv_prefix_register(pool, r, np.concatenate([got, fresh]).astype(np.int32))
        t3 = time.perf_counter()
        t_match += t1 - t0
        t_reg += t3 - t2
        reused += len(got)
    return {"workload": f"{num_requests} requests, {prefix_tokens}-token shared prompt + "
                        f"1..{suffix_max - 1} own tokens",
            "match_us_per_request": round(t_match / num_requests * 1e6, 2),
            "register_us_per_request": round(t_reg / num_requests * 1e6, 2),
            "blocks_reused_frac": round(reused / need, 4),
            "blocks_in_use": int(capi.kv_pool_stats(pool)["num_used"]),
            "blocks_without_reuse": need}


def kv_bytes(lens, num_kv_heads, head_dim, elem=2) -> int:
    return int(lens.astype("int64").sum()) * 2 * num_kv_heads * head_dim * elem


def paged_vs_contiguous(dev, w, q, out, reps: int):
    """Decode alone, back to back, on two fresh pools with the workload's
    prefill state: the same lengths and values, once in the workload's
    scattered block order and once with each sequence's blocks consecutive
    (identity free-list order).  Runs after the timed steps: building and
    freeing two more pools before them slowed those steps by ~3 %."""
    import torch
    from paged_kv_cache_102_amd.driver import PagedKV, replay_prefill
    import numpy as np
    s = w.spec

    def to_dev(rows):
        return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).to(dev).view(torch.bfloat16)
    times = {}
    for name, order in (("paged", w.pool_order), ("contiguous", None)):
        obj = PagedKV(num_blocks=w.num_blocks, num_seqs=s.num_seqs,
                      max_blocks_per_seq=w.max_blocks_per_seq, num_q_heads=s.num_q_heads,
                      num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, dtype=s.dtype, device=dev,
                      init_order=order)
        replay_prefill(obj, w, to_dev)
        obj.decode(q, s.scale, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            obj.decode(q, s.scale, out=out)
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / reps
        del obj
        torch.cuda.empty_cache()
    return {"paged_ms": round(times["paged"], 4), "contiguous_ms": round(times["contiguous"], 4),
            "paged_overhead_pct": round(100 * (times["paged"] / times["contiguous"] - 1), 2),
            "note": "fresh pools after prefill, same lengths and values; contiguous = each "
                    "sequence's blocks consecutive in the pool"}


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
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="skip the sliding-window, swap and prefix-cache measurements")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the per-workload measurements of every config")
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="seconds of oracle work per workload and core setting")
    ap.add_argument("--cpu-child", type=float, default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_child is not None:      # the CPU baseline's own process: no GPU
        cpu_child(args.cpu_child)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path "
              "runs on a single GPU.", file=sys.stderr)
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
    w = synth.generate(WORKLOAD, extra_tokens=steps + warm + FUSED_WARM + max(10, steps // 2) +
                       args.decode_only_steps + 1)
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

    def step():
        kv.append(k_new, v_new)
        kv.decode(q, s.scale, out=out)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    # timed region: K whole steps.  The library times decode launches 0,
    # PROFILE_EVERY, 2 PROFILE_EVERY, ... with HIP events on the step's
    # stream; each recorded pair adds two markers to its step.
    bytes_total = bytes_prof = 0
    capi.pkv_profile_begin(PROFILE_EVERY)
    torch.cuda.synchronize()
    wait0 = kv._staging.wait_s if kv._staging is not None else 0.0
    t0 = time.perf_counter()
    for i in range(steps):
        step()
        b = kv_bytes(kv.lens, s.num_kv_heads, s.head_dim)
        bytes_total += b
        if i % PROFILE_EVERY == 0:
            bytes_prof += b
    t_issued = time.perf_counter()
    host_wait = (kv._staging.wait_s if kv._staging is not None else 0.0) - wait0
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nlaunch, kern_ms = capi.pkv_profile_end()
    dt = t1 - t0
    ms_per_step = dt * 1e3 / steps
    value = bytes_total / dt / 1e9
    bytes_per_launch = bytes_prof / max(nlaunch, 1)   # of the timed launches
    avg_kernel_ms = kern_ms / max(nlaunch, 1)
    achieved = bytes_per_launch / (avg_kernel_ms * 1e-3) / 1e9

    # the same step in one launch (paged_kv_append_decode), for context
    fused = None
    if args.partition == 0 and args.decode_only_steps > 0:
        n2 = max(10, steps // 2)
        for _ in range(FUSED_WARM):   # the first launches of its kernel load its code
            kv.decode_step(q, k_new, v_new, s.scale, out=out)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(n2):
            kv.decode_step(q, k_new, v_new, s.scale, out=out)
        torch.cuda.synchronize()
        fms = (time.perf_counter() - t2) * 1e3 / n2
        fused = {"ms": round(fms, 4), "steps": n2,
                 "kv_gb_per_s": round(kv_bytes(kv.lens, s.num_kv_heads, s.head_dim) / fms / 1e6, 1),
                 "note": "one launch per step: the new tokens attended from their rows and written "
                         "at the end of the launch; timed after the headline steps"}

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

    # paged vs contiguous block placement, on fresh pools
    paged_vs_contig = None
    if args.contiguous and args.decode_only_steps > 0:
        paged_vs_contig = paged_vs_contiguous(dev, w, q, out, args.decode_only_steps)

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

    stats = capi.kv_pool_stats(kv.pool)
    waste = float(np.sum(-(-kv.lens // 16) * 16 - kv.lens) / np.sum(-(-kv.lens // 16) * 16))
    swap = window = prefix = None
    if args.extras:
        swap = swap_measure(dev, kv)
        window = window_measure(dev, kv, q, s.scale)   # releases blocks: after the rest
        prefix = prefix_measure()
    fp8 = fp8_measure(dev, w) if args.fp8 else None
    prefill = prefill_fp8 = None
    if args.prefill:
        torch.cuda.synchronize()
        prefill = prefill_measure(dev)
        prefill_fp8 = prefill_measure(dev, cache="fp8") if args.fp8 else None

    traffic = committed_traffic()
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
        "fused_step": fused,
        "host_issue_ms_per_step": round((t_issued - t0) * 1e3 / steps, 4),
        # of which the host waited for a staging buffer (the ring holds 16 steps'
        # inputs, so a host ahead of the GPU waits there); the rest is planning,
        # packing and the launches themselves
        "host_wait_ms_per_step": round(host_wait * 1e3 / steps, 4),
        "kv_waste_fraction": round(waste, 5),
        "pool_usage_percent": round(stats["usage_percent"], 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": kernel_name(args.partition),
                     "avg_launch_ms": round(avg_kernel_ms, 5), "launches": nlaunch,
                     "launches_sampled_every": PROFILE_EVERY,
                     "algorithmic_bytes_per_launch": int(bytes_per_launch)},
        "paged_vs_contiguous": paged_vs_contig,
        "prefill_chunked": prefill,
        "prefill_chunked_fp8": prefill_fp8,
        "fp8_decode": fp8,
        "sliding_window_decode": window,
        "block_swap": swap,
        "prefix_cache_host": prefix,
        "hbm_read_ceiling_gbs": round(ceiling, 1) if ceiling else None,
        "decode_frac_of_read_ceiling": round(achieved / ceiling, 4) if ceiling else None,
    }
    del kv
    torch.cuda.empty_cache()
    result["configs"] = configs_measure(dev) if args.configs else None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
