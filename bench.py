#!/usr/bin/env python3
"""Benchmark: one decode step of paged attention at the OPT-13B layer shape.

A step is the whole hot path for one batch: the host block manager's append
for every sequence (done ahead of the timed region; its inputs are resident
in HBM before timing starts), the copy-on-write block copies it asks for
(none in this workload), ``pa_reshape_and_cache`` of the 64 new tokens' K/V,
and ``pa_paged_decode``.

Workload: 64 sequences, 40 heads, head_dim 128, fp16 K/V/Q ~ N(0,1), scale
1/sqrt(128), block size 16, history lengths uniform on [1, 2048] drawn from
SeedSequence(76002), blocks taken from a seeded-shuffled pool sized to the
blocks needed + 10% (+ room for the steps' growth).  Step i decodes one new
token per sequence, so its contexts are the drawn lengths + i.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode-attn achieved HBM GB/s (% of peak) + seq-steps/s, OPT-13B shape"
PEAK_HBM_GBS = 8000.0
S, H, D, B = 64, 40, 128, 16
DTYPE = "f16"
ELEM = 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


SETTLE_MS = 60.0


def settle(launch, ms: float = SETTLE_MS) -> int:
    """Repeat ``launch`` (one read-only kernel launch) until ``ms`` of
    sustained GPU work have passed, right before a timed loop.  Measured on
    the MI355X: after an idle phase (building a workload on the host) the
    clocks take some 10-30 ms of load to reach their steady state (a 5 ms
    pass of shared-block decode steps ran at 82-84 us per step cold and at
    74 us after 30 ms of load), so a short timed loop would otherwise measure
    the ramp.  Returns the number of launches made."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            launch()
        torch.cuda.synchronize()
        n += 8
    log(f"clocks settled: {n} read-only launches over {ms:.0f} ms")
    return n


FLUSH_BYTES = 1 << 30


class CacheFlush:
    """Evicts the GPU's caches between timed launches: a plain read (a sum
    over int32 words, temporal loads) of 1 GiB, four times the MI355X's
    256 MB Infinity Cache and far more than the XCDs' L2s.  Reads allocate
    in the Infinity Cache (measured: such a pass also evicts lines a previous
    write left dirty), and the pass leaves no dirty lines of its own; a
    read-modify-write flush would, and their write-back would slow the timed
    launch (by ~5 us on a 75 us decode, measured).  A launch timed right
    after the pass reads its bytes from HBM, whatever the previous launch
    left cached."""

    def __init__(self):
        import torch

        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        self.sink = None

    def __call__(self) -> None:
        self.sink = self.buf.sum()


def flushed_replays(launch, n: int) -> list[float]:
    """Durations (ms) of launch(i) for i < n, each timed with events right
    after a cache flush."""
    import torch

    flush = CacheFlush()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for _ in range(20):   # keeps the clocks up after the host-side set-up
        flush()
    for i in range(n):
        flush()
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    del flush
    return [a.elapsed_time(b) for a, b in ev]


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


COUNTERS = os.path.join(ROOT, "profiles", "decode_opt13b_fp16_b16_counters.txt")
DECODE_SOURCES = ("paged_kv_cache_76_amd/csrc/paged_decode.hip", "paged_kv_cache_76_amd/csrc/pa_device.h")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_opt66b_bf16_8x1024_counters.txt")
PREFILL_SOURCES = ("paged_kv_cache_76_amd/csrc/paged_prefill.hip",)


def measured_traffic(path=COUNTERS, sources=DECODE_SOURCES, kernels=("decode_partition_kernel",
                                                                        "decode_reduce_kernel")) -> dict | None:
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (scaled by the copy-kernel calibration), summed over ``kernels``, and
    their ratio to the algorithmic bytes per launch of the same profiled run;
    None if the kernel sources changed since those counters were taken."""
    import hashlib

    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in sources:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != kv["kernel_source_sha256"]:
            return None
        fs, ws = float(kv["fetch_scale"]), float(kv["write_scale"])
        kib = sum(float(kv[f"{k}_fetch_kib"]) * fs + float(kv[f"{k}_write_kib"]) * ws for k in kernels)
        alg = float(kv["algorithmic_bytes_per_dispatch"])
        return {"bytes": round(kib * 1024.0), "ratio": round(kib * 1024.0 / alg, 4)}
    except (OSError, KeyError, ValueError):
        return None


def achievable_reads(cache, tables, lens, reps: int = 10) -> dict:
    """The achievable HBM read rates a decode step is measured against: a
    front-to-back stream over 2 GiB, and the (block, head) key and value tiles
    one decode step reads (the same tiles, in [sequence][head][block] order),
    read with no arithmetic.  Medians of `reps` timed launches."""
    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L

    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    H, B = cache.num_heads, cache.block_size
    tile_bytes = B * cache.head_dim * cache.k.element_size()
    ids = []
    for s, n in enumerate(lens):
        nb = -(-int(n) // B)
        ids.append((tables[s, :nb][None, :].astype(np.int64) * H + np.arange(H)[:, None]).reshape(-1))
    tiles = torch.from_numpy(np.concatenate(ids).astype(np.int32)).cuda()
    stream_bytes = 2 << 30
    buf = torch.empty(stream_bytes, dtype=torch.uint8, device="cuda")

    def timed(fn):
        # back-to-back launches with an event pair around each and one host
        # synchronisation at the end, as the decode's own launches are timed
        # (a synchronisation after every launch lets the GPU idle between
        # them, which measured 5 % slower on these reads)
        for _ in range(3):
            fn()
        evs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = [e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs]
        return sorted(ts)[len(ts) // 2]

    t_stream = timed(lambda: L.pa_read_stream(buf, sink))
    t_tiles = timed(lambda: (L.pa_read_tiles(cache.k, tile_bytes, tiles, sink),
                             L.pa_read_tiles(cache.v, tile_bytes, tiles, sink)))
    tile_total = 2 * tiles.numel() * tile_bytes
    del buf
    return {"stream_read_GBps": round(stream_bytes / t_stream / 1e9, 1),
            "kv_tile_read_GBps": round(tile_total / t_tiles / 1e9, 1),
            "kv_tile_bytes": tile_total, "tile_bytes": tile_bytes,
            "kernels": "pa_read_stream / pa_read_tiles (plain 16-byte non-temporal reads, no arithmetic)"}


def cpu_baseline(batch, n_seq: int, repeats: int = 10) -> dict:
    """The float64 oracle on the first ``n_seq`` sequences of the step (all
    heads), timed on this host's cores."""
    import numpy as np

    from oracle import attention as oa
    from paged_kv_cache_76_amd import workloads

    qs = [batch.q[s].numpy() for s in range(n_seq)]
    ks = [batch.k_hist[s].numpy() for s in range(n_seq)]
    vs = [batch.v_hist[s].numpy() for s in range(n_seq)]
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        for s in range(n_seq):
            oa.decode(qs[s], ks[s], vs[s], batch.scale)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    nbytes = workloads.decode_bytes(batch.lens[:n_seq], H, D, ELEM, B)
    # the same sample with the BLAS pool held to one thread (median of 3)
    from threadpoolctl import threadpool_limits

    times1 = []
    with threadpool_limits(limits=1):
        for _ in range(3):
            t0 = time.perf_counter()
            for s in range(n_seq):
                oa.decode(qs[s], ks[s], vs[s], batch.scale)
            times1.append(time.perf_counter() - t0)
    dt1 = sorted(times1)[1]
    # the reported value is the faster of the two runs, with the threads it used
    best, threads = (dt, blas_threads()) if dt < dt1 else (dt1, 1)
    return {
        "value": nbytes / best / 1e9, "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": f"{n_seq} of {S} sequences (all {H} heads, contexts {int(batch.lens[:n_seq].sum())} tokens), "
                  f"one decode step, float64 NumPy on a {os.cpu_count()}-core host ({cpu_model()}); "
                  f"median of {repeats} with {blas_threads()} BLAS threads, of 3 with 1",
        "seq_steps_per_s": n_seq / best, "seconds": best,
        "GBps_by_threads": {str(blas_threads()): nbytes / dt / 1e9, "1": nbytes / dt1 / 1e9},
    }


def copy_calibration(args) -> int:
    """pa_copy_blocks of 2048 (src, dst) pairs of OPT-13B blocks (40 heads x 16
    tokens x 128 x fp16 = 160 KiB per pool): 640 MiB read + 640 MiB written per
    launch.  Its HBM counters, divided by these known sizes, give the scale
    factors applied to the decode kernel's counters."""
    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L

    n, N = 2048, 4096
    cache = L.KVCache.empty(N, H, B, D, torch.float16)
    cache.k.fill_(1.0)
    cache.v.fill_(2.0)
    ids = np.random.default_rng(0).permutation(N)
    pairs = torch.from_numpy(np.stack([ids[:n], ids[n:]], axis=1).astype(np.int64)).cuda()
    for _ in range(args.warmup):
        L.pa_copy_blocks(cache, pairs)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        L.pa_copy_blocks(cache, pairs)
        b.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    moved = 2 * 2 * n * H * B * D * ELEM           # read + write, keys and values
    rec = {"metric": "pa_copy_blocks HBM GB/s (read + write), 2048 OPT-13B blocks", "value": round(moved / (avg_ms * 1e-3) / 1e9, 2),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": {"workload": "pa_copy_blocks calibration", "pairs": n, "bytes_read_per_launch": moved // 2,
                      "bytes_written_per_launch": moved // 2}}
    print(json.dumps(rec), flush=True)
    return 0


PEAK_BF16_TFLOPS = 2500.0


def gemm_ceiling(n: int = 8192, reps: int = 10) -> dict:
    """A measured dense bf16 ceiling: torch.matmul (hipBLASLt) of two
    contiguous n x n bf16 matrices, median of ``reps`` after warm-up."""
    import torch

    gen = torch.Generator(device="cuda").manual_seed(76005)
    a = torch.randn((n, n), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((n, n), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        torch.matmul(a, b, out=c)
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    del a, b, c
    return {"kernel": f"torch.matmul bf16 {n}x{n}x{n}", "tflops": round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)}


PREFILL_METRIC = "paged causal prefill TFLOP/s, OPT-66B shape (8 x 1024 tokens, 72 heads, d128, bf16)"


def prefill_measure(steps: int, warmup: int, cpu_sample: bool, gemm: bool = True) -> dict:
    """8 prompts x 1024 tokens, 72 heads, d=128, bf16, block 16 (OPT-66B
    layer shape): one step writes the prompts' K/V through their slots and runs
    the causal paged prefill.  Returns the launch figures, the roofline of the
    prefill kernel and (optionally) the float64 oracle on one sequence."""
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd import workloads

    S5, H5, L5 = 8, 72, 1024
    lens = [L5] * S5
    log(f"building OPT-66B prefill workload: {S5} x {L5} tokens, H={H5}, d={D}, bf16, B={B}")
    b = workloads.build_prefill_batch(5, lens, lens, H5, D, B, "bf16", nan_fill=False)
    h = workloads.host_histories(5, lens, H5, D, B, "bf16")
    k_all, v_all = h.k_all.cuda(), h.v_all.cuda()
    slots = torch.from_numpy(h.slots).cuda()
    out = torch.empty((S5 * L5, H5, D), dtype=torch.bfloat16, device="cuda")
    flops = workloads.prefill_flops(lens, lens, H5, D)
    pbytes = workloads.prefill_bytes(lens, lens, H5, D, 2, B)
    wbytes = 2 * 2 * S5 * L5 * H5 * D * 2
    n = steps + warmup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    L.pa_reshape_and_cache(b.cache, k_all, v_all, slots)
    settle(lambda: L.pa_paged_prefill(b.cache, out, b.q_dev, b.tables_dev, b.cu_q_dev, b.lens_dev, L5, L5, b.scale))
    for i in range(n):
        if i == warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        ev[i][0].record()
        L.pa_reshape_and_cache(b.cache, k_all, v_all, slots)
        ev[i][1].record()
        L.pa_paged_prefill(b.cache, out, b.q_dev, b.tables_dev, b.cu_q_dev, b.lens_dev, L5, L5, b.scale)
        ev[i][2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    K = steps
    w_ms = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(warmup, n)) / K
    p_all = sorted(ev[i][1].elapsed_time(ev[i][2]) for i in range(warmup, n))
    p_ms = sum(p_all) / K
    p_pct = [round(p_all[min(K - 1, int(q * K))] * 1e3, 2) for q in (0.1, 0.5, 0.9)]
    tflops = flops / (p_ms * 1e-3) / 1e12
    log(f"prefill {p_ms * 1e3:.1f} us -> {tflops:.1f} TFLOP/s; write {w_ms * 1e3:.1f} us -> "
        f"{wbytes / (w_ms * 1e-3) / 1e9:.0f} GB/s")
    ceiling = None
    if gemm:
        ceiling = gemm_ceiling()
        log(f"dense bf16 GEMM ceiling on this GPU: {ceiling['tflops']:.0f} TFLOP/s")
    cpu = None
    if cpu_sample:
        # the float64 oracle on a bounded sample: sequence 0, all heads, every query
        from oracle import attention as oa

        qh = b.q[:L5].to(torch.float64).numpy()
        kh = b.k_hist[0].to(torch.float64).numpy()
        vh = b.v_hist[0].to(torch.float64).numpy()
        times = []
        for _ in range(3):
            t1 = time.perf_counter()
            oa.prefill(qh, kh, vh, b.scale)
            times.append(time.perf_counter() - t1)
        dt = sorted(times)[1]
        sample_flops = workloads.prefill_flops([L5], [L5], H5, D)
        cpu = {"value": sample_flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"sequence 0 of {S5} (all {H5} heads, {L5} causal queries), median of 3, float64 NumPy on "
                         f"{os.cpu_count()} host cores ({cpu_model()})", "seconds": dt}
        log(f"cpu oracle sample: {dt:.2f} s -> {cpu['value'] * 1e3:.3f} GFLOP/s")
    traffic = measured_traffic(PREFILL_COUNTERS, PREFILL_SOURCES, ("prefill_kernel",))
    # arithmetic intensity flops / bytes ~ 256 is below the ridge 2.5 PFLOP/s / 8 TB/s = 312.5, so the
    # binding roof at the published peaks is HBM (attainable 256 x 8 TB/s = 2.05 PFLOP/s); the MFMA
    # view of the same launch is given beside it
    roof = {"bound": "hbm", "kernel": "pa_paged_prefill",
            "achieved": round(pbytes / (p_ms * 1e-3) / 1e9, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(pbytes / (p_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": traffic and traffic["bytes"], "traffic_over_algorithmic": traffic and traffic["ratio"],
            "avg_launch_us": round(p_ms * 1e3, 2), "launch_us_p10_p50_p90": p_pct,
            "algorithmic_bytes_per_launch": pbytes,
            "arithmetic_intensity": round(flops / pbytes, 1),
            "ridge": round(PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
            "mfma": {"achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "algorithmic_flops_per_launch": flops}}
    return {"tflops": tflops, "elapsed": elapsed, "steps": K, "warmup": warmup, "roofline": roof,
            "gemm_ceiling": ceiling and dict(ceiling, pct_achieved=round(100 * tflops / ceiling["tflops"], 2)),
            "write": {"kernel": "pa_reshape_and_cache", "avg_launch_us": round(w_ms * 1e3, 2),
                      "achieved_GBps": round(wbytes / (w_ms * 1e-3) / 1e9, 1), "bytes_per_launch": wbytes},
            "cpu_baseline": cpu,
            "config": {"workload": "paged prefill step (prompt write + causal prefill)", "prompts": S5,
                       "prompt_len": L5, "heads": H5, "head_dim": D, "block_size": B,
                       "seed": "SeedSequence(76005)"}}


def prefill_bench(args) -> int:
    m = prefill_measure(args.steps, args.warmup, args.cpu_seqs > 0)
    K = m["steps"]
    rec = {"metric": PREFILL_METRIC, "value": round(m["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": round(m["elapsed"] / K * 1e3, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": m["config"],
           "roofline": m["roofline"], "gemm_ceiling": m["gemm_ceiling"], "write": m["write"],
           "cpu_baseline": m["cpu_baseline"]}
    print(json.dumps(rec), flush=True)
    return 0


def _line(metric, value, unit, steps, warmup, ms_per_step, dtype, config, **extra) -> None:
    rec = {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": steps,
           "warmup": warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config}
    rec.update(extra)
    print(json.dumps(rec), flush=True)


SERVING_METRIC = "paged serving-loop decode seq-steps/s, OPT-13B shape (256 seqs, 32 steps)"


def serving_measure(bs: int, steps: int = 32, wall_pass: bool = True,
                    fused: bool = False) -> tuple[float, float, dict, dict]:
    """``steps`` consecutive steps of a 256-sequence serving loop at the OPT-13B
    shape (fp16), block size ``bs``.  The host block-manager work of all
    steps runs first (timed on its own); the device loop then runs from
    inputs already in HBM.  With ``wall_pass``, a second, interleaved pass
    (host step -> pinned upload -> kernels, every step) gives the wall time
    per step.  ``fused``: the decode launch writes the new tokens
    (pa_paged_decode_append) instead of a pa_reshape_and_cache launch.
    Returns (seq-steps/s, ms per step, config, extra keys)."""
    import torch

    from paged_kv_cache_76_amd import workloads
    from paged_kv_cache_76_amd.serving import ServingLoop, opt13b_serving_lengths

    prompt, out, start = opt13b_serving_lengths(3, 256)
    log(f"serving loop: 256 seqs, B={bs}, fused={fused}")
    # device pass: every step's plan made ahead and resident in HBM
    loop = ServingLoop(3, prompt, out, start, H, D, bs, DTYPE, keep_history=False, fused=fused)
    counts = loop.active_counts(steps)
    toks = [loop.tokens(n, "cuda") for n in counts]
    prepared = []
    for t in range(steps):
        rows = loop.active_rows()
        assert len(rows) == counts[t]
        host, lens = loop.plan(rows)
        loop.finish(rows)
        prepared.append((rows, {k: v.cuda() for k, v in host.items()}, lens))
    bm_ms = loop.bm_seconds / steps * 1e3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    from paged_kv_cache_76_amd import _lib as L
    outs = torch.empty((256, H, D), dtype=torch.float16, device="cuda")
    # one untimed decode of step 0's inputs (read-only): the first launch of
    # a kernel in the process loads its code object (~2 ms), which must not
    # land inside the timed steps
    # (a fused loop's warm-up is step 0's appending decode: it stores step
    # 0's tokens early, into slots no row reads yet; step 0 stores them again)
    rows0, dev0, lens0 = prepared[0]
    if fused:
        L.pa_paged_decode_append(loop.cache, outs[: len(rows0)], toks[0][2], toks[0][0], toks[0][1],
                                 dev0["tables"], dev0["lens"], int(lens0.max()), loop.scale, 1, loop.ws)
    else:
        L.pa_paged_decode(loop.cache, outs[: len(rows0)], toks[0][2], dev0["tables"], dev0["lens"],
                          int(lens0.max()), loop.scale, loop.ws)
    # (then step 0's plain decode, read-only, until the clocks have settled)
    settle(lambda: L.pa_paged_decode(loop.cache, outs[: len(rows0)], toks[0][2], dev0["tables"], dev0["lens"],
                                     int(lens0.max()), loop.scale, loop.ws))
    t0 = time.perf_counter()
    for i, (rows, dev, lens) in enumerate(prepared):
        k, v, q = toks[i]
        ev[i][0].record()
        if dev["pairs"].shape[0]:
            L.pa_copy_blocks(loop.cache, dev["pairs"])
        if fused:
            L.pa_paged_decode_append(loop.cache, outs[: len(rows)], q, k, v, dev["tables"], dev["lens"],
                                     int(lens.max()), loop.scale, 1, loop.ws)
        else:
            L.pa_reshape_and_cache(loop.cache, k, v, dev["slots"])
            L.pa_paged_decode(loop.cache, outs[: len(rows)], q, dev["tables"], dev["lens"],
                              int(lens.max()), loop.scale, loop.ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    gpu_s = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    seq_steps = sum(len(r) for r, _, _ in prepared)
    nbytes = sum(workloads.decode_bytes(lens, H, D, ELEM, bs) + 4 * len(rows) * H * D * ELEM
                 for rows, _, lens in prepared)
    # tail waste (allocated but unused slots) averaged over the steps' batches
    waste = [int(sum(-(-int(x) // bs) * bs - int(x) for x in lens)) for _, _, lens in prepared]
    used = [int(sum(int(x) for x in lens)) for _, _, lens in prepared]
    stats = loop.mgr.stats()
    finished = 256 - len(loop.active_rows())
    del loop, prepared
    extra = {}
    if wall_pass:
        # interleaved pass: block-manager step -> pinned upload of the plan ->
        # kernels, every step (activations already on the device, as a
        # model's projections would be)
        loop2 = ServingLoop(3, prompt, out, start, H, D, bs, DTYPE, keep_history=False, fused=fused)
        toks2 = [loop2.tokens(n, "cuda") for n in loop2.active_counts(steps)]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for t in range(steps):
            loop2.step(toks=toks2[t])
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t1
        del loop2, toks2
        extra["wall_ms_per_step_interleaved"] = round(wall_s / steps * 1e3, 3)
    kernel_s = sum(step_ms) * 1e-3
    config = {"workload": "serving loop (append, write, decode per step; finished sequences freed)",
              "sequences": 256, "heads": H, "head_dim": D, "block_size": bs,
              "step_launches": "copies, then pa_paged_decode_append" if fused
              else "copies, pa_reshape_and_cache, pa_paged_decode",
              "lengths": "prompt lognormal(160,1)<=1024, output lognormal(300,1), total<=2048, "
                         "uniform progress at step 0", "seed": "SeedSequence(76003)"}
    extra.update(achieved_GBps=round(nbytes / kernel_s / 1e9, 1),
                 pct_of_peak=round(100 * nbytes / kernel_s / 1e9 / PEAK_HBM_GBS, 2),
                 seq_steps=seq_steps, finished_in_loop=finished,
                 host_block_manager_ms_per_step=round(bm_ms, 3),
                 gpu_loop_wall_ms_per_step=round(gpu_s / steps * 1e3, 3),
                 tail_waste_slots_mean=round(sum(waste) / steps, 1),
                 tail_waste_pct_mean=round(100 * sum(waste) / (sum(waste) + sum(used)), 3),
                 tail_waste_slots_end=stats["tail_waste_slots"],
                 slot_utilisation_end=round(stats["slot_utilisation"], 4))
    return seq_steps / kernel_s, sum(step_ms) / steps, config, extra


def serving_bench(args) -> int:
    """The serving loop at block size 16 and 32 (with the interleaved wall-time
    pass), each with the separate write and with the appending decode."""
    for bs in (16, 32):
        for fused in (False, True):
            v, ms, config, extra = serving_measure(bs, fused=fused)
            _line(SERVING_METRIC, v, "seq-steps/s", 32, 0, ms, "f16", config, **extra)
    return 0


SHARED_METRIC = "paged decode with shared blocks, unique-HBM GB/s, OPT-13B shape, bf16"


def shared_measure(beam: bool, grouped: bool, steps: int = 64,
                   fused: bool = False) -> tuple[float, float, dict, dict]:
    """32 prompt groups of 512 tokens x 4 sequences at the OPT-13B shape in
    bf16: parallel sampling (prompt blocks shared, reference count 4) or beam
    search (per-step fork/free remaps, copy-on-write of shared partial blocks
    through pa_copy_blocks), ``steps`` decode steps.  Returns (unique-byte
    GB/s, ms per step, config, extra keys)."""
    import torch

    from paged_kv_cache_76_amd import workloads
    from paged_kv_cache_76_amd.serving import BeamLoop

    log(f"shared blocks: beam={beam} grouped={grouped} fused={fused}")
    loop = BeamLoop(4, 32, 4, 512, steps, H, D, B, "bf16", beam=beam, keep_history=False, grouped=grouped,
                    fused=fused)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    logical = unique = copies = cow_tokens = 0
    saved, uniq_steps = [], []
    # host work (remaps, appends, activations, uploads) for every step first,
    # so the timed launches find everything resident in HBM
    plans = []
    for i in range(steps):
        p = loop.plan()
        logical += workloads.decode_bytes(p["lens"], H, D, 2, B)
        uniq_steps.append(loop.unique_blocks_read(p["rows"]) * B * H * D * 2 * 2)
        unique += uniq_steps[-1]
        copies += p["n_pairs"]
        cow_tokens += p["cow_tokens"]
        saved.append(loop.mgr.blocks_saved_by_sharing())
        plans.append(p)
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    loop.warm(plans[0])                             # first-launch code loading, untimed
    # the first step's plain decode, read-only, until the clocks have settled
    out0 = torch.empty((len(plans[0]["rows"]), H, D), dtype=torch.bfloat16, device="cuda")
    d0 = plans[0]["dev"]
    from paged_kv_cache_76_amd import _lib as L
    if grouped:
        settle(lambda: L.pa_paged_decode_grouped(loop.cache, out0, d0["q"], d0["tables"], d0["lens"],
                                                 plans[0]["max_ctx"], loop.scale, 4, loop.ws))
    else:
        settle(lambda: L.pa_paged_decode(loop.cache, out0, d0["q"], d0["tables"], d0["lens"], plans[0]["max_ctx"],
                                         loop.scale, loop.ws))
    # the timed span has no per-step instrumentation (an event pair per
    # step costs several us); per-launch decode durations come from a
    # replay of every step's decode with events around it afterwards
    span[0].record()
    for i in range(steps):
        loop.launch(plans[i])
    span[1].record()
    torch.cuda.synchronize()
    kernel_s = span[0].elapsed_time(span[1]) * 1e-3
    for i in range(steps):
        ev[i][0].record()
        loop.decode_only(plans[i])
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    # the same replays, each right after a cache flush: a step's unique bytes
    # (its prompt blocks above all, re-read every step) fit in part in the
    # 256 MB Infinity Cache, which back-to-back steps could otherwise hit
    cold = flushed_replays(lambda i: loop.decode_only(plans[i]), steps)
    # the copies' algorithmic bytes: each copy carries the appending row's
    # tokens before its newest (read once, written once, K and V)
    cow_bytes = cow_tokens * 2 * 2 * H * D * 2
    name = ("beam search (width 4)" if beam else "parallel sampling (4 per prompt)") + \
        (", grouped decode" if grouped else "")
    config = {"workload": f"shared-block decode: {name}", "groups": 32, "width": 4, "prompt_len": 512,
              "heads": H, "head_dim": D, "block_size": B, "seed": "SeedSequence(76004)",
              "decode_entry": ("pa_paged_decode_append" if fused else
                               "pa_paged_decode_grouped" if grouped else "pa_paged_decode")
              + (" (group 4)" if grouped else ""),
              "step_launches": ("the appending decode alone (it makes the copy-on-write copies and writes the new "
                                "tokens)" if loop.fold_copies else
                                "copies, then the appending decode (it writes the new tokens)") if fused
              else "copies, pa_reshape_and_cache, decode"}
    extra = dict(logical_GBps=round(logical / kernel_s / 1e9, 1),
                 pct_of_peak_unique=round(100 * (unique + cow_bytes) / kernel_s / 1e9 / PEAK_HBM_GBS, 2),
                 seq_steps_per_s=round(128 * steps / kernel_s, 1),
                 cow_pairs_per_step=round(copies / steps, 2), cow_tokens_per_step=round(cow_tokens / steps, 1),
                 cow_GB_per_step=round(cow_bytes / steps / 1e9, 4), blocks_saved_by_sharing_mean=round(sum(saved) / steps, 1),
                 logical_GB_per_step=round(logical / steps / 1e9, 4), unique_GB_per_step=round(unique / steps / 1e9, 4),
                 decode_launch_us_p10_p50_p90=[round(sorted(ms)[int(q * (steps - 1))] * 1e3, 1) for q in (0.1, 0.5, 0.9)],
                 decode_launch_us_mean=round(sum(ms) / steps * 1e3, 1),
                 decode_unique_GBps=round(sum(uniq_steps) / (sum(ms) * 1e-3) / 1e9, 1),
                 after_cache_flush=dict(
                     decode_launch_us_mean=round(sum(cold) / steps * 1e3, 1),
                     decode_unique_GBps=round(sum(uniq_steps) / (sum(cold) * 1e-3) / 1e9, 1),
                     pct_of_peak_unique=round(100 * sum(uniq_steps) / (sum(cold) * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                     flush="a 1 GiB read pass before each replayed decode"),
                 timing=f"span of the {steps} steps' launches with no per-step instrumentation; decode launch "
                        "durations from replays of every step's decode with events around each (a fused loop's "
                        "replay stores each newest token again, with the same bits, and makes no copies)")
    del plans, loop
    return (unique + cow_bytes) / kernel_s / 1e9, kernel_s / steps * 1e3, config, extra


def shared_bench(args) -> int:
    """Parallel sampling and beam search, each with pa_paged_decode and
    pa_paged_decode_grouped, with the separate write and fused into the
    appending decode."""
    for beam, grouped in ((False, False), (False, True), (True, False), (True, True)):
        for fused in (False, True):
            v, ms, config, extra = shared_measure(beam, grouped, fused=fused)
            name = config["workload"].split(": ", 1)[1]
            _line(f"{SHARED_METRIC}, {name}", v, "GB/s", 64, 0, ms, "bf16", config, **extra)
    return 0


LONG_METRIC = "paged long-context decode HBM GB/s (16 x 32768 tokens, 72 heads, d128, bf16)"


def longdecode_measure(steps: int, warmup: int, cpu_sample: bool) -> tuple[float, float, dict, dict]:
    """16 sequences x 32768 tokens, 72 heads, d=128, bf16, B=16 (19.3 GB of
    K/V read per step): repeated decode steps over the same cache."""
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd import workloads

    S5, C5, H5 = 16, 32768, 72
    log("building the 32K long-context cache (device-generated, 19.3 GB)")
    sample = ((0, 0), (0, 71), (15, 0), (15, 71)) if cpu_sample else ()
    ld = workloads.build_long_decode(5, S5, C5, H5, D, B, "bf16", samples=sample)
    ws = L.decode_workspace(ld.cache, S5, C5)
    out = torch.empty((S5, H5, D), dtype=torch.bfloat16, device="cuda")
    n = steps + warmup
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    settle(lambda: L.pa_paged_decode(ld.cache, out, ld.q_dev, ld.tables_dev, ld.lens_dev, C5, ld.scale, ws))
    for i in range(n):
        if i == warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        ev[i][0].record()
        L.pa_paged_decode(ld.cache, out, ld.q_dev, ld.tables_dev, ld.lens_dev, C5, ld.scale, ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(warmup, n)) / steps
    nbytes = workloads.decode_bytes(ld.lens, H5, D, 2, B)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"long decode {ms * 1e3:.1f} us -> {gbs:.0f} GB/s")
    cpu = None
    if sample:
        # the float64 oracle on 2 of the 16 sequences (2 heads each), scaled to
        # the whole step by the share of (sequence, head) pairs timed
        import numpy as np
        from oracle import attention as oa

        data = [(np.asarray(q.to(torch.float64)), np.asarray(K.to(torch.float64)), np.asarray(V.to(torch.float64)))
                for q, K, V in (ld.samples[k] for k in sample)]
        times = []
        for _ in range(3):
            t1 = time.perf_counter()
            for q, K, V in data:
                oa.attend(q, K, V, ld.scale)
            times.append(time.perf_counter() - t1)
        dt = sorted(times)[1] * (S5 * H5) / len(sample)
        cpu = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"sequences 0 and 15, heads 0 and 71 ({len(sample)} of {S5 * H5} (sequence, head) pairs, "
                         f"32768 tokens each), median of 3, scaled to the whole step; float64 NumPy on "
                         f"{os.cpu_count()} host cores ({cpu_model()})", "seconds_whole_step": round(dt, 2)}
        log(f"cpu oracle sample: {cpu['value']} GB/s (whole step {dt:.1f} s)")
    config = {"workload": "long-context decode", "sequences": S5, "context": C5, "heads": H5, "head_dim": D,
              "block_size": B, "seed": "torch.Generator(76005) on device"}
    extra = dict(roofline={"bound": "hbm", "kernel": "pa_paged_decode (partition + merge kernels)",
                           "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                           "avg_launch_us": round(ms * 1e3, 2), "algorithmic_bytes_per_launch": nbytes},
                 seq_steps_per_s=round(S5 / (ms * 1e-3), 1), cpu_baseline=cpu)
    del ld, ws, out
    return gbs, elapsed / steps * 1e3, config, extra


def longdecode_bench(args) -> int:
    gbs, ms, config, extra = longdecode_measure(args.steps, args.warmup, args.cpu_seqs > 0)
    _line(LONG_METRIC, gbs, "GB/s", args.steps, args.warmup, ms, "bf16", config, **extra)
    return 0


APPEND_METRIC = "decode step latency, cache write + decode in two launches vs one appending launch"


def append_bench(args) -> int:
    """One decode step's device work at the OPT-13B shape (fp16, B=16): the
    new tokens' write (pa_reshape_and_cache) followed by pa_paged_decode, vs
    pa_paged_decode_append, for batches from 1 to 256 sequences.  Each sample
    is 20 back-to-back steps over inputs resident in HBM (the steady state of
    a serving loop); the median of 15 interleaved samples is reported."""
    import math
    import statistics

    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd import workloads

    for S, Ln in ((1, 512), (4, 512), (16, 512), (64, 1024), (256, 1024)):
        log(f"appending decode: {S} x {Ln}")
        h = workloads.host_histories(5, [Ln] * S, H, D, B, DTYPE)
        mgr = h.manager
        cache = L.KVCache.empty(mgr.num_blocks + 1, H, B, D, torch.float16)
        L.pa_reshape_and_cache(cache, h.k_all.cuda(), h.v_all.cuda(), torch.from_numpy(h.slots).cuda())
        newest = np.cumsum(h.lens) - 1
        key, val = h.k_all[newest].cuda(), h.v_all[newest].cuda()
        slots = torch.from_numpy(h.slots[newest]).cuda()
        q, tables = h.q.cuda(), torch.from_numpy(mgr.tables).cuda()
        lens = torch.from_numpy(h.lens.astype(np.int32)).cuda()
        ws = L.decode_workspace(cache, S, Ln)
        out = torch.empty((S, H, D), dtype=torch.float16, device="cuda")
        scale = 1 / math.sqrt(D)

        def pair():
            L.pa_reshape_and_cache(cache, key, val, slots)
            L.pa_paged_decode(cache, out, q, tables, lens, Ln, scale, ws)

        def fused():
            L.pa_paged_decode_append(cache, out, q, key, val, tables, lens, Ln, scale, 1, ws)

        pair(), fused()
        settle(lambda: L.pa_paged_decode(cache, out, q, tables, lens, Ln, scale, ws))
        res = {"pair": [], "fused": []}
        for name, fn in (("pair", pair), ("fused", fused)) * 15:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn()
            e1.record()
            torch.cuda.synchronize()
            res[name].append(e0.elapsed_time(e1) * 1e3 / 20)
        pair_us, fused_us = statistics.median(res["pair"]), statistics.median(res["fused"])
        nbytes = workloads.decode_bytes(h.lens, H, D, ELEM, B) + 2 * S * H * D * ELEM
        _line(APPEND_METRIC, round(fused_us, 2), "us", 20, 1, fused_us * 1e-3, "f16",
              {"workload": "one decode step: new tokens' write and the decode", "sequences": S, "context": Ln,
               "heads": H, "head_dim": D, "block_size": B},
              higher_is_better=False, two_launches_us=round(pair_us, 2), one_launch_us=round(fused_us, 2),
              saved_pct=round(100 * (1 - fused_us / pair_us), 1),
              one_launch_GBps=round(nbytes / (fused_us * 1e-6) / 1e9, 1))
        del cache
    # beam search (width 4, bf16, 512-token prompts): copy-on-write copies,
    # write and grouped decode as three launches, or all in one appending launch
    from paged_kv_cache_76_amd.serving import BeamLoop
    for groups in (1, 4, 32):
        log(f"appending decode, beam search: {groups} groups of 4")
        res = {}
        for fused in (False, True):
            loop = BeamLoop(4, groups, 4, 512, 40, H, D, B, "bf16", beam=True, keep_history=False, grouped=True,
                            fused=fused)
            plans = [loop.plan() for _ in range(40)]
            loop.warm(plans[0])
            d0, out0 = plans[0]["dev"], torch.empty((4 * groups, H, D), dtype=torch.bfloat16, device="cuda")
            settle(lambda: L.pa_paged_decode_grouped(loop.cache, out0, d0["q"], d0["tables"], d0["lens"],
                                                     plans[0]["max_ctx"], loop.scale, 4, loop.ws))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for p in plans:
                loop.launch(p)
            e1.record()
            torch.cuda.synchronize()
            res[fused] = (e0.elapsed_time(e1) * 1e3 / len(plans), sum(p["n_pairs"] for p in plans) / len(plans))
            del loop, plans
        _line(APPEND_METRIC + ", beam search", round(res[True][0], 2), "us", 40, 1, res[True][0] * 1e-3, "bf16",
              {"workload": "beam-search step: copy-on-write copies, new tokens' write and grouped decode",
               "groups": groups, "width": 4, "prompt_len": 512, "heads": H, "head_dim": D, "block_size": B,
               "seed": "SeedSequence(76004)"},
              higher_is_better=False, three_launches_us=round(res[False][0], 2), one_launch_us=round(res[True][0], 2),
              saved_pct=round(100 * (1 - res[True][0] / res[False][0]), 1),
              cow_pairs_per_step=round(res[False][1], 2),
              timing="span of 40 consecutive steps planned ahead, no per-step instrumentation")
    return 0


def accounting_bench(args) -> int:
    """Share of held KV slots that store tokens, contiguous reservation vs
    paged blocks, on the serving-loop length mix (no GPU involved)."""
    from paged_kv_cache_76_amd import accounting
    from paged_kv_cache_76_amd.serving import opt13b_serving_lengths

    prompt, out, start = opt13b_serving_lengths(3, 256)
    for bs in (16, 32):
        u = accounting.utilisation(prompt, out, prompt + start, 2048, bs)
        _line("KV memory holding token states (fraction of held slots)", 100 * u["paged"], "%", 1, 0, 0.0, "int64",
              {"workload": "reservation accounting, 256-request serving snapshot", "block_size": bs,
               "max_len": 2048, "seed": "SeedSequence(76003)"},
              contiguous_max_pct=round(100 * u["max"], 2), contiguous_pow2_pct=round(100 * u["pow2"], 2),
              contiguous_oracle_pct=round(100 * u["oracle"], 2), paged_pct=round(100 * u["paged"], 2))
    return 0


def blocksize_bench(args) -> int:
    """Block sizes 8..128: the OPT-13B decode workload (64 x 40 heads, d=128,
    fp16, contexts U[1,2048]) and the 256-sequence serving loop, decode GB/s
    against tail waste."""
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd import workloads

    lens = workloads.opt13b_decode_lengths(2, S)
    nbytes = None
    for bs in (8, 16, 32, 64, 128):
        b = workloads.build_decode_batch(2, lens, H, D, bs, DTYPE, nan_fill=False)
        ws = L.decode_workspace(b.cache, S, b.max_context_len)
        out = torch.empty((S, H, D), dtype=torch.float16, device="cuda")
        fn = lambda: L.pa_paged_decode(b.cache, out, b.q_dev, b.tables_dev, b.lens_dev, b.max_context_len,
                                       b.scale, ws)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[args.steps // 2]
        nbytes = workloads.decode_bytes(lens, H, D, ELEM, bs)
        waste = int(b.manager.tail_waste().sum())
        _line("paged decode HBM GB/s vs block size, OPT-13B shape", nbytes / (ms * 1e-3) / 1e9, "GB/s",
              args.steps, args.warmup, ms, "f16",
              {"workload": "block-size sweep of the OPT-13B decode", "block_size": bs, "sequences": S, "heads": H,
               "head_dim": D, "seed": "SeedSequence(76002)"},
              pct_of_peak=round(100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2), median_us=round(ms * 1e3, 2),
              tail_waste_slots=waste, tail_waste_pct=round(100 * waste / (waste + int(lens.sum())), 3))
        del b, ws, out
    # the same sweep on the 256-sequence serving loop (device pass only)
    for bs in (8, 16, 32, 64, 128):
        v, ms, config, extra = serving_measure(bs, wall_pass=False)
        config["workload"] = "block-size sweep of the serving loop"
        _line(SERVING_METRIC, v, "seq-steps/s", 32, 0, ms, "f16", config, **extra)
    return 0


def paging_cost_bench(args) -> int:
    """What scattering the blocks costs the decode: the OPT-13B decode (64 x
    40 heads, d=128, fp16, contexts U[1,2048], B=16) on its seeded-shuffled
    pool, and on a copy of that pool in which every sequence's blocks sit at
    consecutive physical ids in logical order (the layout a contiguous,
    unpaged cache would have).  The kernel, the lengths, the queries and the
    arithmetic are the same, so the outputs must be bit-identical; the time
    difference is the cost of the scattered block placement ("vLLM /
    PagedAttention", awesome.papernotes.org, key design 5, puts the kernel
    overhead of paging at 20-26 %).  Both layouts are also
    read with no arithmetic (their K/V tiles in the decode's order), the
    achievable rate of each access pattern."""
    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd import workloads

    lens = workloads.opt13b_decode_lengths(2, S)
    b = workloads.build_decode_batch(2, lens, H, D, B, DTYPE, nan_fill=False)
    tables = b.manager.tables[:S]
    nblk = [-(-int(n) // B) for n in lens]
    first = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
    src_ids = np.concatenate([tables[s, :nblk[s]] for s in range(S)]).astype(np.int64)
    total = int(src_ids.size)
    contig = L.KVCache.empty(total + 1, H, B, D, torch.float16)
    idx = torch.from_numpy(src_ids).cuda()
    contig.k[:total] = b.cache.k[idx]
    contig.v[:total] = b.cache.v[idx]
    ct = np.full_like(tables, total)        # unused entries: the spare block past the sequences
    for s in range(S):
        ct[s, :nblk[s]] = first[s] + np.arange(nblk[s])
    ctables = torch.from_numpy(np.ascontiguousarray(ct)).cuda()
    ws = L.decode_workspace(b.cache, S, b.max_context_len)
    outs = {n: torch.empty((S, H, D), dtype=torch.float16, device="cuda") for n in ("scattered", "contiguous")}
    runs = {"scattered": lambda: L.pa_paged_decode(b.cache, outs["scattered"], b.q_dev, b.tables_dev, b.lens_dev,
                                                   b.max_context_len, b.scale, ws),
            "contiguous": lambda: L.pa_paged_decode(contig, outs["contiguous"], b.q_dev, ctables, b.lens_dev,
                                                    b.max_context_len, b.scale, ws)}
    for fn in runs.values():
        fn()
    torch.cuda.synchronize()
    same = torch.equal(outs["scattered"].view(torch.int16), outs["contiguous"].view(torch.int16))
    log(f"decode output on the two layouts bit-identical: {same}")
    settle(runs["scattered"])
    # the layouts in alternating blocks of back-to-back launches (a block of
    # one layout, then one of the other, five rounds), an event pair around
    # each launch, no host synchronisation inside a block; a block starts with
    # a few untimed launches, so no launch is timed right after the other
    # layout's
    times = {n: [] for n in runs}
    per_block = max(args.steps, 5)
    for _ in range(5):
        for n, fn in runs.items():
            for _ in range(3):
                fn()
            ev = []
            for _ in range(per_block):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                ev.append((e0, e1))
            torch.cuda.synchronize()
            times[n] += [a.elapsed_time(z) for a, z in ev]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    tile_bytes = B * D * ELEM

    def tile_list(tab):
        ids = [(tab[s, :nblk[s]][None, :].astype(np.int64) * H + np.arange(H)[:, None]).reshape(-1) for s in range(S)]
        return torch.from_numpy(np.concatenate(ids).astype(np.int32)).cuda()

    reads = {}
    for n, (cache, tab) in {"scattered": (b.cache, tables), "contiguous": (contig, ct)}.items():
        tl = tile_list(tab)
        evs = []
        for _ in range(max(args.steps, 5)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            L.pa_read_tiles(cache.k, tile_bytes, tl, sink)
            L.pa_read_tiles(cache.v, tile_bytes, tl, sink)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = [a.elapsed_time(z) for a, z in evs]
        reads[n] = 2 * tl.numel() * tile_bytes / (sorted(ts)[len(ts) // 2] * 1e-3) / 1e9
    nbytes = workloads.decode_bytes(lens, H, D, ELEM, B)
    med = {n: sorted(t)[len(t) // 2] for n, t in times.items()}
    for n in runs:
        gbs = nbytes / (med[n] * 1e-3) / 1e9
        _line("paged decode HBM GB/s, scattered vs contiguous block placement, OPT-13B shape", gbs, "GB/s",
              len(times[n]), 0, med[n], "f16",
              {"workload": f"OPT-13B decode, {n} block placement", "sequences": S, "heads": H, "head_dim": D,
               "block_size": B, "seed": "SeedSequence(76002)"},
              pct_of_peak=round(100 * gbs / PEAK_HBM_GBS, 2), median_us=round(med[n] * 1e3, 2),
              plain_tile_read_GBps=round(reads[n], 1), outputs_bit_identical=same)
    log(f"scattered {med['scattered'] * 1e3:.1f} us, contiguous {med['contiguous'] * 1e3:.1f} us: "
        f"scattered placement costs {100 * (med['scattered'] / med['contiguous'] - 1):.1f} %")
    return 0


def copy_ablation_bench(args) -> int:
    """Copy-on-write copies issued as one batched pa_copy_blocks launch versus
    one device-to-device memcpy per block and pool (the alternative the pages
    reject), for bursts of 8..512 OPT-13B blocks."""
    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L

    N = 2048
    cache = L.KVCache.empty(N, H, B, D, torch.float16)
    cache.k.fill_(1.0)
    cache.v.fill_(2.0)
    ids = np.random.default_rng(0).permutation(N)
    for n in (8, 38, 96, 512):
        pairs_np = np.stack([ids[:n], ids[n:2 * n]], axis=1).astype(np.int64)
        pairs = torch.from_numpy(pairs_np).cuda()

        def fused():
            L.pa_copy_blocks(cache, pairs)

        def per_block():
            for s_, d_ in pairs_np:
                cache.k[d_].copy_(cache.k[s_], non_blocking=True)
                cache.v[d_].copy_(cache.v[s_], non_blocking=True)

        res = {}
        for name, fn in (("fused", fused), ("memcpy_per_block", per_block)):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            for _ in range(args.steps):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            res[name] = (ev0.elapsed_time(ev1) / args.steps, (time.perf_counter() - t0) / args.steps * 1e3)
        moved = 2 * 2 * n * H * B * D * ELEM
        _line("copy-on-write block copies GB/s (read + write), batched kernel", moved / (res["fused"][0] * 1e-3) / 1e9,
              "GB/s", args.steps, args.warmup, res["fused"][0], "f16",
              {"workload": "CoW copy burst", "pairs": n, "heads": H, "block_size": B, "head_dim": D},
              fused_us=round(res["fused"][0] * 1e3, 2), per_block_memcpy_us=round(res["memcpy_per_block"][0] * 1e3, 2),
              per_block_memcpy_host_ms=round(res["memcpy_per_block"][1], 3),
              speedup=round(res["memcpy_per_block"][0] / res["fused"][0], 2))
    return 0


def prefix_bench(args) -> int:
    """A provider prefix of 1024 tokens (a few-shot prompt) shared by 32
    requests whose task inputs are lognormal (median 100, sigma 1, <= 1024),
    OPT-13B heads, bf16: prefill over the task inputs only (the prefix's K/V
    are cached) against prefilling every full prompt."""
    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd import inputs, workloads

    r_len = inputs.streams(6, workloads.STREAMS)[0]
    tasks = inputs.lognormal_lengths(r_len, 32, 100, 1.0, 1, 1024)
    prefix = 1024
    b = workloads.build_shared_prefix(6, prefix, tasks, H, D, B, "bf16")
    full = workloads.build_prefill_batch(6, prefix + tasks, prefix + tasks, H, D, B, "bf16", nan_fill=False)
    res = {}
    for name, bb, qmax in (("task_only", b, int(tasks.max())), ("full_prompt", full, int((prefix + tasks).max()))):
        rows = int(bb.cu_q[-1])
        out = torch.empty((rows, H, D), dtype=torch.bfloat16, device="cuda")
        fn = lambda: L.pa_paged_prefill(bb.cache, out, bb.q_dev, bb.tables_dev, bb.cu_q_dev, bb.lens_dev, qmax,
                                        int(bb.lens.max()), bb.scale)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        res[name] = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[args.steps // 2]
    f_task = workloads.prefill_flops(prefix + tasks, tasks, H, D)
    f_full = workloads.prefill_flops(prefix + tasks, prefix + tasks, H, D)
    _line("prefill time saved by a cached shared prefix (speedup vs full-prompt prefill)",
          res["full_prompt"] / res["task_only"], "x", args.steps, args.warmup, res["task_only"], "bf16",
          {"workload": "shared prefix: 32 requests, 1024-token cached prefix, lognormal(100,1) task inputs",
           "heads": H, "head_dim": D, "block_size": B, "seed": "SeedSequence(76006)"},
          task_only_us=round(res["task_only"] * 1e3, 1), full_prompt_us=round(res["full_prompt"] * 1e3, 1),
          task_only_TFLOPs=round(f_task / (res["task_only"] * 1e-3) / 1e12, 1),
          full_prompt_TFLOPs=round(f_full / (res["full_prompt"] * 1e-3) / 1e12, 1),
          flop_ratio=round(f_full / f_task, 2), cow_copies=b.copies)
    return 0


def swap_bench(args) -> int:
    """Preemption by swapping: 16 sequences x 1024 tokens at the OPT-13B
    shape (fp16) leave the device for a pinned host pool in one batched call
    and come back in another (1024 blocks, 320 MiB each way)."""
    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd.block_manager import BlockManager

    S16, L16 = 16, 1024
    nblk = S16 * L16 // B
    N = nblk + 64
    cache = L.KVCache.empty(N, H, B, D, torch.float16)
    cache.k.fill_(1.0)
    cache.v.fill_(2.0)
    m = BlockManager(N, B, max_rows=S16, max_blocks_per_seq=L16 // B, host_blocks=nblk,
                     free_order=np.random.default_rng(0).permutation(N))
    for s_ in range(S16):
        m.add_prompt(s_, L16)
    host_k = torch.empty((nblk, H, B, D), dtype=torch.float16, pin_memory=True)
    host_v = torch.empty((nblk, H, B, D), dtype=torch.float16, pin_memory=True)
    t_host = time.perf_counter()
    out_np = m.swap_out(range(S16))
    in_np = m.swap_in(range(S16))
    bm_ms = (time.perf_counter() - t_host) * 1e3 / 2
    out_pairs, in_pairs = torch.from_numpy(out_np).cuda(), torch.from_numpy(in_np).cuda()
    moved = 2 * nblk * H * B * D * 2                 # keys and values, one direction
    staging = L.swap_staging(cache, 256)             # 80 MiB: the 1024-block group moves in 4 chunks

    def swap(form, pairs_dev, pairs_np, direction, stream=None):
        # the kernel form takes device pairs, the copy-engine form host pairs
        if form == "kernel":
            L.pa_swap_blocks(cache, host_k, host_v, pairs_dev, direction, stream=stream)
        else:
            L.pa_swap_blocks_dma(cache, host_k, host_v, pairs_np, direction, staging, stream=stream,
                                 pairs_dev=pairs_dev)

    res = {}
    for form in ("kernel", "dma"):
        for name, pairs, pairs_np, direction in (("out", out_pairs, out_np, L.PA_SWAP_OUT),
                                                 ("in", in_pairs, in_np, L.PA_SWAP_IN)):
            for _ in range(args.warmup):
                swap(form, pairs, pairs_np, direction)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for e0, e1 in ev:
                e0.record()
                swap(form, pairs, pairs_np, direction)
                e1.record()
            torch.cuda.synchronize()
            res[(form, name)] = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[args.steps // 2]
    # reference: one plain host<->device copy of the same number of bytes
    flat_dev = cache.k.view(-1)[: nblk * H * B * D]
    flat_host = host_k.view(-1)
    flat_host.copy_(flat_dev, non_blocking=True)     # untimed first copy
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(2):
        flat_host.copy_(flat_dev, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    memcpy_gbs = 2 * flat_dev.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9

    # Overlap: the OPT-13B decode step of the sequences that stay runs on the
    # current stream while the group swaps out on a second stream (default
    # priority); each stream is timed with its own events.
    from paged_kv_cache_76_amd import workloads
    lens0 = workloads.opt13b_decode_lengths(2, S)
    db = workloads.build_decode_batch(2, lens0, H, D, B, DTYPE, nan_fill=False)
    dws = L.decode_workspace(db.cache, S, db.max_context_len)
    dout = torch.empty((S, H, D), dtype=torch.float16, device="cuda")
    n_dec = 30

    def decode():
        L.pa_paged_decode(db.cache, dout, db.q_dev, db.tables_dev, db.lens_dev, db.max_context_len, db.scale, dws)

    side = torch.cuda.Stream()

    def run(with_swap: bool, with_decode: bool, form: str = "kernel"):
        es = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ed = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        torch.cuda.synchronize()
        if with_swap:
            es[0].record(side)
            swap(form, out_pairs, out_np, L.PA_SWAP_OUT, stream=side)
            es[1].record(side)
        if with_decode:
            ed[0].record()
            for _ in range(n_dec):
                decode()
            ed[1].record()
        torch.cuda.synchronize()
        return (ed[0].elapsed_time(ed[1]) * 1e3 / n_dec if with_decode else None,
                es[0].elapsed_time(es[1]) * 1e-3 if with_swap else None)

    settle(decode)
    med = lambda v: sorted(v)[len(v) // 2]
    dec_bytes = workloads.decode_bytes(lens0, H, D, 2, B)
    overlaps = {}
    for form in ("kernel", "dma"):
        for _ in range(2):
            run(True, True, form)
        alone = [run(False, True)[0] for _ in range(5)]
        swap_alone = [run(True, False, form)[1] for _ in range(5)]
        both = [run(True, True, form) for _ in range(5)]
        overlap = {"decode_alone_us": round(med(alone), 1),
                   "decode_during_swap_us": round(med([b[0] for b in both]), 1),
                   "decode_alone_GBps": round(dec_bytes / (med(alone) * 1e-6) / 1e9, 1),
                   "decode_during_swap_GBps": round(dec_bytes / (med([b[0] for b in both]) * 1e-6) / 1e9, 1),
                   "swap_out_alone_GBps": round(moved / med(swap_alone) / 1e9, 1),
                   "swap_out_during_decode_GBps": round(moved / med([b[1] for b in both]) / 1e9, 1),
                   "decodes_per_swap": n_dec}
        log(f"overlap ({form}): decode {overlap['decode_alone_us']} us alone, {overlap['decode_during_swap_us']} us "
            f"during the swap; swap-out {overlap['swap_out_alone_GBps']} GB/s alone, "
            f"{overlap['swap_out_during_decode_GBps']} GB/s during the decodes")
        overlaps[form] = overlap
    for form, entry in (("kernel", "pa_swap_blocks (a kernel)"), ("dma", "pa_swap_blocks_dma (copy engines)")):
        _line(f"preemption swap GB/s (device -> pinned host), 16 x 1024 OPT-13B tokens, {entry}",
              moved / (res[(form, "out")] * 1e-3) / 1e9, "GB/s", args.steps, args.warmup, res[(form, "out")], "f16",
              {"workload": "swap out / swap in of a 16-sequence group", "blocks": nblk, "heads": H,
               "block_size": B, "head_dim": D, "bytes_each_way": moved, "entry": entry},
              swap_in_GBps=round(moved / (res[(form, "in")] * 1e-3) / 1e9, 1),
              swap_out_us=round(res[(form, "out")] * 1e3, 1), swap_in_us=round(res[(form, "in")] * 1e3, 1),
              contiguous_memcpy_d2h_GBps=round(memcpy_gbs, 1), host_block_manager_ms=round(bm_ms, 3),
              overlap_with_decode=overlaps[form])
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seqs", type=int, default=64, help="sequences in the CPU-oracle sample (0: skip)")
    ap.add_argument("--prefill-steps", type=int, default=10,
                    help="decode workload: timed steps of the OPT-66B prefill sub-record (0: skip)")
    ap.add_argument("--other-configs", type=int, default=1,
                    help="decode workload: 1 adds short sub-records for the serving loop (B=16), grouped "
                         "shared-block decoding (sampling, beam) and the 32K long-context decode; 0 skips them")
    ap.add_argument("--workload", choices=["decode", "copy", "prefill", "serving", "shared", "longdecode",
                                           "blocksize", "copyablation", "accounting", "prefix", "swap", "append",
                                           "pagingcost"],
                    default="decode",
                    help="decode: the OPT-13B decode step (default); copy: pa_copy_blocks over 2048 "
                         "OPT-13B blocks, a plain copy of known size used to calibrate HBM counters; "
                         "prefill: 8 x 1024-token prompts at the OPT-66B shape (write + causal prefill); "
                         "serving: 32 steps of a 256-sequence serving loop (B=16 and 32); shared: parallel "
                         "sampling and beam search over shared prompt blocks (bf16); longdecode: 16 x 32768 "
                         "tokens at the OPT-66B head count (bf16); blocksize: OPT-13B decode for block "
                         "sizes 8..128; copyablation: one batched pa_copy_blocks vs one memcpy per block; "
                         "accounting: KV utilisation of contiguous reservation vs paged blocks (host only); "
                         "prefix: prefill over task inputs only, with a cached 1024-token shared prefix; "
                         "swap: a preempted group's blocks to pinned host memory and back; append: one decode "
                         "step as write + decode launches vs one pa_paged_decode_append launch, 1..256 "
                         "sequences, and beam-search steps with their copy-on-write copies folded in; "
                         "pagingcost: the OPT-13B decode on its shuffled pool vs the same blocks placed "
                         "contiguously per sequence")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a design "
              "note, not a measured path", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_kv_cache_76_amd import _lib as L
    from paged_kv_cache_76_amd import inputs, workloads

    if args.workload == "accounting":
        return accounting_bench(args)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.workload == "blocksize":
        return blocksize_bench(args)
    if args.workload == "copyablation":
        return copy_ablation_bench(args)
    if args.workload == "pagingcost":
        return paging_cost_bench(args)
    if args.workload == "prefix":
        return prefix_bench(args)
    if args.workload == "swap":
        return swap_bench(args)
    if args.workload == "copy":
        return copy_calibration(args)
    if args.workload == "prefill":
        return prefill_bench(args)
    if args.workload == "serving":
        return serving_bench(args)
    if args.workload == "shared":
        return shared_bench(args)
    if args.workload == "longdecode":
        return longdecode_bench(args)
    if args.workload == "append":
        return append_bench(args)
    K, W = args.steps, args.warmup
    # warm-up, then K timed steps with no per-step instrumentation (the
    # throughput); every step appends one token per sequence.  Then the
    # decodes of those same K steps run again with events around each launch
    # (the launch durations of the roofline): decode only reads the cache, and
    # the later steps' writes went to positions past every replayed context,
    # so a replay reads exactly the bytes its step read.
    n_steps = W + K

    lens0 = workloads.opt13b_decode_lengths(2, S)
    log(f"building OPT-13B decode workload: S={S} H={H} d={D} B={B} fp16, "
        f"tokens={int(lens0.sum())}, steps={n_steps}")
    extra = S * (-(-n_steps // B) + 1)
    batch = workloads.build_decode_batch(2, lens0, H, D, B, DTYPE, slack=1.10, extra_blocks=extra,
                                         grow_tokens=n_steps, nan_fill=False)
    mgr = batch.manager
    r_step = inputs.streams(2, workloads.STREAMS)[5]   # new tokens' k, v and q, step by step

    # host block-manager steps, done ahead of time; everything lands in HBM
    steps = []
    host_ms = []
    rows = np.arange(S)
    for i in range(n_steps):
        t0 = time.perf_counter()
        slots, pairs = mgr.append_step(rows)
        tables = mgr.tables.copy()
        lens = mgr.lens.astype(np.int32).copy()
        host_ms.append((time.perf_counter() - t0) * 1e3)
        k_new = inputs.normal(r_step, (S, H, D), DTYPE)
        v_new = inputs.normal(r_step, (S, H, D), DTYPE)
        q = inputs.normal(r_step, (S, H, D), DTYPE)
        steps.append(dict(
            slots=torch.from_numpy(slots).cuda(), pairs=torch.from_numpy(pairs).cuda(), n_pairs=len(pairs),
            k=k_new.cuda(), v=v_new.cuda(), q=q.cuda(), tables=torch.from_numpy(tables).cuda(),
            lens=torch.from_numpy(lens).cuda(), max_ctx=int(lens.max()), lens_host=lens))
    max_ctx = max(st["max_ctx"] for st in steps)
    ws = L.decode_workspace(batch.cache, S, max_ctx)
    out = torch.empty((S, H, D), dtype=torch.float16, device="cuda")
    scale = 1.0 / math.sqrt(D)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]

    def decode(i):
        st = steps[i]
        L.pa_paged_decode(batch.cache, out, st["q"], st["tables"], st["lens"], max_ctx, scale, ws)

    def step(i):
        st = steps[i]
        if st["n_pairs"]:
            L.pa_copy_blocks(batch.cache, st["pairs"])
        L.pa_reshape_and_cache(batch.cache, st["k"], st["v"], st["slots"])
        decode(i)

    for i in range(W):
        step(i)
    # then the last warm-up step's decode, read-only, until the clocks settle
    n_settle = settle(lambda: decode(max(W - 1, 0)))
    log(f"warmup done ({W} steps, then {n_settle} read-only decodes over {SETTLE_MS:.0f} ms); timing {K} steps")
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"replaying the decodes of those {K} steps with events around each launch")
    for i in range(W, W + K):
        ev[i][0].record()
        decode(i)
        ev[i][1].record()
    torch.cuda.synchronize()

    write_bytes = 2 * 2 * S * H * D * ELEM          # read + write, keys and values
    step_bytes = sum(workloads.decode_bytes(steps[i]["lens_host"], H, D, ELEM, B) + write_bytes
                     + 2 * 2 * steps[i]["n_pairs"] * H * B * D * ELEM for i in range(W, W + K))
    dec_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(W, W + K)]
    dec_bytes = [workloads.decode_bytes(steps[i]["lens_host"], H, D, ELEM, B) for i in range(W, W + K)]
    # every decode dispatch of this run (warm-up, timed steps, replays), for
    # matching rocprofv3 counter averages against algorithmic bytes
    all_dispatch_bytes = [workloads.decode_bytes(steps[i]["lens_host"], H, D, ELEM, B)
                          for i in list(range(W + K)) + list(range(W, W + K))]
    all_dispatch_bytes += [workloads.decode_bytes(steps[max(W - 1, 0)]["lens_host"], H, D, ELEM, B)] * n_settle
    log(f"algorithmic bytes per decode dispatch, averaged over all {len(all_dispatch_bytes)} of this run: "
        f"{sum(all_dispatch_bytes) / len(all_dispatch_bytes):.0f}")
    value = step_bytes / elapsed / 1e9
    ms_per_step = elapsed / K * 1e3
    dec_avg_ms = sum(dec_ms) / K
    dec_sorted = sorted(dec_ms)
    pct = lambda q: dec_sorted[min(K - 1, int(q * K))] * 1e3
    dec_gbs = (sum(dec_bytes) / K) / (dec_avg_ms * 1e-3) / 1e9
    log(f"step {ms_per_step:.3f} ms, decode {dec_avg_ms * 1e3:.1f} us -> {dec_gbs:.0f} GB/s")
    # the same decodes again, each right after a cache flush: what a launch
    # reaches when nothing it reads is left in the Infinity Cache or the L2s
    cold_ms = flushed_replays(lambda j: decode(W + j), K)
    cold_avg_ms = sum(cold_ms) / K
    cold_gbs = (sum(dec_bytes) / K) / (cold_avg_ms * 1e-3) / 1e9
    log(f"decode after a cache flush: {cold_avg_ms * 1e3:.1f} us -> {cold_gbs:.0f} GB/s")

    cpu = None
    if args.cpu_seqs > 0:
        log(f"timing the CPU oracle on {args.cpu_seqs} sequences")
        cpu = cpu_baseline(batch, args.cpu_seqs)

    traffic = measured_traffic()
    prefill = None
    if args.prefill_steps > 0:
        log(f"prefill sub-record: OPT-66B 8 x 1024 prompts, {args.prefill_steps} steps")
        prefill = prefill_measure(args.prefill_steps, 2, args.cpu_seqs > 0, gemm=False)
    others = {}
    if args.other_configs:
        # the other workloads of the same hot path, one short pass each (the
        # serving and shared-block steps in one appending launch each, the
        # faster form; --workload serving / shared time both forms)
        v, ms, config, extra = serving_measure(16, wall_pass=False, fused=True)
        others["serving"] = dict(metric=SERVING_METRIC, value=round(v, 1), unit="seq-steps/s", steps=32,
                                 ms_per_step=round(ms, 4), dtype="f16", config=config, **extra)
        for beam in (False, True):
            v, ms, config, extra = shared_measure(beam, True, fused=True)
            others["shared_beam" if beam else "shared_sampling"] = dict(
                metric=f"{SHARED_METRIC}, {config['workload'].split(': ', 1)[1]}", value=round(v, 2), unit="GB/s",
                steps=64, ms_per_step=round(ms, 4), dtype="bf16", config=config, **extra)
        v, ms, config, extra = longdecode_measure(5, 2, False)
        others["longdecode"] = dict(metric=LONG_METRIC, value=round(v, 2), unit="GB/s", steps=5, warmup=2,
                                    ms_per_step=round(ms, 4), dtype="bf16", config=config, **extra)
    last = steps[-1]
    ach = achievable_reads(batch.cache, last["tables"].cpu().numpy(), last["lens_host"])
    ach["decode_frac_of_kv_tile_read"] = round(dec_gbs / ach["kv_tile_read_GBps"], 4)
    ach["decode_frac_of_stream_read"] = round(dec_gbs / ach["stream_read_GBps"], 4)
    log(f"achievable reads: stream {ach['stream_read_GBps']:.0f} GB/s, decode's K/V tiles "
        f"{ach['kv_tile_read_GBps']:.0f} GB/s; decode at {100 * ach['decode_frac_of_kv_tile_read']:.1f} % of the latter")
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "OPT-13B-shaped single-layer paged decode step (write + decode)",
                   "sequences": S, "heads": H, "head_dim": D, "block_size": B, "kv_dtype": "f16",
                   "context_lens": "uniform[1,2048] + step index", "seed": "SeedSequence(76002)",
                   "pool_blocks": batch.cache.num_blocks, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "seq_steps_per_s": round(S * K / elapsed, 1),
        "host_block_manager_ms_per_step": round(sum(host_ms) / len(host_ms), 4),
        "roofline": {"bound": "hbm", "kernel": "pa_paged_decode (partition kernel; its merge kernel runs only for "
                                               "contexts longer than one 4096-token partition)", "achieved": round(dec_gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic and traffic["bytes"],
                     "traffic_over_algorithmic": traffic and traffic["ratio"],
                     "avg_launch_us": round(dec_avg_ms * 1e3, 2),
                     "launch_us_p10_p50_p90": [round(pct(0.1), 2), round(pct(0.5), 2), round(pct(0.9), 2)],
                     "algorithmic_bytes_per_launch": int(sum(dec_bytes) / K),
                     "after_cache_flush": {"avg_launch_us": round(cold_avg_ms * 1e3, 2),
                                           "achieved": round(cold_gbs, 2),
                                           "frac": round(cold_gbs / PEAK_HBM_GBS, 4),
                                           "flush": "a 1 GiB read pass before each launch"}},
        "cpu_baseline": cpu,
        "achievable": ach,
        "timing": (f"value and ms_per_step: {K} steps with no per-step instrumentation after {W} warm-up steps; "
                   f"roofline launch durations: the decodes of the same {K} steps replayed with events around "
                   f"each launch (decode is read-only: a replay reads the bytes of its step); after_cache_flush: "
                   f"the same replays, each after a 1 GiB read pass that evicts the Infinity Cache and L2s"),
    }
    if prefill is not None:
        rec["prefill"] = {"metric": PREFILL_METRIC, "value": round(prefill["tflops"], 2), "unit": "TFLOP/s",
                          "steps": prefill["steps"], "warmup": prefill["warmup"],
                          "ms_per_step": round(prefill["elapsed"] / prefill["steps"] * 1e3, 4),
                          "dtype": "bf16", "config": prefill["config"], "roofline": prefill["roofline"],
                          "write": prefill["write"], "cpu_baseline": prefill["cpu_baseline"]}
    rec.update(others)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
