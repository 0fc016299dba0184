#!/usr/bin/env python3
"""FedAvg aggregation benchmark on one MI355X.

Headline: resident dense FedAvg of K=16 bf16 clients of a 1,921,878,016-
parameter transformer-shaped tensor list (fp32 accumulation, bf16 output);
one step = one fedavg_aggregate call over all clients.  The same JSON line
also carries every other aggregation mode at its full workload size:

  dense_small  K=3 fp32 clients of 10^6 parameters (launch-latency bound)
  adapter      K=8 clients, LoRA q,k,v,o adapters of 32 layers (16.8M bf16),
               each client sending a Bernoulli(0.6) subset of the modules
  streaming    8,030,261,248 bf16 parameters, K=32 clients arriving one by
               one as 64 MiB chunks from pinned host memory (PCIe bound), and
               the accumulate kernel alone on device-resident chunks
  windows      the streaming workload with the accumulator cut into 4 windows
               of the parameter space (for accumulators larger than HBM)
  sparse       10^9 fp32 parameters, K=20 clients each sending its top 10%
               (sorted int64 index, fp32 value) pairs
  topk         client-side top-10% selection from a 10^9-parameter fp32 update
  hierarchical two-level aggregation: 4 silo partials of 8,030,261,248 fp32
               sums merged into the top-level accumulator
  sparse_stream  the sparse lists scattered one client at a time into the
               streaming accumulator (partial mode)
  checksum     order-independent hash and fixed-order fp64 value sum of a
               10^9-element fp32 buffer

Inputs are seeded synthetic data generated on the GPU before timing.  The
roofline object reports the headline kernel against MI355X's 8 TB/s HBM; the
cpu_baseline object times the CPU oracle on a sample of the headline
workload.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
PCIE_PEAK_GBS = 64.0       # PCIe Gen5 x16 per direction, GB/s
METRIC = "aggregated params/sec and achieved HBM GB/s (% of MI355X peak), K clients"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "dense_k16_bf16_2b_hbm_counters.md")
KERNEL_SOURCE = os.path.join(ROOT, "weighted_model_update_amd", "csrc", "fedavg_kernels.hip")


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def kernel_source_sha():
    """SHA-256 of the source the headline kernel is built from: the kernels
    file up to the end of its resident-dense section (shared load/store
    helpers and the dense kernels) and the launch code from the residency
    helper through the dense launcher.  Edits elsewhere in the file leave it
    unchanged."""
    with open(KERNEL_SOURCE) as f:
        text = f.read()
    head = text[:text.index("// ================================================================ per-segment masks")]
    i0 = text.index("// Streaming kernels over HBM run fastest with few resident waves per CU")
    i1 = text.index("template <int X, int O, int B, int M> struct DenseRun")
    return hashlib.sha256((head + text[i0:i1]).encode()).hexdigest()


def timed(fn, steps, warmup):
    """Run fn(i) warmup times untimed, then exactly `steps` times between two
    device synchronizations.  Returns (wall seconds over the steps, list of
    per-step event durations in ms measured on the current stream)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(warmup + i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [s.elapsed_time(e) for s, e in zip(starts, ends)]


def stats(durs):
    """mean, median and min of per-launch durations (ms)."""
    d = sorted(durs)
    m = len(d)
    med = d[m // 2] if m % 2 else 0.5 * (d[m // 2 - 1] + d[m // 2])
    return {"mean_ms": sum(d) / m, "median_ms": med, "min_ms": d[0]}


def free_gpu():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# headline: dense K=16, 2B bf16
# --------------------------------------------------------------------------

def bench_dense_2b(steps, warmup):
    """The headline: the 16 clients and the output in one allocation laid out
    by the library's arena_layout (buffer j staggered j x 32 KiB within its
    2 MiB page); then the same clients copied into separate allocations,
    timed the same way for comparison (same bits required)."""
    import torch
    import synth
    import synth.device as sd
    import weighted_model_update_amd as fa
    K, N = 16, synth.numel_of(synth.dense_2b_tensor_shapes())
    log("dense 2B: generating 16 bf16 clients in one staggered allocation")
    arena, views = fa.client_arena(K + 1, N, torch.bfloat16)
    n, xs = sd.dense_2b(K=K, N=N, dest=views[:K])
    out = views[K]
    nl = n.tolist()
    log(f"dense 2B: K={K} N={N} timing {steps} steps")
    wall, durs = timed(lambda i: fa.fedavg_aggregate(xs, nl, out), steps, warmup)
    out_hash = fa.fedavg_checksum(out)
    log("dense 2B: the same clients in separate allocations")
    sep = [x.clone() for x in xs]
    out_sep = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    _, durs_sep = timed(lambda i: fa.fedavg_aggregate(sep, nl, out_sep), steps, warmup)
    same = bool(torch.equal(out.view(torch.int16), out_sep.view(torch.int16)))
    del xs, out, views, arena, sep, out_sep
    free_gpu()
    assert same, "the two layouts gave different outputs"
    algo_bytes = (K + 1) * 2 * N
    st, st_sep = stats(durs), stats(durs_sep)
    return {
        "K": K, "N": N, "wall_s": wall, "avg_launch_ms": st["mean_ms"], "min_launch_ms": st["min_ms"],
        "median_launch_ms": st["median_ms"], "algo_bytes": algo_bytes, "out_checksum": f"{out_hash:016x}",
        "separate_allocations": {"avg_launch_ms": st_sep["mean_ms"], "median_launch_ms": st_sep["median_ms"],
                                 "min_launch_ms": st_sep["min_ms"],
                                 "hbm_frac": algo_bytes / (st_sep["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "same_output": same},
    }


# --------------------------------------------------------------------------
# other modes
# --------------------------------------------------------------------------

def bench_dense_small(reps=2000, replicas=64):
    import torch
    import synth.device as sd
    import weighted_model_update_amd as fa
    n, xs = sd.dense_small()
    N = xs[0].numel()
    sets = [[x.clone() for x in xs] for _ in range(replicas)]     # 64 x 12 MB: beyond the caches
    outs = [torch.empty(N, dtype=torch.float32, device="cuda") for _ in range(replicas)]
    nl = n.tolist()
    fn = lambda i: fa.fedavg_aggregate(sets[i % replicas], nl, outs[i % replicas])
    for i in range(50):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(reps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1000.0 / reps
    # the same calls captured once in a HIP graph (one call per replica set)
    # and replayed: what a caller that aggregates in a loop can reach
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(replicas):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(replicas):
            fn(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    greps = max(1, reps // replicas)
    s.record()
    for _ in range(greps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    us_graph = s.elapsed_time(e) * 1000.0 / (greps * replicas)
    bytes_ = 4 * 4 * N
    del sets, outs, g
    free_gpu()
    return {"K": 3, "N": N, "dtype": "f32", "us_per_call": us, "algo_bytes": bytes_,
            "hbm_gbs": bytes_ / (us * 1e-6) / 1e9, "params_per_s": 3 * N / (us * 1e-6),
            "us_per_call_graph": us_graph, "hbm_gbs_graph": bytes_ / (us_graph * 1e-6) / 1e9,
            "replica_sets": replicas,
            "note": "launch-latency bound: 16 MB of traffic is 2 us at 8 TB/s; the graph figure "
                    "replays the calls captured once"}


def bench_adapter(reps=400, replicas=4):
    import numpy as np
    import torch
    import synth.device as sd
    import weighted_model_update_amd as fa
    n, xs, base, bounds, present = sd.adapter()
    K, N = len(xs), xs[0].numel()
    seg = np.diff(bounds)
    sent_params = int((present * seg[None, :]).sum())
    nobody = int(seg[present.sum(0) == 0].sum())
    algo_bytes = 2 * sent_params + 2 * N + 2 * nobody
    d_bounds = torch.from_numpy(bounds).cuda()
    d_present = torch.from_numpy(np.ascontiguousarray(present, np.uint8)).cuda()
    sets = [([x.clone() for x in xs], base.clone()) for _ in range(replicas)]   # > 2x the 256 MB MALL
    outs = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(replicas)]
    nl = n.tolist()

    def fn(i):
        c, b = sets[i % replicas]
        fa.fedavg_aggregate(c, nl, outs[i % replicas], base=b, seg_bounds=d_bounds, present=d_present)

    for i in range(20):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(reps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1000.0 / reps
    # per-launch events as well, for the median and the minimum
    _, d = timed(fn, reps, 0)
    st = stats(d)
    # the calls captured once in a HIP graph (one per replica set) and replayed
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(replicas):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(replicas):
            fn(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    greps = max(1, reps // replicas)
    s.record()
    for _ in range(greps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    us_graph = s.elapsed_time(e) * 1000.0 / (greps * replicas)
    del sets, outs, xs, base, g
    free_gpu()
    return {"K": K, "N": N, "dtype": "bf16", "segments": int(len(seg)),
            "client_segments_sent": int(present.sum()), "us_per_call": us,
            "algo_bytes": algo_bytes, "hbm_gbs": algo_bytes / (us * 1e-6) / 1e9,
            "hbm_frac": algo_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "params_per_s": sent_params / (us * 1e-6), "replica_sets": replicas,
            "median_us_per_launch": st["median_ms"] * 1e3, "min_us_per_launch": st["min_ms"] * 1e3,
            "hbm_frac_median_launch": algo_bytes / (st["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "us_per_call_graph": us_graph,
            "hbm_frac_graph": algo_bytes / (us_graph * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "note": "us_per_call: back-to-back launches between two events; the graph figure "
                    "replays the calls captured once"}


def bench_streaming(clients=32, slots=3):
    import torch
    import synth.device as sd
    import synth
    import weighted_model_update_amd as fa
    chunk_bytes = synth.CHUNK_BYTES_8B
    per = chunk_bytes // 2
    log("streaming: building the pinned 4 GiB chunk pool and the 8B bf16 base")
    pool = sd.stream_8b_pool()
    P = pool.shape[0]
    base = sd.stream_8b_base()
    N = base.numel()
    n = sd.stream_8b_counts(32)[:clients]
    cpc = (N + per - 1) // per
    acc_b, _, _, stag_b = fa.fedavg_workspace_size(N, 0, chunk_bytes, slots)
    acc = torch.empty(acc_b // 4, dtype=torch.float32, device="cuda")
    staging = torch.empty(stag_b, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()

    def one_pass(n_clients):
        h = fa.fedavg_begin(N, "deltas", False, acc, None, None, staging, chunk_bytes, slots,
                            copy_stream=copy_stream)
        for k in range(n_clients):
            for c in range(cpc):
                off = c * per
                ln = min(per, N - off)
                fa.fedavg_accumulate(h, k, int(n[k]), pool[sd.pool_index(k, c, cpc, P)][:ln], off)
        fa.fedavg_finalize(h, base, base)        # in place: global += weighted mean delta
        fa.fedavg_sync(h)
        fa.fedavg_destroy(h)

    log("streaming: warm-up pass with 1 client")
    one_pass(1)
    torch.cuda.synchronize()
    log(f"streaming: timed pass, {clients} clients x {cpc} chunks")
    t0 = time.perf_counter()
    one_pass(clients)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pcie_bytes = 2 * N * clients

    # the accumulate kernel alone, chunks already in HBM
    dchunk = pool[0].cuda()
    h = fa.fedavg_begin(N, "deltas", False, acc, None, None, staging, chunk_bytes, slots)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fa.fedavg_accumulate(h, 0, 1, dchunk, 0)
    torch.cuda.synchronize()
    s.record()
    for c in range(1, cpc - 1):
        fa.fedavg_accumulate(h, 0, 1, dchunk, c * per)
    e.record()
    torch.cuda.synchronize()
    k_us = s.elapsed_time(e) * 1000.0 / (cpc - 2)
    fa.fedavg_destroy(h)
    k_bytes = 10 * per                      # bf16 chunk read + fp32 acc read and write
    del pool, base, acc, staging, dchunk
    free_gpu()
    return {"K": clients, "N": N, "dtype": "bf16 in, fp32 accumulator", "chunk_bytes": chunk_bytes,
            "staging_slots": slots, "wall_s": wall, "pcie_bytes": pcie_bytes,
            "pcie_gbs": pcie_bytes / wall / 1e9, "pcie_frac": pcie_bytes / wall / 1e9 / PCIE_PEAK_GBS,
            "params_per_s": N * clients / wall,
            "accumulate_kernel": {"us_per_chunk": k_us, "algo_bytes": k_bytes,
                                  "hbm_gbs": k_bytes / (k_us * 1e-6) / 1e9,
                                  "hbm_frac": k_bytes / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS}}


def bench_hierarchical(silos=4):
    """Two-level aggregation at the 8B streaming workload's size: the top-level
    accumulator takes `silos` silo partials (fp32 sums over all N parameters,
    already in HBM) as pseudo-clients; each merge reads the partial and
    reads and writes the accumulator (12 B per parameter)."""
    import torch
    import synth
    import weighted_model_update_amd as fa
    N = synth.numel_of(synth.stream_8b_tensor_shapes())
    log(f"hierarchical: {silos} silo partials of {N} fp32 sums")
    acc_b, _, _, stag_b = fa.fedavg_workspace_size(N, 0, 1 << 20, 1)
    acc = torch.empty(acc_b // 4, dtype=torch.float32, device="cuda")
    staging = torch.empty(stag_b, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(2026)
    part = torch.empty(N, dtype=torch.float32, device="cuda")
    part.normal_(0.0, 1.0, generator=g)
    W = [int(w) for w in synth.sample_counts(synth.CFG_STREAM_8B, silos, 1000, 80000)]
    h = fa.fedavg_begin(N, "deltas", False, acc, None, None, staging, 1 << 20, 1)
    fa.fedavg_accumulate_partial(h, 0, W[0], 8, part, offset=0)       # warm-up merge
    torch.cuda.synchronize()
    fa.fedavg_destroy(h)
    h = fa.fedavg_begin(N, "deltas", False, acc, None, None, staging, 1 << 20, 1)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for k in range(silos):
        fa.fedavg_accumulate_partial(h, k, W[k], 8, part, offset=0)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / silos
    fa.fedavg_destroy(h)
    algo = 12 * N
    del acc, staging, part
    free_gpu()
    return {"silos": silos, "N": N, "dtype": "fp32 partial sums", "ms_per_merge": ms,
            "algo_bytes_per_merge": algo, "hbm_gbs": algo / (ms * 1e-3) / 1e9,
            "hbm_frac": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_topk(steps=10, warmup=2):
    """Client-side top-10% selection over one 10^9-parameter fp32 update
    (Laplace(0, 1e-3) deltas): sampled threshold range, one split pass with
    staging, radix select over the candidates, tile counts, offset scan and
    ordered write, timed as one call.  Algorithmic bytes: one read of the
    update (4 B per parameter) and the kept (int64 index, fp32 value) pairs."""
    import torch
    import synth.device as sd
    import weighted_model_update_amd as fa
    N = 10 ** 9
    log("topk: generating a 10^9-parameter Laplace client update")
    x = sd.client_delta_1b(0, N)
    k = fa.topk_count(N, 0.1)
    idx = torch.empty(k, dtype=torch.int64, device="cuda")
    val = torch.empty(k, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.topk_workspace_size(N, k, x.dtype), dtype=torch.uint8, device="cuda")
    fn = lambda i: fa.topk_select(x, k, idx, val, ws)
    _, times = timed(fn, steps, warmup)
    st = stats(times)
    ms = st["mean_ms"]
    algo = 4 * N + 12 * k
    del x, idx, val, ws
    free_gpu()
    return {"N": N, "k": k, "dtype": "f32", "ms_per_call": ms, "algo_bytes": algo,
            "hbm_gbs": algo / (ms * 1e-3) / 1e9, "hbm_frac": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "params_per_s": N / (ms * 1e-3), "input_passes": 1, "median_ms": st["median_ms"],
            "min_ms": st["min_ms"],
            "note": "a 2^20-key sample bounds the threshold; one pass over the update counts the "
                    "keys above the range, compacts the candidates inside it and stages every "
                    "entry at or above its floor; the radix digits and tile counts read only the "
                    "candidates, and the ordered write reads the staged entries"}


def bench_windows(clients=32, windows=4, slots=3):
    """The 8B streaming workload with the accumulator cut into `windows`
    windows of the parameter space (stream_windows: for models whose fp32
    accumulator does not fit in HBM): every client's chunks are streamed once
    per window, clipped to it, so the PCIe bytes equal the single-handle
    run's."""
    import torch
    import synth.device as sd
    import synth
    import weighted_model_update_amd as fa
    chunk_bytes = synth.CHUNK_BYTES_8B
    per = chunk_bytes // 2
    log(f"windows: the 8B streaming workload in {windows} windows")
    pool = sd.stream_8b_pool()
    P = pool.shape[0]
    base = sd.stream_8b_base()
    N = base.numel()
    n = sd.stream_8b_counts(32)[:clients]
    cpc = (N + per - 1) // per
    window = -(-N // windows)

    def chunks_of(k):
        def gen():
            for c in range(cpc):
                off = c * per
                yield off, pool[sd.pool_index(k, c, cpc, P)][:min(per, N - off)]
        return gen

    fa.stream_windows(N, [(0, int(n[0]), chunks_of(0))], base, base, window=window, mode="deltas",
                      chunk_bytes=chunk_bytes, n_slots=slots)                       # warm-up, 1 client
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    nw = fa.stream_windows(N, [(k, int(n[k]), chunks_of(k)) for k in range(clients)], base, base,
                           window=window, mode="deltas", chunk_bytes=chunk_bytes, n_slots=slots)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pcie_bytes = 2 * N * clients
    del pool, base
    free_gpu()
    return {"K": clients, "N": N, "windows": nw, "window_params": window,
            "accumulator_bytes_per_window": 4 * window, "wall_s": wall, "pcie_bytes": pcie_bytes,
            "pcie_gbs": pcie_bytes / wall / 1e9, "pcie_frac": pcie_bytes / wall / 1e9 / PCIE_PEAK_GBS}


def bench_sparse(steps=10, warmup=2):
    import torch
    import synth.device as sd
    import weighted_model_update_amd as fa
    log("sparse: generating 20 top-10% client lists over 10^9 parameters")
    n, idx, val, base = sd.sparse_1b()
    K, N = len(idx), base.numel()
    nnz = sum(int(i.numel()) for i in idx)
    out = torch.empty(N, dtype=torch.float32, device="cuda")
    counts = torch.empty(N, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(fa.sparse_workspace_size(K, N), dtype=torch.uint8, device="cuda")
    nl = n.tolist()
    fn = lambda i: fa.sparse_masked_accumulate(idx, val, nl, N, base, out, counts=counts, workspace=ws,
                                               err_flag=err)
    wall, durs = timed(fn, steps, warmup)
    assert int(err.item()) == 0
    algo = 12 * nnz + 9 * N
    st = stats(durs)
    avg = st["mean_ms"]
    del idx, val, base, out, counts, ws
    free_gpu()
    return {"K": K, "N": N, "dtype": "f32", "pairs": nnz, "ms_per_call": avg, "algo_bytes": algo,
            "hbm_gbs": algo / (avg * 1e-3) / 1e9, "hbm_frac": algo / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "params_per_s": nnz / (avg * 1e-3), "median_ms": st["median_ms"], "min_ms": st["min_ms"],
            "hbm_frac_median": algo / (st["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}


def bench_sparse_stream(clients=20):
    """Client-at-a-time sparse accumulate: the 10^9-parameter top-10% lists
    of the sparse workload, each client's (index, value) pairs entered into
    the streaming accumulator in partial mode (fp32 sum, uint32 weight sum,
    uint8 count per parameter), then one finalize.  Pair-level bytes are 12 B
    read plus 18 B of read-modify-write per pair; DRAM moves whole lines, so
    the line-level figure counts every 64-byte line of the three arrays a
    client touches, read and written, plus the pairs.  The default path
    reads and writes the accumulator in dense tiles at this density; the
    scatter path (FA_OPT_INDEX_TILES = 1) is timed on the same lists."""
    import torch
    import synth.device as sd
    import weighted_model_update_amd as fa
    log("sparse_stream: generating 20 top-10% client lists over 10^9 parameters")
    n, idx, val, base = sd.sparse_1b(K=clients)
    K, N = len(idx), base.numel()
    nnz = [int(i.numel()) for i in idx]
    lines = []
    for i in idx:
        lines.append(int(torch.unique_consecutive(i // 16).numel()) * 2 * 64 * 2   # acc, wsum
                     + int(torch.unique_consecutive(i // 64).numel()) * 64 * 2)    # count
    out = torch.empty(N, dtype=torch.float32, device="cuda")

    def run(path):
        fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, path)
        times = []
        try:
            with fa.StreamingAccumulator(N, mode="deltas", partial=True, chunk_bytes=1 << 20, n_slots=2) as acc:
                for k in range(K):
                    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s.record()
                    acc.accumulate(k, int(n[k]), val[k], indices=idx[k])
                    e.record()
                    times.append((s, e))
                fs, fe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                fs.record()
                acc.finalize(base, out)
                fe.record()
                acc.sync()
        finally:
            fa.fedavg_set_option(fa.FA_OPT_INDEX_TILES, 0)
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) for a, b in times[1:]]     # the first client warms up
        return sum(per) / len(per), fs.elapsed_time(fe)

    ms, fin_ms = run(0)
    ms_scatter, _ = run(1)
    pair_bytes = 30 * sum(nnz[1:]) / (K - 1)
    line_bytes = (12 * sum(nnz[1:]) + sum(lines[1:])) / (K - 1)
    del idx, val, base, out
    free_gpu()
    return {"K": K, "N": N, "pairs_per_client": nnz[0], "ms_per_client": ms,
            "pair_bytes_per_client": pair_bytes, "line_bytes_per_client": line_bytes,
            "hbm_gbs_lines": line_bytes / (ms * 1e-3) / 1e9,
            "hbm_frac_lines": line_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_per_client_scatter": ms_scatter,
            "hbm_frac_lines_scatter": line_bytes / (ms_scatter * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "finalize_ms": fin_ms, "finalize_bytes": 13 * N,
            "note": "default path: each client's list is checked, then the accumulator's tiles holding it "
                    "are read and written whole (about 19 GB per client at this density, the sums and "
                    "weight sums of 64-byte runs no entry touched not written); the scatter path moves "
                    "the touched lines as scattered read-modify-writes; the one-pass sparse merge "
                    "(mode sparse) avoids both"}


def bench_checksum(reps=10):
    """Checksum of a 10^9-parameter fp32 buffer: one read, 4 B per element."""
    import torch
    import weighted_model_update_amd as fa
    N = 10 ** 9
    x = torch.empty(N, dtype=torch.float32, device="cuda")
    x.normal_()
    h = torch.zeros(1, dtype=torch.int64, device="cuda")
    _, durs = timed(lambda i: fa.fedavg_checksum(x, hash_out=h), reps, 2)
    ms = sum(durs) / len(durs)
    # the same read giving the hash and the fixed-order fp64 value sum, and
    # the sum alone (each call: the tile pass plus a one-block finish)
    ws = torch.empty(fa.fedavg_sum_workspace_size(N), dtype=torch.uint8, device="cuda")
    sm = torch.zeros(1, dtype=torch.float64, device="cuda")
    _, d2 = timed(lambda i: fa.fedavg_checksum_sum(x, workspace=ws, hash_out=h, sum_out=sm), reps, 2)
    _, d3 = timed(lambda i: fa.fedavg_checksum_sum(x, workspace=ws, sum_out=sm), reps, 2)
    ms2, ms3 = sum(d2) / len(d2), sum(d3) / len(d3)
    del x, h, ws, sm
    free_gpu()
    gbs = lambda m: 4 * N / (m * 1e-3) / 1e9
    return {"N": N, "dtype": "f32", "ms_per_call": ms, "algo_bytes": 4 * N,
            "hbm_gbs": gbs(ms), "hbm_frac": gbs(ms) / HBM_PEAK_GBS,
            "hash_and_sum_ms_per_call": ms2, "hash_and_sum_hbm_frac": gbs(ms2) / HBM_PEAK_GBS,
            "sum_ms_per_call": ms3, "sum_hbm_frac": gbs(ms3) / HBM_PEAK_GBS}


def bench_copy_calibration(gib=4):
    """A plain device copy of known size, so hardware byte counters can be
    scaled: the library's element copy (the no-contributor path of
    fedavg_aggregate, convert_kernel<f32,f32>) reads and writes exactly
    `gib` GiB."""
    import torch
    import weighted_model_update_amd as fa
    n = (gib << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dummy = torch.empty(n, dtype=torch.float32, device="cuda")
    for _ in range(3):
        fa.fedavg_aggregate([dummy], [0], dst, mode="deltas", base=src)
    torch.cuda.synchronize()
    del src, dst, dummy
    free_gpu()
    return {"kernel": "convert_kernel<0, 0>", "bytes_read": gib << 30, "bytes_written": gib << 30,
            "launches": 3}


def bench_dense_k(Ks=(4, 8, 16, 20, 32, 64), total_bytes=65_343_852_544, reps=10, warmup=2):
    """Resident dense aggregation at runtime client counts: K bf16 clients
    and a bf16 output of N parameters each, N chosen so the (K+1)*2*N bytes
    match the 2.0B K=16 workload's 65.3 GB.  K = 3, 8 and 16 have kernels
    of their own; the others take the generic kernel (clients in batches of
    8, of 16 above 16 clients).  The residency cap follows the client count
    (the library's default).  Values do not change the time, so the clients are filled with a
    constant.  Each K runs with separate allocations and again with the
    clients and output in one arena_layout allocation."""
    import torch
    import weighted_model_update_amd as fa
    rows = []
    for K in Ks:
        N = total_bytes // ((K + 1) * 2) // 256 * 256
        xs = [torch.full((N,), 0.01 * (k + 1), dtype=torch.bfloat16, device="cuda") for k in range(K)]
        out = torch.empty(N, dtype=torch.bfloat16, device="cuda")
        n = [100 + 37 * k for k in range(K)]
        _, d = timed(lambda i: fa.fedavg_aggregate(xs, n, out), reps, warmup)
        st = stats(d)
        del xs, out
        free_gpu()
        arena, views = fa.client_arena(K + 1, N, torch.bfloat16)
        for k in range(K):
            views[k].fill_(0.01 * (k + 1))
        _, d = timed(lambda i: fa.fedavg_aggregate(views[:K], n, views[K]), reps, warmup)
        sta = stats(d)
        del arena, views
        free_gpu()
        nb = (K + 1) * 2 * N
        rows.append({"K": K, "N": N, "bytes": nb, **st,
                     "hbm_gbs_median": nb / (st["median_ms"] * 1e-3) / 1e9,
                     "hbm_frac_median": nb / (st["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "params_per_s_median": K * N / (st["median_ms"] * 1e-3),
                     "arena_median_ms": sta["median_ms"], "arena_min_ms": sta["min_ms"],
                     "arena_hbm_frac_median": nb / (sta["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "kernel": ("dense_vec_kernel<K>" if K in (3, 8, 16) else
                                "dense_vec_kernel<batches of 16>" if K > 16 else "dense_vec_kernel<batches of 8>")})
        log(f"dense K={K}: {st['median_ms']:.3f} ms median, {rows[-1]['hbm_frac_median']:.3f} of peak; "
            f"in an arena {sta['median_ms']:.3f} ms, {rows[-1]['arena_hbm_frac_median']:.3f}")
    return {"rows": rows}


def bench_streaming_chunks(chunk_mib=(16, 64, 256), slots=(2, 3, 4), clients=4):
    """Chunk size against staging slots for the streaming path: the 8B bf16
    workload's first `clients` clients streamed from pinned host memory in
    chunks of each size, through 2, 3 or 4 staging slots (chunk size trades
    request overhead against per-chunk memory: FLARE page, Tensor
    Downloader).  Chunks come from a pinned pool of 4 GiB cut at each size."""
    import torch
    import synth
    import synth.device as sd
    import weighted_model_update_amd as fa
    base = sd.stream_8b_base()
    N = base.numel()
    n = sd.stream_8b_counts(32)[:clients]
    pool = sd.stream_8b_pool().view(-1)           # 4 GiB of distinct bf16 deltas
    rows = []
    acc_b, _, _, _ = fa.fedavg_workspace_size(N, 0, 1 << 20, 1)
    acc = torch.empty(acc_b // 4, dtype=torch.float32, device="cuda")
    copy_stream = torch.cuda.Stream()
    for mib in chunk_mib:
        per = (mib << 20) // 2
        P = pool.numel() // per
        chunks = pool[:P * per].view(P, per)
        cpc = (N + per - 1) // per
        for sl in slots:
            _, _, _, stag_b = fa.fedavg_workspace_size(N, 0, mib << 20, sl)
            staging = torch.empty(stag_b, dtype=torch.uint8, device="cuda")

            def one_pass(nc):
                h = fa.fedavg_begin(N, "deltas", False, acc, None, None, staging, mib << 20, sl,
                                    copy_stream=copy_stream)
                for k in range(nc):
                    for c in range(cpc):
                        off = c * per
                        fa.fedavg_accumulate(h, k, int(n[k]), chunks[(k * cpc + c) * 37 % P][:min(per, N - off)],
                                             off)
                fa.fedavg_finalize(h, base, base)
                fa.fedavg_sync(h)
                fa.fedavg_destroy(h)

            one_pass(1)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            one_pass(clients)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            pb = 2 * N * clients
            rows.append({"chunk_mib": mib, "slots": sl, "clients": clients, "wall_s": wall,
                         "pcie_gbs": pb / wall / 1e9, "pcie_frac": pb / wall / 1e9 / PCIE_PEAK_GBS,
                         "staging_bytes": stag_b})
            log(f"streaming {mib} MiB x {sl} slots: {pb / wall / 1e9:.1f} GB/s")
            del staging
    del base, pool, acc, chunks
    free_gpu()
    return {"N": N, "rows": rows}


def bench_spill(gib=1):
    """Spill and resume of a streaming aggregate (FLARE page, "Offload
    Aggregation to Disk"): a partial-mode accumulator of gib GiB of fp32
    sums (plus its uint32 weight sums and uint8 counts) written to a
    directory under the temporary directory with StreamingAccumulator.save
    and read back with load.  Reported: bytes per second for each, and for
    the device-to-pinned-host copies alone (the library's side of it)."""
    import shutil
    import tempfile
    import torch
    import weighted_model_update_amd as fa
    N = (gib << 30) // 4
    d = tempfile.mkdtemp(prefix="fedavg_spill_")
    try:
        acc = fa.StreamingAccumulator(N, mode="deltas", partial=True, chunk_bytes=1 << 20, n_slots=2)
        x = torch.full((N,), 0.5, dtype=torch.float32, device="cuda")
        acc.accumulate(0, 3, x, offset=0)
        acc.sync()
        nbytes = 9 * N
        t0 = time.perf_counter()
        acc.save(d)
        t_save = time.perf_counter() - t0
        acc.close()
        del acc
        t0 = time.perf_counter()
        back = fa.StreamingAccumulator.load(d, N, mode="deltas", partial=True, chunk_bytes=1 << 20, n_slots=2)
        torch.cuda.synchronize()
        t_load = time.perf_counter() - t0
        ok = bool(torch.equal(back.acc[:N], torch.full((N,), 1.5, dtype=torch.float32, device="cuda")))
        back.close()
        # the device <-> pinned host copies alone, 64 MiB at a time
        bounce = torch.empty(64 << 20, dtype=torch.uint8, pin_memory=True)
        flat = x.view(torch.uint8)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for off in range(0, flat.numel(), bounce.numel()):
            m = min(bounce.numel(), flat.numel() - off)
            bounce[:m].copy_(flat[off:off + m])
        t_d2h = time.perf_counter() - t0
        del x, flat, bounce
    finally:
        shutil.rmtree(d, ignore_errors=True)
        free_gpu()
    return {"N": N, "bytes": nbytes, "save_s": t_save, "save_gbs": nbytes / t_save / 1e9,
            "load_s": t_load, "load_gbs": nbytes / t_load / 1e9, "resumed_bits_ok": ok,
            "d2h_pinned_gbs": 4 * N / t_d2h / 1e9,
            "where": "a directory under the temporary directory of the host"}


# --------------------------------------------------------------------------
# HBM ceilings of the dense pattern
# --------------------------------------------------------------------------

# Pol codes of the ceiling kernels (csrc/hbm_ceiling.hip)
P_GLOBAL, P_GLOBAL_NT, P_BUF, P_BUF_NT, P_BUF_SC1, P_BUF_SC0SC1, P_BUF_SC1NT, P_BUF_SC0SC1NT = range(8)
POL_NAMES = ["global", "global nt", "buffer", "buffer nt", "buffer sc1", "buffer sc0 sc1",
             "buffer sc1 nt", "buffer sc0 sc1 nt"]
# (name, pattern 0 read / 1 read+write, streams read, load policy, store policy, vectors per thread)
CEILING_CASES = [
    ("read16 nt", 0, 16, P_GLOBAL_NT, P_GLOBAL, 1),
    ("read16", 0, 16, P_GLOBAL, P_GLOBAL, 1),
    ("read17 nt", 0, 17, P_GLOBAL_NT, P_GLOBAL, 1),
    ("read17", 0, 17, P_GLOBAL, P_GLOBAL, 1),
    ("copy nt/nt", 1, 1, P_GLOBAL_NT, P_GLOBAL_NT, 1),
    ("copy plain/plain", 1, 1, P_GLOBAL, P_GLOBAL, 1),
    ("copy nt/plain", 1, 1, P_GLOBAL_NT, P_GLOBAL, 1),
    ("copy nt/nt vpt4", 1, 1, P_GLOBAL_NT, P_GLOBAL_NT, 4),
    ("mix2 nt/nt", 1, 2, P_GLOBAL_NT, P_GLOBAL_NT, 1),
    ("mix4 nt/nt", 1, 4, P_GLOBAL_NT, P_GLOBAL_NT, 1),
    ("mix8 nt/nt", 1, 8, P_GLOBAL_NT, P_GLOBAL_NT, 1),
    ("mix16 nt/nt", 1, 16, P_GLOBAL_NT, P_GLOBAL_NT, 1),
    ("mix16 plain/nt", 1, 16, P_GLOBAL, P_GLOBAL_NT, 1),
    ("mix16 buf/nt", 1, 16, P_BUF, P_GLOBAL_NT, 1),
    ("mix16 buf nt/nt", 1, 16, P_BUF_NT, P_GLOBAL_NT, 1),
    ("mix16 buf sc1/nt", 1, 16, P_BUF_SC1, P_GLOBAL_NT, 1),
    ("mix16 buf sc0sc1/nt", 1, 16, P_BUF_SC0SC1, P_GLOBAL_NT, 1),
    ("mix16 buf sc1nt/nt", 1, 16, P_BUF_SC1NT, P_GLOBAL_NT, 1),
    ("mix16 nt/plain", 1, 16, P_GLOBAL_NT, P_GLOBAL, 1),
    ("mix16 nt/buf", 1, 16, P_GLOBAL_NT, P_BUF, 1),
    ("mix16 nt/buf nt", 1, 16, P_GLOBAL_NT, P_BUF_NT, 1),
    ("mix16 nt/buf sc1", 1, 16, P_GLOBAL_NT, P_BUF_SC1, 1),
    ("mix16 nt/buf sc0sc1", 1, 16, P_GLOBAL_NT, P_BUF_SC0SC1, 1),
    ("mix16 nt/buf sc1nt", 1, 16, P_GLOBAL_NT, P_BUF_SC1NT, 1),
    ("mix16 nt/buf sc0sc1nt", 1, 16, P_GLOBAL_NT, P_BUF_SC0SC1NT, 1),
    ("mix16 buf nt/buf nt", 1, 16, P_BUF_NT, P_BUF_NT, 1),
    ("mix16 buf nt/buf sc1nt", 1, 16, P_BUF_NT, P_BUF_SC1NT, 1),
    ("mix16 nt/nt vpt2", 1, 16, P_GLOBAL_NT, P_GLOBAL_NT, 2),
    ("mix16 nt/nt vpt4", 1, 16, P_GLOBAL_NT, P_GLOBAL_NT, 4),
    ("mix16 nt/plain vpt2", 1, 16, P_GLOBAL_NT, P_GLOBAL, 2),
    ("mix16 nt/plain vpt4", 1, 16, P_GLOBAL_NT, P_GLOBAL, 4),
]


def bench_ceiling(reps=10, warmup=2, residents=(2, 0, 1, 3, 4)):
    """What HBM gives the headline's byte pattern on this part, measured in
    the same run as the headline kernel: kernels that move the dense
    aggregation's bytes (16 bf16 client streams of 1,921,878,016 parameters
    read, one written) with no arithmetic, over load and store cache
    policies, write batching and residency caps; the 16- and 17-stream reads
    alone and a plain copy bound it from both sides.  The dense kernel itself
    is timed on the same buffers at each residency cap.  The 17 buffers lie
    in one allocation placed by arena_layout, as the headline's do."""
    import ctypes
    import torch
    import synth
    import weighted_model_update_amd as fa
    from weighted_model_update_amd import build as nb
    lib = ctypes.CDLL(nb.CEILING_PATH)
    lib.hc_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                              ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int64, ctypes.c_void_p]
    lib.hc_stream.restype = ctypes.c_int
    N = synth.numel_of(synth.dense_2b_tensor_shapes())
    nvec = N * 2 // 16
    log(f"ceiling: 17 streams of {nvec * 16} bytes")
    # laid out as the headline's clients and output are (arena_layout)
    arena, bufs = fa.client_arena(17, nvec * 16, torch.uint8)
    for i, b in enumerate(bufs):
        b.view(torch.int32).fill_(0x3c003c00 + i)        # bf16 values near 1, distinct per stream
    srcs = (ctypes.c_void_p * 17)(*[b.data_ptr() for b in bufs])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rows = []

    def record(name, pattern, ns, lp, sp, vpt, res, fn, nbytes):
        _, d = timed(fn, reps, warmup)
        st = stats(d)
        rows.append({"name": name, "streams_read": ns, "stream_written": pattern == 1,
                     "load": POL_NAMES[lp] if lp is not None else "kernel",
                     "store": POL_NAMES[sp] if sp is not None else "kernel",
                     "vectors_per_thread": vpt, "resident_per_cu": res, "bytes": nbytes, **st,
                     "gbs_median": nbytes / (st["median_ms"] * 1e-3) / 1e9,
                     "frac_median": nbytes / (st["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "frac_min_time": nbytes / (st["min_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS})

    for res in residents:
        for name, pattern, ns, lp, sp, vpt in CEILING_CASES:
            if res != residents[0] and not name.startswith(("mix", "read16 nt", "copy nt/nt")):
                continue        # the policy sweep runs at the default cap only
            if (res != residents[0] and name.startswith("mix16") and "nt/nt" not in name
                    and name != "mix16 buf nt/buf sc1nt"):
                continue
            dst = bufs[16].data_ptr() if ns < 17 else bufs[0].data_ptr()
            nb_ = (ns + (1 if pattern == 1 else 0)) * nvec * 16

            def fn(i, pattern=pattern, ns=ns, lp=lp, sp=sp, vpt=vpt, res=res, dst=dst):
                rc = lib.hc_stream(pattern, ns, srcs, ctypes.c_void_p(dst), nvec, lp, sp, vpt, res, 0,
                                   stream)
                if rc != 0:
                    raise RuntimeError(f"hc_stream failed: {rc}")
            record(name, pattern, ns, lp, sp, vpt, res, fn, nb_)
        # the dense aggregation kernel itself on the same buffers
        xs = [b.view(torch.bfloat16) for b in bufs[:16]]
        out = bufs[16].view(torch.bfloat16)
        n = [int(v) for v in synth.sample_counts(synth.CFG_DENSE_2B, 16, 100, 1000)]
        fa.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, res)
        try:
            record("dense kernel K=16 bf16", 1, 16, None, None, 1, res,
                   lambda i: fa.fedavg_aggregate(xs, n, out), 17 * 2 * N)
        finally:
            fa.fedavg_set_option(fa.FA_OPT_RESIDENT_PER_CU, -1)
        log(f"ceiling: resident {res} done")
    del bufs, arena
    free_gpu()
    mixed = [r for r in rows if r["streams_read"] == 16 and r["stream_written"] and r["load"] != "kernel"]
    best = min(mixed, key=lambda r: r["median_ms"])
    dense_default = [r for r in rows if r["name"].startswith("dense kernel")
                     and r["resident_per_cu"] == residents[0]][0]
    return {"N": N, "bytes_per_stream": nvec * 16, "rows": rows,
            "best_mixed": {"name": best["name"], "resident_per_cu": best["resident_per_cu"],
                           "median_ms": best["median_ms"], "frac_median": best["frac_median"]},
            "dense_median_ms": dense_default["median_ms"],
            "dense_over_best_mixed": dense_default["median_ms"] / best["median_ms"]}


# --------------------------------------------------------------------------
# CPU oracle baseline
# --------------------------------------------------------------------------

def _time_oracle(fn, units, budget_s):
    """Calls fn() until budget_s has passed (at least once); returns units
    per second and the number of calls."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return units * reps / el, reps


def cpu_baseline(budget_s=2.0):
    """The oracle (plain C, fp64, OpenMP over parameters) timed on this
    host, on every host thread and on one, for the small dense, adapter,
    2.0B dense and sparse workloads, each on a bounded sample of the
    workload (whole for the two small ones).  Inputs are host-generated with
    the same distributions, already in host memory when the clock starts;
    the unit is aggregated params/s (parameters the clients contributed, per
    second), the headline's unit."""
    import numpy as np
    import oracle
    import synth
    all_threads = oracle.set_threads(0)
    host = {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "omp_threads": all_threads}
    log(f"cpu baseline: oracle on {all_threads} threads and on 1 (host nproc {host['nproc']})")
    cases = {}

    # small dense: K=3 fp32 clients of 10^6, whole
    K, N = 3, 1_000_000
    xs = synth.dense_clients_f32(synth.CFG_DENSE_SMALL, K, N, 0.02)
    n = synth.sample_counts(synth.CFG_DENSE_SMALL, K, 100, 1000)
    cases["dense_small"] = (lambda: oracle.weighted_average(xs, n), K * N,
                            "whole workload: K=3 fp32 clients of 1,000,000 parameters")

    # adapters: K=8 LoRA q,k,v,o adapters of 32 layers, whole, per-module masks
    bounds, module_of = synth.adapter_segments()
    bounds = np.asarray(bounds, np.int64)
    Na, Ka = int(bounds[-1]), 8
    na = synth.sample_counts(synth.CFG_ADAPTER, Ka, 500, 5000)
    pres = synth.adapter_presence(synth.CFG_ADAPTER, Ka, max(module_of) + 1, 0.6)[:, module_of]
    seg_of = np.repeat(np.arange(len(bounds) - 1), np.diff(bounds))
    sent = [np.ascontiguousarray(pres[k][seg_of], np.uint8) for k in range(Ka)]
    xa = [synth.bf16_bits_from_f32(synth.normal_f32(synth.CFG_ADAPTER, synth.ROLE_VALUES, k, Na, 0.01))
          for k in range(Ka)]
    ba = synth.bf16_bits_from_f32(synth.normal_f32(synth.CFG_ADAPTER, synth.ROLE_BASE, 0, Na, 0.01))
    sent_params = int(sum(s_.sum(dtype=np.int64) for s_ in sent))
    cases["adapter"] = (lambda: oracle.weighted_average(xa, na, base=ba, x_dtype=oracle.BF16,
                                                        base_dtype=oracle.BF16, sent=sent),
                        sent_params, "whole workload: K=8 clients, 16,777,216 bf16 parameters, "
                                     "Bernoulli(0.6) module masks")

    # 2.0B dense: K=16 bf16, the first 2^22 parameters
    S = 1 << 22
    _, xd = synth.dense_clients_bf16(synth.CFG_DENSE_2B, 16, S, 0.02, 1e-3)
    nd = synth.sample_counts(synth.CFG_DENSE_2B, 16, 100, 1000)
    cases["dense_2b"] = (lambda: oracle.weighted_average(xd, nd, x_dtype=oracle.BF16), 16 * S,
                         f"the first {S} parameters of the K=16 bf16 dense workload")

    # sparse: K=20 top-10% lists over a 2^22-parameter slice of the index space
    Ns = 1 << 22
    si = [synth.uniform_sparse_support(synth.CFG_SPARSE_1B, k, Ns, Ns // 10) for k in range(20)]
    sv = [synth.laplace_tail_values(synth.CFG_SPARSE_1B, k, Ns // 10, 0.1, 1e-3) for k in range(20)]
    bs = synth.normal_f32(synth.CFG_SPARSE_1B, synth.ROLE_BASE, 0, Ns, 0.02)
    ns = synth.sample_counts(synth.CFG_SPARSE_1B, 20, 100, 1000)
    cases["sparse"] = (lambda: oracle.sparse_average(si, sv, ns, Ns, mode=oracle.DELTAS, base=bs),
                       sum(x.size for x in si),
                       f"K=20 top-10% lists over {Ns} parameters (the workload's density and "
                       f"value distribution)")

    out = {}
    for name, (fn, units, sample) in cases.items():
        fn()                                            # warm-up
        res = {"sample": sample}
        for label, t in (("all", all_threads), ("one", 1)):
            oracle.set_threads(t)
            v, reps = _time_oracle(fn, units, budget_s)
            res[f"params_per_s_{label}_threads"] = v
            res[f"calls_{label}_threads"] = reps
        oracle.set_threads(all_threads)
        out[name] = res
        log(f"cpu baseline {name}: {res['params_per_s_all_threads']:.3e} params/s on {all_threads} "
            f"threads, {res['params_per_s_one_threads']:.3e} on 1")
    head = out["dense_2b"]
    return {"value": head["params_per_s_all_threads"], "unit": "params/s", "cores": all_threads,
            "kind": "oracle",
            "sample": head["sample"] + f"; plain C oracle (fp64), OpenMP over parameters on "
                                       f"{all_threads} threads",
            "one_thread_value": head["params_per_s_one_threads"], "host": host, "workloads": out}


def traffic_from_counters():
    """HBM bytes per launch of the headline kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary (scaled by a copy of known size), or None
    when it is absent or the kernel source has changed since it was taken."""
    try:
        with open(COUNTERS_FILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(re.findall(r"^(kernel_source_sha256|traffic_bytes_per_launch):\s*(\S+)\s*$", text, re.M))
    if fields.get("kernel_source_sha256") != kernel_source_sha():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default="all",
                    help="comma list of: dense,dense_small,adapter,streaming,windows,sparse,topk,"
                         "hierarchical,sparse_stream,checksum,ceiling,dense_k,streaming_chunks,spill,"
                         "cpu,copycal (default all but copycal)")
    ap.add_argument("--stream-clients", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: every output "
              f"parameter depends only on the same parameter of each client, so more GPUs would each "
              f"run these kernels on one contiguous slice of the parameters", file=sys.stderr)
        sys.exit(2)

    import torch
    import weighted_model_update_amd as fa
    fa.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    only = set(args.only.split(",")) if args.only != "all" else {"dense", "dense_small", "adapter",
                                                                 "streaming", "windows", "sparse", "topk",
                                                                 "hierarchical", "sparse_stream",
                                                                 "checksum", "ceiling", "dense_k",
                                                                 "streaming_chunks", "spill", "cpu"}
    if args.no_cpu_baseline:
        only.discard("cpu")

    modes = {}
    head = None
    if "dense" in only:
        head = bench_dense_2b(args.steps, args.warmup)
        log(f"dense 2B: {head['avg_launch_ms']:.3f} ms/launch "
            f"({head['separate_allocations']['avg_launch_ms']:.3f} in separate allocations)")
    if "dense_small" in only:
        modes["dense_small"] = bench_dense_small()
        log(f"dense_small: {modes['dense_small']['us_per_call']:.2f} us/call, "
            f"{modes['dense_small']['us_per_call_graph']:.2f} from a graph")
    if "adapter" in only:
        modes["adapter"] = bench_adapter()
        log(f"adapter: {modes['adapter']['us_per_call']:.2f} us/call")
    if "sparse" in only:
        modes["sparse"] = bench_sparse()
        log(f"sparse: {modes['sparse']['ms_per_call']:.3f} ms/call")
    if "streaming" in only:
        modes["streaming"] = bench_streaming(args.stream_clients)
        log(f"streaming: {modes['streaming']['wall_s']:.2f} s")
    if "topk" in only:
        modes["topk"] = bench_topk()
        log(f"topk: {modes['topk']['ms_per_call']:.3f} ms/call")
    if "hierarchical" in only:
        modes["hierarchical"] = bench_hierarchical()
        log(f"hierarchical: {modes['hierarchical']['ms_per_merge']:.3f} ms per silo merge")
    if "sparse_stream" in only:
        modes["sparse_stream"] = bench_sparse_stream()
        log(f"sparse_stream: {modes['sparse_stream']['ms_per_client']:.3f} ms per client "
            f"({modes['sparse_stream']['ms_per_client_scatter']:.3f} scattered)")
    if "windows" in only:
        modes["windows"] = bench_windows(args.stream_clients)
        log(f"windows: {modes['windows']['wall_s']:.2f} s in {modes['windows']['windows']} windows "
            f"({modes['windows']['pcie_gbs']:.1f} GB/s over PCIe)")
    if "checksum" in only:
        modes["checksum"] = bench_checksum()
        log(f"checksum: {modes['checksum']['ms_per_call']:.3f} ms/call, with the value sum "
            f"{modes['checksum']['hash_and_sum_ms_per_call']:.3f}, sum alone "
            f"{modes['checksum']['sum_ms_per_call']:.3f}")
    if "ceiling" in only:
        modes["ceiling"] = bench_ceiling()
        c = modes["ceiling"]
        log(f"ceiling: best mixed pattern {c['best_mixed']['name']} at {c['best_mixed']['median_ms']:.3f} ms; "
            f"dense kernel {c['dense_median_ms']:.3f} ms ({c['dense_over_best_mixed']:.3f}x)")
    if "dense_k" in only:
        modes["dense_k"] = bench_dense_k()
    if "streaming_chunks" in only:
        modes["streaming_chunks"] = bench_streaming_chunks()
    if "spill" in only:
        modes["spill"] = bench_spill()
        log(f"spill: save {modes['spill']['save_gbs']:.2f} GB/s, load {modes['spill']['load_gbs']:.2f} GB/s")
    if "copycal" in only:
        modes["copy_calibration"] = bench_copy_calibration()
    cpu = cpu_baseline() if "cpu" in only else None

    rec = {"metric": METRIC, "unit": "params/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic (seeded, generated on the GPU)"}
    if head is not None:
        ms = head["wall_s"] * 1000.0 / args.steps
        achieved = head["algo_bytes"] / (head["avg_launch_ms"] * 1e-3) / 1e9
        rec.update({
            "value": head["K"] * head["N"] / (ms * 1e-3),
            "ms_per_step": ms,
            "config": {"workload": "dense FedAvg, K=16 resident bf16 clients of a 1,921,878,016-parameter "
                                   "transformer tensor list, fp32 accumulation, bf16 output",
                       "K": head["K"], "N": head["N"], "mode": "weights", "io_dtype": "bf16",
                       "buffers": "the 16 clients and the output in one allocation, buffer j at "
                                  "j x (2 MiB-rounded size + 32 KiB) (arena_layout)",
                       "hbm_gbs": achieved},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_counters(),
                         "kernel": "dense_vec_kernel<bf16,bf16,K=16>",
                         "algo_bytes_per_launch": head["algo_bytes"],
                         "avg_launch_ms": head["avg_launch_ms"],
                         "median_launch_ms": head["median_launch_ms"],
                         "min_launch_ms": head["min_launch_ms"],
                         "separate_allocations": head["separate_allocations"]},
        })
    else:
        rec.update({"value": None, "ms_per_step": None, "config": {"workload": "partial run: " + args.only}})
    rec["cpu_baseline"] = cpu
    rec["modes"] = modes
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
