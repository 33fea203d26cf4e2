"""Benchmark of the paged decode-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|opt13b_b64|...]

A step is one decode iteration of the hot path over one batch (the loop the
Korean review of the vLLM paper, mz-moonzoo.tistory.com/116, section 4.3,
describes): write each sequence's new K/V into its cache slot
(reshape_and_cache), then attend with one query per sequence over the paged
cache (decode partition pass + reduce pass). Inputs are seeded synthetic
tensors of the workload's shapes, resident in HBM before timing starts.

The timed steps are eager launches of the step's kernels with nothing else
between the two events that bracket them. --graph replays the step captured
once as a HIP graph instead (one graph per pool replica: the same kernels on
the same buffers); on ROCm 7 that measured slower than eager launches.
By default (--step fused) a decode step with one new token per sequence is
two launches: the partition pass reads each sequence's newest token from its
new K/V rows, and the reduce pass stores those rows into the cache after
every read (paged_attention_decode_append); --step separate launches
reshape_and_cache first, then the plain passes. --prefill-step fused runs the
chunked prefill with its fused-write kernel instead of reshape_and_cache
first.

Prints ONE JSON line. `value` is decode tokens/s for one layer call (one
query token per sequence per step) on opt13b_b64 (64 sequences, OPT-13B
layer shapes); `per_model_step` divides it over OPT-13B's 40 layers.
`roofline` is for the dominant kernel, the decode partition pass, whose
launches are bracketed by HIP events on the stream they run on, in a
separate eager pass. `cpu_baseline` times the CPU oracle (test
infrastructure, never tuned) on the same batch on the host cores. With the
default --workload all, `workloads` holds the same figures for the other
workloads -- large_batch_b256, parallel_sampling (plain and shared-prefix
steps, the 40-layer copy-on-write copy, swaps) and chunked_prefill (with the
MFMA fraction) -- each with its own roofline and a shorter oracle sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak
METRIC = "paged decode attn tokens/s + effective KV GB/s (% HBM peak), OPT-13B shapes"
MODEL_LAYERS = 40  # OPT-13B: one decode step of the model is 40 layer calls


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    choices=["all", "opt13b_b64", "large_batch_b256", "parallel_sampling", "chunked_prefill"],
                    help="all: opt13b_b64 as the headline line, the others under its `workloads` key")
    ap.add_argument("--replicas", type=int, default=2,
                    help="copies of the KV pool used in turn, so no step finds the last one's data in cache")
    ap.add_argument("--split-workers", type=int, default=0,
                    help="worker waves the tile stream is cut among (0: as many as the GPU holds)")
    ap.add_argument("--dtype", default=None, choices=["f16", "bf16", "f32"],
                    help="element type of the decode workloads (default: the workload's own, fp16)")
    ap.add_argument("--num-seqs", type=int, default=None,
                    help="batch size of the opt13b_b64 (uniform lengths) or large_batch_b256 (lognormal "
                         "lengths) decode workload (default: 64 and 256)")
    ap.add_argument("--block-size", type=int, default=16,
                    help="tokens per KV block for the decode workloads (4, 8, 16, 32 or 64)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured as a HIP graph instead of eager launches")
    ap.add_argument("--step", default="fused", choices=["fused", "separate"],
                    help="decode workloads with one new token per sequence: the partition pass reads the new "
                         "token from its rows and the reduce pass stores it (fused, paged_attention_decode_append: "
                         "two launches), or reshape_and_cache first (separate: three launches)")
    ap.add_argument("--prefill-step", default="separate", choices=["fused", "separate"],
                    help="chunked_prefill: the fused-write kernel (the chunk's K/V stored by the prefill kernel) or "
                         "reshape_and_cache first")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle on the batch until this much time has passed (at least 3 runs)")
    ap.add_argument("--cpu-seconds-others", type=float, default=4.0,
                    help="the same for the other workloads of --workload all")
    return ap.parse_args()


# The sources a kernel is built from: the decode partition kernel's walk is
# in pa_stream.h, its launch and plan in pa_decode.hip.
DECODE_SOURCES = ("pa_decode.hip", "pa_stream.h")


def kernel_source_digest(source=DECODE_SOURCES) -> str:
    """sha256 (first 16 hex digits) of a kernel's source files, concatenated."""
    names = (source,) if isinstance(source, str) else source
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_109_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(profile: str, source=DECODE_SOURCES):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary (profiles/<profile>_counters.md), if that summary was taken on
    the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{profile}_counters.md")
    if not os.path.exists(path):
        print(f"[bench] no counter summary {os.path.basename(path)}: traffic = null", file=sys.stderr)
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_digest(source):
        print(f"[bench] {os.path.basename(path)} was taken on other {'/'.join((source,) if isinstance(source, str) else source)} sources "
              f"({m.group(1) if m else '?'} vs {kernel_source_digest(source)}): traffic = null", file=sys.stderr)
        return None
    return float(t.group(1))


def traffic_source(profile: str) -> str:
    return f"profiles/{profile}_counters.md (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated; taken on this kernel source)"


def calibrate_counters(torch, dev):
    """A plain 1 GiB device copy, the reference the HBM byte counters are
    scaled by (its FETCH_SIZE and WRITE_SIZE must read 1 GiB each)."""
    src = torch.empty(1 << 29, dtype=torch.float16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def measure_stream_read(torch, pa, dev, gib: int = 4):
    """Same-device reference for the memory-bound kernels: the library's plain
    streaming-read kernel over a 4 GiB buffer, at a few grid sizes; the best
    median rate counts."""
    import numpy as np
    buf = torch.empty(gib << 28, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * 4
    best = None
    for groups in (1024, 2048, 4096, 8192, 16384):
        sink = torch.empty(pa.STREAM_SINK_WORDS_PER_GROUP * groups, dtype=torch.int32, device=dev)
        pa.stream_read(buf, sink, groups)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, z in ev:
            a.record()
            pa.stream_read(buf, sink, groups)
            z.record()
        torch.cuda.synchronize()
        gbps = nbytes / (float(np.median([a.elapsed_time(z) for a, z in ev])) * 1e-3) / 1e9
        if best is None or gbps > best["gbps"]:
            best = {"gbps": gbps, "workgroups": groups, "bytes": nbytes, "kernel": "stream_read_kernel"}
    del buf
    torch.cuda.empty_cache()
    print(f"[bench] streaming read {best['gbps']:.0f} GB/s ({best['workgroups']} workgroups)", file=sys.stderr,
          flush=True)
    return best


def capture_steps(torch, step, n):
    """One HIP graph per pool replica of the whole step (torch.cuda.graph):
    the same kernels on the same buffers, launched as one graph. Warmed up
    eagerly on a side stream first, as torch asks."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def timed_steps(torch, step, args, n_replicas):
    """Warm-up, then args.steps steps between two events on the launch stream
    (synchronised before and after), with nothing else in the timed region.
    Returns (ms per step, how the step was launched)."""
    graphs = capture_steps(torch, step, n_replicas) if args.graph else None
    run = (lambda i: graphs[i % n_replicas].replay()) if graphs else step
    for i in range(args.warmup):
        run(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        run(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / args.steps, ("hip graph replay" if graphs else "eager launches")



def cpu_model() -> str:
    """The host CPU's model name (for the oracle timing), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()

def time_oracle(fn, seconds: float):
    """Run fn repeatedly for at least `seconds` (and at least 3 times);
    return the per-run times."""
    times, start = [], time.perf_counter()
    while len(times) < 3 or time.perf_counter() - start < seconds:
        t = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t)
    return times


def launch_stats(ms):
    """Median, min and max of per-launch event times (ms) in microseconds."""
    import numpy as np
    return {"median_launch_us": float(np.median(ms)) * 1e3, "min_launch_us": float(min(ms)) * 1e3,
            "max_launch_us": float(max(ms)) * 1e3}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_109_amd as pa

    if args.workload == "all" and (args.num_seqs is not None or args.dtype or args.block_size != 16):
        print("--num-seqs, --dtype and --block-size apply to a single --workload", file=sys.stderr)
        sys.exit(2)
    if args.workload == "chunked_prefill" and args.block_size != 16:
        print("the chunked_prefill workload uses 16-token blocks", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    calibrate_counters(torch, dev)
    stream_read = measure_stream_read(torch, pa, dev)
    if args.workload == "chunked_prefill":
        result = run_prefill(args, stream_read, args.cpu_seconds)
    else:
        first = "opt13b_b64" if args.workload == "all" else args.workload
        result = run_decode(first, args, stream_read, args.cpu_seconds)
    if args.workload == "all":
        others = {}
        for name in ("large_batch_b256", "parallel_sampling", "chunked_prefill"):
            torch.cuda.empty_cache()
            line = (run_prefill(args, stream_read, args.cpu_seconds_others) if name == "chunked_prefill"
                    else run_decode(name, args, stream_read, args.cpu_seconds_others))
            for k in ("n_gpus", "steps", "warmup", "higher_is_better", "scaling", "data", "stream_read"):
                line.pop(k, None)
            others[name] = line
        result["workloads"] = others
    print(json.dumps(result))


def oracle_baseline(fn, seconds: float, units: int, unit: str, what: str, kv_bytes: int = 0):
    """The CPU oracle (test infrastructure, never tuned) repeated on a batch
    for about `seconds` on every host core this process may use."""
    import numpy as np
    import oracle
    oracle.load()
    threads = len(os.sched_getaffinity(0))
    times = time_oracle(lambda: fn(threads), seconds)
    t_med = float(np.median(times))
    cpu = {"value": units / t_med, "unit": unit, "cores": threads, "kind": "oracle",
           "sample": f"{what} {len(times)} times ({sum(times):.1f}s) by the fp64 C oracle with OpenMP; median "
                     f"{t_med:.2f}s per batch; CPU {cpu_model()}"}
    if kv_bytes:
        cpu["effective_kv_gbps"] = kv_bytes / t_med / 1e9
    return cpu


def run_decode(name, args, stream_read, cpu_seconds):
    """One decode workload: the timed step, the partition pass's roofline,
    the other kernels of the step, and the oracle baseline."""
    import numpy as np
    import torch

    import paged_kv_cache_109_amd as pa
    import workloads as W

    t0 = time.time()
    extra = {"dtype": args.dtype} if args.dtype else {}
    if args.num_seqs is not None:
        if name not in ("opt13b_b64", "large_batch_b256") or args.num_seqs < 1:
            print("--num-seqs applies to the opt13b_b64 and large_batch_b256 workloads (>= 1)", file=sys.stderr)
            sys.exit(2)
        extra["num_seqs"] = args.num_seqs
    case = {"opt13b_b64": W.opt13b_b64, "large_batch_b256": W.large_batch_b256,
            "parallel_sampling": W.parallel_sampling}[name](block_size=args.block_size, **extra)
    print(f"[bench] workload {case.name} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]

    def to_dev(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if case.dtype == "bf16" and dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    S, H, D, B = case.num_seqs, case.num_heads, case.head_dim, case.block_size
    q = to_dev(case.q, case.dtype)
    pools = [(to_dev(case.k_cache, case.dtype), to_dev(case.v_cache, case.dtype)) for _ in range(args.replicas)]
    block_tables = to_dev(case.block_tables)
    context_lens = to_dev(case.context_lens)
    writes = case.new_key is not None
    if writes:
        slots = pa.slot_mapping(block_tables, to_dev(case.new_seq.astype(np.int32)),
                                to_dev(case.new_pos.astype(np.int32)), B, case.num_blocks)
        new_k, new_v = to_dev(case.new_key, case.dtype), to_dev(case.new_value, case.dtype)
    copies = case.block_mapping is not None
    if copies:
        mapping = to_dev(case.block_mapping)
    # The fused step needs exactly one new token per sequence, at its last
    # position, and nothing written before it.
    fused = (args.step == "fused" and writes and not copies and len(case.new_seq) == S
             and (case.new_seq == np.arange(S)).all() and (case.new_pos == case.context_lens - 1).all())
    out = torch.empty_like(q)
    max_ctx = case.max_context_len
    workers = args.split_workers
    ws = pa.alloc_decode_workspace(S, H, D, max_ctx, B, workers, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        # ev: four events on the launch stream -- step start, after the cache
        # write / copy, after the partition pass, after the reduce.
        k_cache, v_cache = pools[i % len(pools)]
        if ev is not None:
            ev[0].record(stream)
        if copies:
            pa.copy_blocks([k_cache], [v_cache], mapping)
        if writes and not fused:
            pa.reshape_and_cache(new_k, new_v, k_cache, v_cache, slots)
        if ev is not None:
            ev[1].record(stream)
        if fused:
            pa.paged_attention_decode_append_partitions(out, q, new_k, new_v, k_cache, v_cache, block_tables,
                                                        context_lens, max_ctx, case.scale, workspace=ws,
                                                        split_workers=workers)
        else:
            pa.paged_attention_decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, max_ctx,
                                                 case.scale, workspace=ws, split_workers=workers)
        if ev is not None:
            ev[2].record(stream)
        if fused:
            pa.paged_attention_decode_append_reduce(out, q, new_k, new_v, k_cache, v_cache, block_tables,
                                                    context_lens, max_ctx, case.scale, workspace=ws,
                                                    split_workers=workers)
        else:
            pa.paged_attention_decode_reduce(out, context_lens, max_ctx, case.max_blocks_per_seq, H, D, B,
                                             workspace=ws, split_workers=workers)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, launch = timed_steps(torch, step, args, len(pools))
    # Per-kernel durations from a separate eager pass with events between the
    # kernels (kept out of the timed region above).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    part_ms = [e[1].elapsed_time(e[2]) for e in evs]
    part_avg_s = float(np.mean(part_ms)) * 1e-3
    pre_avg_s = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    red_avg_s = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) * 1e-3
    print(f"[bench] step {ms_per_step * 1e3:.1f} us; partition pass avg {part_avg_s * 1e6:.1f} us "
          f"(min {min(part_ms) * 1e3:.1f}, max {max(part_ms) * 1e3:.1f}); write/copy {pre_avg_s * 1e6:.1f} us; "
          f"reduce {red_avg_s * 1e6:.1f} us", file=sys.stderr, flush=True)

    elt = case.elt_bytes
    kv_bytes = W.logical_kv_bytes(case.context_lens, H, D, elt)
    nblocks = int(sum(W.blocks_needed(n, B) for n in case.context_lens))
    # Algorithmic bytes of one partition-pass launch: every valid token's K and
    # V row once, q in, the output out, the table entries and lengths; fused,
    # also the new token's K and V rows written into the cache.
    alg_bytes = kv_bytes + 2 * S * H * D * elt + 4 * nblocks + 4 * S + (2 * S * H * D * elt if fused else 0)
    achieved = alg_bytes / part_avg_s / 1e9
    tokens_per_s = S / (ms_per_step * 1e-3)
    # Counter summaries are committed for the 16-token-block workloads only.
    traffic = (committed_traffic("decode_partition_" + ("append_" if fused else "") + case.name.rsplit("_", 1)[0])
               if B == 16 and case.dtype == "f16" else None)

    # The other kernels of the step, each timed by its own events: algorithmic
    # bytes are what the call must read plus what it must write.
    components = {"decode_reduce_kernel": {"avg_us": red_avg_s * 1e6}}
    row = H * D * elt
    if writes and not fused:
        T = int(case.new_key.shape[0])
        b = 2 * (2 * T * row) + 8 * T
        components["reshape_and_cache_kernel"] = {"tokens": T, "alg_bytes": b, "avg_us": pre_avg_s * 1e6,
                                                  "gbps": b / pre_avg_s / 1e9}
    if copies:
        P = int(case.block_mapping.shape[0])
        blk = row * B
        b1 = 2 * (2 * P * blk) + 16 * P
        components["copy_blocks_kernel"] = {"pairs": P, "layers": 1, "alg_bytes": b1, "avg_us": pre_avg_s * 1e6,
                                            "gbps": b1 / pre_avg_s / 1e9}
        # The same copy-on-write over every layer of the model in one launch.
        L = 40
        layers = [pools[0]] + [(pools[0][0].clone(), pools[0][1].clone()) for _ in range(L - 1)]
        ks, vs = [k for k, _ in layers], [v for _, v in layers]
        pa.copy_blocks(ks, vs, mapping)
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, z in ce:
            a.record(stream)
            pa.copy_blocks(ks, vs, mapping)
            z.record(stream)
        torch.cuda.synchronize()
        t_l = float(np.mean([a.elapsed_time(z) for a, z in ce])) * 1e-3
        components["copy_blocks_kernel_40_layers"] = {"pairs": P, "layers": L, "alg_bytes": L * b1,
                                                      "avg_us": t_l * 1e6, "gbps": L * b1 / t_l / 1e9}
        print(f"[bench] copy_blocks {P} pairs x {L} layers: {t_l * 1e6:.1f} us, {L * b1 / t_l / 1e9:.0f} GB/s",
              file=sys.stderr, flush=True)
        del layers, ks, vs
        # Swapping the same blocks of one layer's K and V out to pinned host
        # memory and back in (one launch each way), over the host link.
        host_pool = [torch.empty((P,) + tuple(pools[0][0].shape[1:]), dtype=pools[0][0].dtype, pin_memory=True)
                     for _ in range(2)]
        out_map = torch.stack([mapping[:, 0], torch.arange(P, device=dev)], dim=1).contiguous()
        in_map = torch.stack([torch.arange(P, device=dev), mapping[:, 1]], dim=1).contiguous()
        srcs = [pools[0][0], pools[0][1]]
        pa.swap_blocks(srcs, host_pool, out_map)
        torch.cuda.synchronize()
        sw = {}
        for name, a_list, b_list, m in (("out", srcs, host_pool, out_map), ("in", host_pool, srcs, in_map)):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
            for a, z in ev:
                a.record(stream)
                pa.swap_blocks(a_list, b_list, m)
                z.record(stream)
            torch.cuda.synchronize()
            sw[name] = float(np.median([a.elapsed_time(z) for a, z in ev])) * 1e-3
        swap_bytes = 2 * P * blk
        components["swap_blocks_kernel"] = {
            "pairs": P, "caches": 2, "bytes_each_way": swap_bytes,
            "to_host_us": sw["out"] * 1e6, "to_host_gbps": swap_bytes / sw["out"] / 1e9,
            "from_host_us": sw["in"] * 1e6, "from_host_gbps": swap_bytes / sw["in"] / 1e9}
        print(f"[bench] swap_blocks {P} blocks x 2 caches: to host {swap_bytes / sw['out'] / 1e9:.1f} GB/s, "
              f"from host {swap_bytes / sw['in'] / 1e9:.1f} GB/s", file=sys.stderr, flush=True)
        del host_pool
    if copies and B < 16:
        components["decode_shared"] = {"skipped": "the shared-prefix decode is built for block sizes 16, 32, 64"}
    if copies and B >= 16:
        # The same step with the sharing-aware decode: each group's shared
        # prompt blocks are read once for all of its samples.
        first = case.block_tables[:, 0]
        groups = [np.flatnonzero(first == b).tolist() for b in np.unique(first)]
        gm, gp, st, maxp = pa.shared_prefix_groups(case.block_tables, case.context_lens, groups, B)
        gm_d, gp_d, st_d = to_dev(gm), to_dev(gp), to_dev(st)
        wss = pa.alloc_decode_shared_workspace(S, H, D, max_ctx, B, gm.shape[0], maxp, workers, device=dev)

        def shared_step(i, ev=None):
            k_cache, v_cache = pools[i % len(pools)]
            pa.copy_blocks([k_cache], [v_cache], mapping)
            if ev is not None:
                ev[0].record(stream)
            pa.paged_attention_decode_shared(out, q, k_cache, v_cache, block_tables, context_lens, max_ctx,
                                             case.scale, gm_d, gp_d, st_d, maxp, workspace=wss,
                                             split_workers=workers)
            if ev is not None:
                ev[1].record(stream)

        for i in range(args.warmup):
            shared_step(i)
        sh_ms, _ = timed_steps(torch, shared_step, args, len(pools))
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            shared_step(i, sev[i])
        torch.cuda.synchronize()
        dec_ms = [a.elapsed_time(z) for a, z in sev]
        dec_s = float(np.mean(dec_ms)) * 1e-3
        distinct = len({b for blocks in case.seq_blocks for b in blocks}) * 2 * row * B
        components["decode_shared"] = {
            "groups": int(gm.shape[0]), "shared_prefix_tokens": int(maxp), "step_us": sh_ms * 1e3,
            "tokens_per_s": S / (sh_ms * 1e-3), "decode_call_avg_us": dec_s * 1e6, **launch_stats(dec_ms),
            "logical_kv_gbps": kv_bytes / dec_s / 1e9, "distinct_kv_gbps": distinct / dec_s / 1e9}
        print(f"[bench] shared-prefix decode: step {sh_ms * 1e3:.1f} us ({S / (sh_ms * 1e-3):.0f} tokens/s); "
              f"decode call {dec_s * 1e6:.1f} us, {distinct / dec_s / 1e9:.0f} GB/s of distinct blocks",
              file=sys.stderr, flush=True)

        # The same plain step told that the sequences share blocks
        # (pa_paged_attention_decode_ex, PA_DECODE_REUSED_BLOCKS): ordinary
        # K/V loads, so the caches can serve the samples' repeated reads.
        def reused_step(i, ev=None):
            k_cache, v_cache = pools[i % len(pools)]
            pa.copy_blocks([k_cache], [v_cache], mapping)
            if ev is not None:
                ev[0].record(stream)
            pa.paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_ctx, case.scale,
                                      workspace=ws, split_workers=workers, reused_blocks=True)
            if ev is not None:
                ev[1].record(stream)

        for i in range(args.warmup):
            reused_step(i)
        ru_ms, _ = timed_steps(torch, reused_step, args, len(pools))
        rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            reused_step(i, rev[i])
        torch.cuda.synchronize()
        ru_calls = [a.elapsed_time(z) for a, z in rev]
        ru_s = float(np.mean(ru_calls)) * 1e-3
        components["decode_reused_blocks"] = {
            "step_us": ru_ms * 1e3, "tokens_per_s": S / (ru_ms * 1e-3), "decode_call_avg_us": ru_s * 1e6,
            **launch_stats(ru_calls), "logical_kv_gbps": kv_bytes / ru_s / 1e9}
        print(f"[bench] plain decode with reused blocks: step {ru_ms * 1e3:.1f} us ({S / (ru_ms * 1e-3):.0f} "
              f"tokens/s); decode call {ru_s * 1e6:.1f} us, {kv_bytes / ru_s / 1e9:.0f} GB/s of logical K/V",
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cpu = oracle_baseline(
            lambda th: oracle.decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                     case.scale, case.dtype, threads=th),
            cpu_seconds, S, "tokens/s",
            f"the whole {case.name} batch ({S} seqs, {int(case.context_lens.sum())} context tokens, {H} heads) "
            f"decoded", kv_bytes)

    traffic_profile = ("decode_partition_" + ("append_" if fused else "") + case.name.rsplit("_", 1)[0])
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": case.name, "num_seqs": S, "num_heads": H, "head_dim": D, "block_size": B,
                   "context_tokens": int(case.context_lens.sum()), "max_context_len": max_ctx,
                   "split_workers": workers or pa.decode_default_workers(tdt, D, B), "pool_replicas": args.replicas,
                   "step_launch": launch,
                   "step": ("copy_blocks(CoW pairs) + " if copies else "")
                   + ("decode partitions (new tokens read from their rows) + decode reduce (stores them into the cache)"
                      if fused else
                      ("reshape_and_cache(new tokens) + " if writes else "") + "decode partitions + decode reduce")},
        "per_model_step": {"layers": MODEL_LAYERS, "tokens_per_s": tokens_per_s / MODEL_LAYERS,
                           "ms_per_model_step": ms_per_step * MODEL_LAYERS,
                           "note": "one layer call per step timed; a model step is 40 of them (OPT-13B)"},
        "effective_kv_gbps": kv_bytes / (ms_per_step * 1e-3) / 1e9,
        "pct_hbm_peak": kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "stream_read": stream_read,
        "pct_of_stream_read": kv_bytes / (ms_per_step * 1e-3) / 1e9 / stream_read["gbps"],
        "roofline": {"bound": "hbm", "kernel": "decode_partition_kernel" + (" (append)" if fused else ""),
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "traffic_source": traffic_source(traffic_profile) if traffic else None,
                     "alg_bytes_per_launch": alg_bytes, "avg_launch_us": part_avg_s * 1e6,
                     **launch_stats(part_ms), "frac_of_stream_read": achieved / stream_read["gbps"]},
        "components": components,
        "cpu_baseline": cpu,
    }
    if copies:
        shared = sorted({b for blocks in case.seq_blocks for b in blocks})
        result["config"]["distinct_blocks_read"] = len(shared)
        result["config"]["distinct_block_bytes"] = len(shared) * 2 * row * B
    return result


def run_prefill(args, stream_read, cpu_seconds):
    """Chunked prefill (16 x 256-query causal chunks, bf16): a step writes the
    chunk's K/V (reshape_and_cache, 4096 tokens) and runs the MFMA kernel."""
    import numpy as np
    import torch

    import paged_kv_cache_109_amd as pa
    import workloads as W

    case = W.chunked_prefill()
    dev = torch.device("cuda:0")

    def to_dev(a, bf=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.int16).view(torch.bfloat16) if bf else t).to(dev)

    S, H, D, B = case.num_seqs, case.num_heads, case.head_dim, case.block_size
    q = to_dev(case.q, True)
    # The pool (~0.5 GB) is only about twice the last-level cache: rotate at
    # least four copies so each launch reads its K/V from HBM.
    pools = [(to_dev(case.k_cache, True), to_dev(case.v_cache, True)) for _ in range(max(4, args.replicas))]
    bt, ctx, cu = to_dev(case.block_tables), to_dev(case.context_lens), to_dev(case.cu_q_lens)
    slots = pa.slot_mapping(bt, to_dev(case.new_seq.astype(np.int32)), to_dev(case.new_pos.astype(np.int32)), B,
                            case.num_blocks)
    nk, nv = to_dev(case.new_key, True), to_dev(case.new_value, True)
    out = torch.empty_like(q)
    q_lens = np.diff(case.cu_q_lens)
    max_q, max_ctx = int(q_lens.max()), case.max_context_len
    stream = torch.cuda.current_stream()

    fused = args.prefill_step == "fused"

    def step(i, ev=None):
        k_cache, v_cache = pools[i % len(pools)]
        if not fused:
            pa.reshape_and_cache(nk, nv, k_cache, v_cache, slots)
        if ev is not None:
            ev[0].record(stream)
        if fused:
            pa.paged_attention_prefill_chunk_append(out, q, nk, nv, cu, k_cache, v_cache, bt, ctx, max_q, max_ctx,
                                                    case.scale)
        else:
            pa.paged_attention_prefill_chunk(out, q, cu, k_cache, v_cache, bt, ctx, max_q, max_ctx, case.scale)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, launch = timed_steps(torch, step, args, len(pools))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_s = float(np.mean(kern_ms)) * 1e-3
    # Causal work: query j of a sequence with c cached tokens sees c + j + 1
    # keys; each key costs 2*D flops for q.k and 2*D for p*v.
    c = case.context_lens - q_lens
    keys = sum(int(q_lens[s]) * int(c[s]) + int(q_lens[s]) * (int(q_lens[s]) + 1) // 2 for s in range(S))
    flops = 4.0 * D * H * keys
    elt = 2
    kv_bytes = W.logical_kv_bytes(case.context_lens, H, D, elt)
    qo_bytes = 2 * int(q_lens.sum()) * H * D * elt
    # Fused, the launch also writes the chunk's K and V rows into the cache.
    write_bytes = 2 * int(q_lens.sum()) * H * D * elt if fused else 0
    tflops = flops / kern_s / 1e12
    gbps = (kv_bytes + qo_bytes + write_bytes) / kern_s / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cpu = oracle_baseline(
            lambda th: oracle.prefill_chunk(case.q, case.cu_q_lens, case.k_cache, case.v_cache, case.block_tables,
                                            case.context_lens, case.scale, case.dtype, threads=th),
            cpu_seconds, int(q_lens.sum()), "query tokens/s",
            f"the whole chunked_prefill batch ({S} x {max_q} queries, {H} heads)")
    profile = "prefill_chunk_" + ("append_" if fused else "") + "chunked_prefill"
    traffic = committed_traffic(profile, "pa_prefill.hip")
    result = {
        "metric": "chunked prefill paged attention query tokens/s (MFMA), OPT-13B shapes",
        "value": int(q_lens.sum()) / (ms_per_step * 1e-3), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": case.name, "num_seqs": S, "q_len": max_q, "num_heads": H, "head_dim": D,
                   "block_size": B, "context_tokens": int(case.context_lens.sum()),
                   "step": ("prefill chunk kernel with the 4096 chunk tokens' cache write fused in" if fused
                            else "reshape_and_cache(4096 chunk tokens) + prefill chunk kernel"),
                   "pool_replicas": len(pools), "step_launch": launch},
        "stream_read": stream_read,
        "roofline": {"bound": "hbm", "kernel": "prefill_chunk_kernel" + (" (append)" if fused else ""),
                     "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "traffic_source": traffic_source(profile) if traffic else None,
                     "alg_bytes_per_launch": kv_bytes + qo_bytes + write_bytes, "avg_launch_us": kern_s * 1e6,
                     **launch_stats(kern_ms), "frac_of_stream_read": gbps / stream_read["gbps"],
                     "mfma_tflops": tflops, "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                     "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS, "causal_flops_per_launch": flops},
        "cpu_baseline": cpu,
    }
    result["per_model_step"] = {"layers": MODEL_LAYERS, "query_tokens_per_s": result["value"] / MODEL_LAYERS,
                                "ms_per_model_step": ms_per_step * MODEL_LAYERS}
    print(f"[bench] prefill step {ms_per_step * 1e3:.1f} us; kernel {kern_s * 1e6:.1f} us; {tflops:.0f} TFLOP/s; "
          f"{gbps:.0f} GB/s", file=sys.stderr, flush=True)
    return result


if __name__ == "__main__":
    main()
