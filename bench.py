#!/usr/bin/env python3
"""Benchmark: paged decode attention on one GPU.

One step = the step's copy-on-write copies (if any) + the append of every
sequence's new K/V + the decode attention, for one layer of one workload,
inputs resident in HBM; append and decode run as one launch (pa_decode_step).  Default workload: the OPT-13B layer (40 heads x 128,
fp16, block 16, 30 sequences, contexts uniform in 128..2048).

Timing (after the method of the "KV 缓存" topic page, level-3 script: inputs
built outside the timed region, warm-up first, median with [min, max]):
W untimed warm-up steps, then exactly K timed steps between device
synchronisations, also split into 10 samples for median [min, max]; these
give the throughput.  Steps rotate over several copies of the pool so
consecutive steps do not find the previous step's K/V in the last-level
cache.  Per-kernel durations (the roofline) come from a second pass of the
same K steps, in which the library records HIP events around its kernels on
their own stream; the events are kept out of the throughput pass because
each is a marker packet between launches that adds its own time to a step.

Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
METRIC = "paged decode attention tokens/s and achieved HBM GB/s (% of peak), 1 GPU"


def workload_label(wl):
    return (f"{wl.name}: {wl.num_q_heads} q heads / {wl.num_kv_heads} kv heads x {wl.head_dim}, kv {wl.kv}, "
            f"act {wl.act}, block {wl.block_size}, {wl.batch} seqs, ctx U[{wl.ctx_lo},{wl.ctx_hi}]"
            + (f" after a shared {wl.prefix_len}-token prefix" if wl.prefix_len else ""))


def decode_kernel_name(wl, shared=False):
    """The decode kernel that serves the workload (matrix cores when query
    heads share KV heads and activations are f16, else the per-head kernel
    and its merge launch), with the prefix pass when a shared prefix takes
    the shared-prefix path: in the same launch as a per-head decode over an
    FP8 pool with blocks of at least 16 tokens (and a wave load's tokens),
    else a launch of its own before the decode."""
    grouped = wl.num_q_heads > wl.num_kv_heads and wl.act == "f16"
    if grouped:
        k = "decode_group_kernel (grouped heads on MFMA: append + split-context attention + merge)"
    else:
        k = "decode_kernel (per head on VALU: append + split-context attention) + merge_kernel (split-context merge)"
    if not shared:
        return k
    pass_ = "the shared blocks once per KV head for every sequence, MFMA"
    per_load = 64 // (wl.head_dim // 16)  # tokens of one wave load of the FP8 per-head kernel
    if (not grouped and wl.act == "f16" and wl.kv == "e4m3" and wl.head_dim in (32, 64, 128)
            and wl.block_size >= max(16, per_load)):
        return ("decode_prefix_fused_kernel (per head on VALU: append + split-context attention; then, in the "
                f"launch's last workgroups, the prefix pass: {pass_}) + merge_kernel (split-context merge)")
    return f"prefix pass (decode_group_kernel: {pass_}) + " + k


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_375_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, launch_bytes):
    """HBM bytes per launch of the decode kernel from the committed counter
    summary, or None when it is missing or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(dr, warmup=2, samples=10):
    """The CPU reference (plain scalar C, fp64) on the same step, by the
    timing method of the "KV 缓存" topic page's level-3 script: inputs built
    outside the timed region, `warmup` untimed runs, then `samples` timed
    runs reported as median [min, max].  The reported value spreads the
    decode's (sequence, head) pairs over the host's threads; the
    single-thread figure times a bounded sample of those pairs (every pair
    costs in proportion to its context) and scales it to the whole step."""
    import numpy as np

    from oracle.allocator import OracleAllocator
    from oracle.reference_step import ReferenceStep, host_threads
    from paged_kv_cache_375_amd.workloads import run_scenario

    ref = ReferenceStep(dr, run_scenario(dr, OracleAllocator(dr.num_blocks, dr.wl.block_size, dr.free_order)))
    T = host_threads()

    def timed(fn):
        for _ in range(warmup):
            fn()
        ts = []
        for _ in range(samples):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        return statistics.median(ts), min(ts), max(ts)

    med, lo, hi = timed(lambda: (ref.append(), ref.decode_threaded(T)))

    # single thread: a seeded sample of (sequence, head) pairs holding about
    # 2.6e7 context elements (~0.5 s here), scaled by the whole step's count
    B, hq, d = dr.q.shape
    ctx = np.asarray(ref.sc.ctx, dtype=np.int64)
    order = np.random.default_rng(0).permutation(B * hq)
    cum = np.cumsum(ctx[order // hq] * d)
    n = int(min(len(order), np.searchsorted(cum, 2.6e7) + 1))
    seqs, heads = (order[:n] // hq).tolist(), (order[:n] % hq).tolist()
    frac = float(cum[n - 1]) / float(cum[-1])
    smed, slo, shi = timed(lambda: ref.decode_pairs(seqs, heads))
    step = f"the whole step (append + decode of all {B} sequences, every head)"
    how = f"warm-up {warmup}, {samples} timed runs, median [min, max]"
    return {"value": B / med, "unit": "tokens/s", "cores": T, "kind": "oracle",
            "sample": f"{step}, decode pairs spread over {T} threads; {how}: {med:.3f} s [{lo:.3f}, {hi:.3f}]",
            "single_thread": {"value": B * frac / smed, "unit": "tokens/s", "cores": 1,
                              "sample": f"decode of {n} of {B * hq} (sequence, head) pairs ({frac:.1%} of the "
                                        f"step's context elements) on one thread, scaled to the whole step; "
                                        f"{how}: {smed:.3f} s [{slo:.3f}, {shi:.3f}]"},
            "cpu": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def _time_ms(fn, reps):
    """Mean milliseconds of fn() over reps calls, between HIP events on the current stream."""
    import torch

    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def bench_writers(wl, dr, step, args):
    """Throughput of the pool writers over algorithmic bytes (each element read
    from the source once and written to the pool once)."""
    import numpy as np
    import torch

    from paged_kv_cache_375_amd import api
    from paged_kv_cache_375_amd.accounting import ELEM_BYTES

    ea, ek = ELEM_BYTES[wl.act], ELEM_BYTES[wl.kv]
    hkv, d, B = wl.num_kv_heads, wl.head_dim, wl.batch
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k_hist, v_hist = dev(dr.k_hist), dev(dr.v_hist)
    rows = int(dr.hist_count.sum())
    tables, hist_row = dev(step.scenario.hist_tables), dev(dr.hist_row)
    start, count = dev(dr.hist_start), dev(dr.hist_count)
    mc = int(dr.hist_count.max())
    lines = []

    ms = _time_ms(lambda: api.kv_write_prompt(step.cache, k_hist, v_hist, hist_row, start, count, tables, mc), 10)
    nbytes = rows * hkv * d * (ea + ek) * 2 + 16 * B
    lines.append(("pa_kv_write_prompt", ms, nbytes, f"{rows} history tokens of {B} sequences"))

    ms = _time_ms(lambda: api.kv_append(step.cache, step.k_new, step.v_new, step.tables, step.ctx), 200)
    nbytes = B * hkv * d * (ea + ek) * 2 + 8 * B
    lines.append(("pa_kv_append", ms, nbytes, f"one token of each of {B} sequences"))

    n = min(1024, dr.num_blocks // 2)
    rng = np.random.default_rng(args.seed)
    perm = rng.permutation(dr.num_blocks).astype(np.int32)
    pairs = dev(np.stack([perm[:n], perm[n:2 * n]], axis=1))
    ms = _time_ms(lambda: api.copy_blocks(step.cache, pairs), 20)
    nbytes = n * 2 * hkv * wl.block_size * d * ek * 2 + 8 * n
    lines.append(("pa_copy_blocks", ms, nbytes, f"{n} random block pairs"))

    for name, ms, nbytes, what in lines:
        gbps = nbytes / (ms / 1e3) / 1e9
        print(json.dumps({"metric": f"{name} HBM GB/s (algorithmic bytes), 1 GPU", "value": gbps, "unit": "GB/s",
                          "n_gpus": 1, "ms_per_call": ms, "algorithmic_bytes": nbytes, "frac_of_peak":
                          gbps / HBM_PEAK_GBPS, "config": {"workload": workload_label(wl), "call": what},
                          "higher_is_better": True, "data": "synthetic"}))


def bench_swap(wl, args):
    """Preemption by swapping: host-link GB/s of pa_swap_blocks moving random
    blocks out to pinned host memory and back, for each block size, beside a
    plain DMA copy of the same bytes between one device buffer and one pinned
    host buffer (the link's ceiling for this amount)."""
    import numpy as np
    import torch

    from paged_kv_cache_375_amd import api
    from paged_kv_cache_375_amd.accounting import ELEM_BYTES

    ek = ELEM_BYTES[wl.kv]
    total = 256 << 20  # K + V bytes moved per call
    for bs in (1, 2, 4, 8, 16, 32, 64):
        block = wl.num_kv_heads * bs * wl.head_dim * ek
        n = total // (2 * block)
        nb = 2 * n
        cache = api.KVCache(nb, bs, wl.num_kv_heads, wl.head_dim, wl.kv, "cuda")
        cache.k.view(torch.uint8).random_(0, 256)
        cache.v.view(torch.uint8).random_(0, 256)
        ids = torch.from_numpy(np.random.default_rng(args.seed).permutation(nb)[:n].astype(np.int32)).cuda()
        hk = torch.empty((n, wl.num_kv_heads, bs, wl.head_dim), dtype=cache.k.dtype).pin_memory()
        hv = torch.empty_like(hk).pin_memory()
        nbytes = 2 * n * block
        for direction in ("out", "in"):
            ms = _time_ms(lambda: api.swap_blocks(cache, hk, hv, ids, direction), 5)
            print(json.dumps({"metric": f"pa_swap_blocks host-link GB/s (swap-{direction}), 1 GPU",
                              "value": nbytes / (ms / 1e3) / 1e9, "unit": "GB/s", "n_gpus": 1, "ms_per_call": ms,
                              "bytes": nbytes, "config": {"workload": workload_label(wl), "block_size": bs,
                                                          "blocks": int(n), "block_bytes_k_plus_v": 2 * block},
                              "higher_is_better": True, "data": "synthetic"}), flush=True)
        del cache, hk, hv
    dev = torch.empty(total, dtype=torch.uint8, device="cuda")
    host = torch.empty(total, dtype=torch.uint8).pin_memory()
    for direction, fn in (("out", lambda: host.copy_(dev, non_blocking=True)),
                          ("in", lambda: dev.copy_(host, non_blocking=True))):
        ms = _time_ms(fn, 5)
        print(json.dumps({"metric": f"contiguous DMA copy host-link GB/s ({direction}), 1 GPU",
                          "value": total / (ms / 1e3) / 1e9, "unit": "GB/s", "n_gpus": 1, "ms_per_call": ms,
                          "bytes": total, "higher_is_better": True, "data": "synthetic"}), flush=True)


def bench_read_ceiling(wl, dr, step, args):
    """The read rate this GPU reaches with no arithmetic: pa_read_probe over
    the workload's own pools and tables, in the decode's load pattern
    ("paged": every sequence's K and V rows through its table) and start to
    end ("linear"), rotating over the same pool copies as the decode, beside
    the decode step timed the same way.  One JSON line per measurement."""
    import torch

    from paged_kv_cache_375_amd import api
    from paged_kv_cache_375_amd.accounting import ELEM_BYTES

    sc = step.scenario
    ek = ELEM_BYTES[wl.kv]
    row = wl.num_kv_heads * wl.head_dim * ek
    paged_bytes = int(sc.ctx.sum()) * 2 * row
    pool_bytes = 2 * step.cache.k.numel() * step.cache.k.element_size()
    rotate = args.rotate or max(1, min(8, math.ceil(2e9 / paged_bytes)))
    caches = [step.cache] + [step.cache.with_pools(step.cache.k.clone(), step.cache.v.clone())
                             for _ in range(rotate - 1)]
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    K = args.steps
    i = [0]

    def rot():
        i[0] += 1
        return caches[i[0] % rotate]

    runs = [("read probe, paged (the decode's load pattern)", paged_bytes,
             lambda: api.read_probe(rot(), step.tables, step.ctx, step.max_ctx, "paged", sink)),
            ("read probe, linear (both pools start to end)", pool_bytes,
             lambda: api.read_probe(rot(), step.tables, step.ctx, step.max_ctx, "linear", sink)),
            ("decode step (pa_decode_step: append + attention + merge)", paged_bytes,
             lambda: step.run(rot()))]
    for what, nbytes, fn in runs:
        for _ in range(max(2, args.warmup)):
            fn()
        ms = _time_ms(fn, K)
        gbps = nbytes / (ms / 1e3) / 1e9
        print(json.dumps({"metric": "HBM read GB/s, 1 GPU", "what": what, "value": gbps, "unit": "GB/s",
                          "frac_of_peak": gbps / HBM_PEAK_GBPS, "ms_per_call": ms, "bytes_read": nbytes,
                          "calls": K, "pool_copies_rotated": rotate,
                          "config": {"workload": workload_label(wl), "sum_ctx": int(sc.ctx.sum())}}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="opt13b")
    ap.add_argument("--block-size", type=int, default=0, help="override the workload's block size")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=0, help="pool copies to rotate over (0: enough for >= 2 GB)")
    ap.add_argument("--cpu-samples", type=int, default=10,
                    help="timed CPU reference runs after two warm-up runs (0 skips the CPU baseline)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM counters) and exit")
    ap.add_argument("--writers", action="store_true",
                    help="instead of the decode step, time the pool writers (prompt write, append, block copy) "
                         "and print one JSON line per writer")
    ap.add_argument("--no-shared", action="store_true",
                    help="decode a prefix workload with pa_decode_step like any other, not the shared-prefix path")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="instead of the decode step, time pa_read_probe (the pools read with the decode's load "
                         "pattern and start to end, no arithmetic) beside the decode step")
    ap.add_argument("--swap", action="store_true",
                    help="instead of the decode step, time block swaps to pinned host memory and back for each "
                         "block size (the workload's heads, head_dim and pool dtype)")
    args = ap.parse_args()

    if args.steps < 1 or args.warmup < 0:
        print(f"bench.py needs --steps >= 1 and --warmup >= 0; got {args.steps}, {args.warmup}", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    from paged_kv_cache_375_amd import api
    from paged_kv_cache_375_amd.accounting import step_bytes, step_flops
    from paged_kv_cache_375_amd.state import DecodeStep
    from paged_kv_cache_375_amd.workloads import WORKLOADS, draw

    wl = WORKLOADS[args.workload]
    if args.block_size:
        wl = wl.with_block_size(args.block_size)
    if args.swap:
        bench_swap(wl, args)
        return
    print(f"bench: building {wl.name}", file=sys.stderr, flush=True)
    dr = draw(wl, args.seed)
    step = DecodeStep(dr, "cuda")
    if args.writers:
        bench_writers(wl, dr, step, args)
        return
    if args.read_ceiling:
        bench_read_ceiling(wl, dr, step, args)
        return
    sc = step.scenario
    sb = step_bytes(sc.ctx, sc.tables, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.act, wl.kv,
                    len(sc.step_pairs))
    pool_bytes = 2 * step.cache.k.numel() * step.cache.k.element_size()
    rotate = args.rotate or max(1, min(8, math.ceil(2e9 / max(1, sb.kv_read_unique))))
    caches = [step.cache] + [step.cache.with_pools(step.cache.k.clone(), step.cache.v.clone())
                             for _ in range(rotate - 1)]
    torch.cuda.synchronize()

    shared = bool(step.shared_blocks) and not args.no_shared
    for i in range(args.warmup):
        step.run(caches[i % rotate], shared=shared)
    torch.cuda.synchronize()

    K = args.steps
    n_samples = 10 if K >= 10 else 1
    per = K // n_samples
    stream = torch.cuda.current_stream()

    # Throughput: exactly K steps with no per-kernel events (each event is a
    # marker packet between launches and would add its own time to a step).
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_samples + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record(stream)
    i = 0
    for smp in range(n_samples):
        n = per if smp < n_samples - 1 else K - per * (n_samples - 1)
        for _ in range(n):
            step.run(caches[i % rotate], shared=shared)
            i += 1
        evs[smp + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = evs[0].elapsed_time(evs[-1])
    sample_ms = []
    for smp in range(n_samples):
        n = per if smp < n_samples - 1 else K - per * (n_samples - 1)
        sample_ms.append(evs[smp].elapsed_time(evs[smp + 1]) / n)

    # Kernel durations: the same K steps again, with the HIP events the
    # library records around its launches on their own stream.
    api.timing_enable(True)
    api.timing_read()
    torch.cuda.synchronize()
    t_k = time.perf_counter()
    for j in range(K):
        step.run(caches[(i + j) % rotate], shared=shared)
    torch.cuda.synchronize()
    wall_kernel_pass = time.perf_counter() - t_k
    part_ms, n_part = api.timing_read()
    api.timing_enable(False)

    ms_per_step = total_ms / K
    tokens_per_s = wl.batch / (ms_per_step / 1e3)
    gbps = sb.total / (ms_per_step / 1e3) / 1e9
    gbps_unique = sb.total_unique / (ms_per_step / 1e3) / 1e9
    part_avg_ms = part_ms / max(1, n_part)
    # the decode kernel appends the new K/V (read from the caller, written into
    # the pool), reads every cached K/V vector once, q and the tables, and
    # writes the output; copy-on-write copies are a separate launch
    part_bytes = sb.total_unique - sb.cow
    achieved = part_bytes / (part_avg_ms / 1e3) / 1e9
    traffic = measured_traffic(wl.name, part_bytes)

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.kv if wl.kv != "e4m3" else "e4m3",
        "accumulate": "f32",
        "data": "synthetic (seeded normal K/V/q, uniform context lengths, shuffled block placement)",
        "config": {
            "workload": workload_label(wl),
            "batch": wl.batch, "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim, "block_size": wl.block_size, "sum_ctx": int(sc.ctx.sum()),
            "max_ctx": int(sc.ctx.max()), "cow_pairs": int(len(sc.step_pairs)), "seed": args.seed,
            "layers": 1, "pool_bytes": pool_bytes, "pool_copies_rotated": rotate,
            "path": "pa_decode_shared_prefix" if shared else "pa_decode_step",
            "shared_prefix_blocks": step.shared_blocks if shared else 0,
        },
        "step_bytes": {"total": sb.total, "kv_read": sb.kv_read, "kv_read_unique": sb.kv_read_unique,
                       "append": sb.append, "q_out": sb.q_out, "tables": sb.tables, "cow": sb.cow},
        "step_flops": step_flops(sc.ctx, wl.num_q_heads, wl.head_dim),
        "gbps_step": gbps,
        "gbps_step_unique": gbps_unique,
        "hbm_frac_step": gbps_unique / HBM_PEAK_GBPS,
        "samples_ms_per_step": {"median": statistics.median(sample_ms), "min": min(sample_ms),
                                "max": max(sample_ms), "n": n_samples},
        "kernels_ms": {"decode_avg": part_avg_ms, "decode_launches": n_part,
                       "pass": "a second pass of the same K steps with the library's HIP events",
                       "wall_s": wall_kernel_pass},
        "wall_s_timed_region": wall,
        "roofline": {"bound": "hbm", "kernel": decode_kernel_name(wl, shared),
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": part_bytes},
    }
    if args.cpu_samples > 0:
        print("bench: timing the CPU reference", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(dr, samples=args.cpu_samples)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
