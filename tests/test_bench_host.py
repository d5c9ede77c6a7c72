"""Host-side parts of the benchmark (no GPU): the threaded CPU reference
(used by the full-size parity tests and the CPU baseline) computes exactly
what the reference's single call does, the CPU baseline runs, and the
one-GPU contract is enforced."""
import subprocess
import sys

import numpy as np

import bench
from oracle.allocator import OracleAllocator
from oracle.reference_step import ReferenceStep
from paged_kv_cache_375_amd.workloads import WORKLOADS, draw, run_scenario


def _ref(wl):
    dr = draw(wl, 0)
    return ReferenceStep(dr, run_scenario(dr, OracleAllocator(dr.num_blocks, wl.block_size, dr.free_order)))


def test_threaded_oracle_decode_equals_single_call():
    for wl in (WORKLOADS["opt13b"].scaled(batch=5, ctx_lo=1, ctx_hi=300),
               WORKLOADS["llama70b_gqa"].scaled(batch=3, ctx_lo=20, ctx_hi=200),
               WORKLOADS["toy"]):
        ref = _ref(wl)
        ref.append()
        want = ref.decode()
        for threads in (1, 3, 8):
            assert np.array_equal(ref.decode_threaded(threads), want)


def test_cpu_baseline_record():
    dr = draw(WORKLOADS["opt13b"].scaled(batch=3, ctx_lo=10, ctx_hi=200), 0)
    rec = bench.cpu_baseline(dr, warmup=1, samples=2)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s" and rec["value"] > 0
    assert rec["cores"] >= 1 and rec["single_thread"]["cores"] == 1 and rec["single_thread"]["value"] > 0
    assert "median" in rec["sample"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_is_used_only_for_the_kernels_it_measured(monkeypatch):
    """The HBM traffic figure comes from a committed counter summary that
    names the kernel sources it measured (a hash); once the sources differ
    it is reported as unknown rather than carried over."""
    rec = bench.measured_traffic("opt13b", 0)
    import json
    import os
    path = os.path.join(bench.ROOT, "profiles", "decode_kernel_opt13b_traffic.json")
    stored = json.load(open(path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: stored["kernel_source_sha"])
    assert bench.measured_traffic("opt13b", 0) == stored["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("opt13b", 0) is None
    assert bench.measured_traffic("no_such_workload", 0) is None
    assert rec is None or rec == stored["hbm_bytes_per_launch"]


def test_kernel_source_hash_covers_every_kernel_source():
    import hashlib
    import os
    csrc = os.path.join(bench.ROOT, "paged_kv_cache_375_amd", "csrc")
    files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    assert "decode.hip" in files and "decode_group.hip" in files and "decode_common.h" in files
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    assert bench.kernel_source_hash() == h.hexdigest()[:16]
