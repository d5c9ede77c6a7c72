"""Kernel timing for measurement (pa_timing_enable / pa_timing_read; needs an
MI355X).  While enabled, every decode call records a pair of HIP events
around its launches on its stream; a read returns their summed time and
count and resets them; at most 4096 calls are kept between reads."""
import pytest
import torch

from paged_kv_cache_375_amd import api
from tests.gpu_helpers import SMALL, build_pair

pytestmark = pytest.mark.gpu


def test_timing_counts_and_times_each_decode_call():
    dr, gpu, ref = build_pair(SMALL["opt13b_fp8_prefix"])
    api.timing_enable(False)
    try:
        api.timing_enable(True)
        for _ in range(5):
            gpu.run()              # append + decode (+ merge launch)
        for _ in range(2):
            gpu.run(shared=True)   # the shared-prefix path
        torch.cuda.synchronize()
        ms, n = api.timing_read()
        print(f"[timing] 7 calls: {n} recorded, {ms:.4f} ms", flush=True)
        assert n == 7
        assert 0.0 < ms < 7 * 5.0  # a small step's launches take microseconds
        ms2, n2 = api.timing_read()
        assert (ms2, n2) == (0.0, 0)  # a read resets
        api.timing_enable(False)
        gpu.run()
        torch.cuda.synchronize()
        assert api.timing_read() == (0.0, 0)  # nothing recorded while disabled
    finally:
        api.timing_enable(False)


def test_timing_keeps_at_most_4096_calls_between_reads():
    dr, gpu, ref = build_pair(SMALL["toy"])
    try:
        api.timing_enable(True)
        for _ in range(4100):
            gpu.run()
        torch.cuda.synchronize()
        ms, n = api.timing_read()
        print(f"[timing] 4100 calls: {n} recorded, {ms:.3f} ms", flush=True)
        assert n == 4096 and ms > 0.0
        gpu.run()
        torch.cuda.synchronize()
        assert api.timing_read()[1] == 1  # recording resumes after the read
    finally:
        api.timing_enable(False)
