"""Steps on several streams and from several host threads at once (needs an
MI355X).

Every device call is ordered on the stream it is given, and calls with
their own pools, outputs and workspaces share nothing on the device.  The
library's host state (the launch-shape cache, the last-error message) is
safe to use from several threads.  Four workloads (the per-head kernel with
its merge launch, the grouped kernel for GQA and for MQA, the shared-prefix
launch over an FP8 pool) run interleaved on four streams, then from four
host threads; each result is checked against the CPU reference and each
pool after the steps is bit-exact.  Repeating a step is idempotent: the new
token is stored again in the same slot."""
import threading

import numpy as np
import pytest
import torch

from tests.gpu_helpers import SMALL, TOL, build_pair, out_f64, pool_bytes

pytestmark = pytest.mark.gpu

NAMES = ["opt13b", "llama70b_gqa", "falcon7b_mqa", "opt13b_fp8_prefix"]


def _setup():
    pairs = [build_pair(SMALL[n]) for n in NAMES]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in NAMES]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    return pairs, streams


def _run(name, gpu, stream):
    return gpu.run(stream=stream, shared=name == "opt13b_fp8_prefix")


def _check(pairs, outs):
    torch.cuda.synchronize()
    for name, (dr, gpu, ref), out in zip(NAMES, pairs, outs):
        ref.append()
        assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8)), name
        assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8)), name
        err = float(np.max(np.abs(out_f64(out) - ref.decode())))
        print(f"[streams] {name}: max abs err {err:.3e} (bound {TOL[SMALL[name].kv]})", flush=True)
        assert err <= TOL[SMALL[name].kv], name


def test_steps_interleaved_on_four_streams():
    pairs, streams = _setup()
    outs = [None] * len(NAMES)
    for _ in range(3):
        for i, (name, (dr, gpu, ref), s) in enumerate(zip(NAMES, pairs, streams)):
            outs[i] = _run(name, gpu, s)
    _check(pairs, outs)


def test_steps_from_four_host_threads():
    pairs, streams = _setup()
    outs = [None] * len(NAMES)
    errors = []

    def work(i):
        try:
            for _ in range(5):
                outs[i] = _run(NAMES[i], pairs[i][1], streams[i])
        except Exception as e:  # reported below, in the main thread
            errors.append((NAMES[i], e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(NAMES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    _check(pairs, outs)
