"""The decode step captured in a HIP graph and replayed (needs an MI355X).

Serving loops capture their per-token launches.  A step (copy-on-write
copies, append + decode, the merge launch or the prefix pass where the path
has them) is captured once and replayed several times, with other GPU work
and synchronisations between replays; every replay must give the eager
step's output bit for bit, leave the pool as the reference does, and leave
the grouped kernel's arrival counters at zero for the next replay."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import SMALL, TOL, build_pair, out_f64, pool_bytes

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(SMALL))
def test_step_replays_from_a_hip_graph(name):
    wl = SMALL[name]
    print(f"[graph] {name}", flush=True)
    dr, gpu, ref = build_pair(wl)
    shared = bool(gpu.shared_blocks)
    eager = out_f64(gpu.run(shared=shared))

    # warm up on a side stream, as graph capture asks, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu.run(shared=shared)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.run(shared=shared)
    torch.cuda.synchronize()

    for i in range(3):
        gpu.out.fill_(float("nan"))  # a fill kernel, outside the graph
        graph.replay()
        torch.cuda.synchronize()
        got = out_f64(gpu.out)
        assert np.array_equal(got, eager), f"replay {i} differs from the eager step"
        # unrelated eager work between replays
        x = torch.randn(1 << 16, device="cuda")
        assert torch.isfinite((x * 2.0).sum()).item()

    ref.append()
    assert np.array_equal(pool_bytes(gpu.cache.k), ref.k.view(np.uint8))
    assert np.array_equal(pool_bytes(gpu.cache.v), ref.v.view(np.uint8))
    err = float(np.max(np.abs(eager - ref.decode())))
    print(f"[graph] {name}: 3 replays bit-identical to eager, max abs err {err:.3e}", flush=True)
    assert err <= TOL[wl.kv]
