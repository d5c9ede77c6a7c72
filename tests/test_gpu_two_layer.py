"""The "KV 缓存" topic page's two-layer model run end to end through the HIP
path (needs an MI355X).

Each of the two layers keeps its K/V in its own paged f32 pool (block size 4,
shuffled placement; one block table serves both layers).  Every generation
step projects only the new position and runs pa_decode_step (append +
attention) per layer.  The last layer's output at every prefix must match
the oracle's recompute path, where every step runs the whole prefix through
both layers, within 1e-5 [AIF level-3 script].  Two layers, because a
single layer cannot tell a correct cache from one that feeds the second
layer stale inputs [AIF level-3 findings].
"""
import math

import numpy as np
import pytest
import torch

from oracle import two_layer
from paged_kv_cache_375_amd import api
from paged_kv_cache_375_amd.workloads import two_layer_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [True, False], ids=["decode_step", "append+decode"])
def test_two_layer_model_cached_on_gpu_equals_recomputed(fused):
    layers, dim, positions, bs = 2, 32, 40, 4
    tokens, weights = two_layer_inputs(0, layers, dim, positions)
    print(f"[two-layer] {layers} layers x dim {dim} x {positions} positions, fused={fused}", flush=True)
    want = two_layer.recompute(weights, tokens)  # [positions][dim], last layer

    nb = 2 * -(-positions // bs)
    order = np.random.Generator(np.random.PCG64(7)).permutation(nb)
    alloc = api.Allocator(nb, bs, order)
    alloc.allocate(0, 0)
    caches = [api.KVCache(nb, bs, 1, dim, "f32", "cuda") for _ in range(layers)]
    max_blocks = -(-positions // bs)
    w32 = weights.astype(np.float32)
    sm_scale = float(np.float32(1.0 / math.sqrt(dim)))
    workspace = api.new_workspace(1, 1, dim, positions, "cuda")
    got = np.zeros((positions, dim))
    for n in range(positions):
        assert alloc.append_slot(0) == (-1, -1)
        tables, ctx = alloc.export([0], max_blocks)
        tables_d = torch.from_numpy(tables).cuda()
        ctx_d = torch.from_numpy(ctx).cuda()
        x = tokens[n].astype(np.float32)
        for li in range(layers):
            Wq, Wk, Wv = w32[li]
            dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).reshape(1, 1, dim)).cuda()
            q, k, v = dev(Wq @ x), dev(Wk @ x), dev(Wv @ x)
            if fused:
                out = api.decode_step(caches[li], q, k, v, tables_d, ctx_d, positions, sm_scale,
                                      workspace=workspace)
            else:
                api.kv_append(caches[li], k, v, tables_d, ctx_d)
                out = api.decode(caches[li], q, tables_d, ctx_d, positions, sm_scale, workspace=workspace)
            torch.cuda.synchronize()
            x = out.cpu().numpy().reshape(dim)
        got[n] = x
    err = float(np.max(np.abs(got - want)))
    print(f"[two-layer] max abs difference over {positions} prefixes: {err:.3e}", flush=True)
    assert err <= 1e-5
