"""Device state of one decode step, built from a workload draw.

Input construction (untimed): the library's allocator lays out the block
tables (``workloads.run_scenario``), the history is written into the pool by
the library's prompt-write kernel (prefix first, then the copy-on-write
copies made while sequences grew, then each sequence's own tokens).

``DecodeStep.run()`` is one step of the hot path: the step's copy-on-write
copies (if any), the append of every sequence's new K/V, and the decode —
by default the append and the decode share one launch (pa_decode_step).
With ``shared=True`` on a workload whose sequences fork one prefix, the
prefix's full blocks, which every table holds in common, go through the
shared-prefix path (pa_decode_shared_prefix): read once per KV head for all
sequences, then each sequence's own tokens.
"""
import math

import numpy as np
import torch

from . import api
from .workloads import Draw, run_scenario


def _to(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DecodeStep:
    def __init__(self, dr: Draw, device="cuda", scenario=None):
        wl = dr.wl
        self.draw = dr
        if scenario is None:
            scenario = run_scenario(dr, api.Allocator(dr.num_blocks, wl.block_size, dr.free_order))
        self.scenario = sc = scenario
        self.device = device
        self.cache = api.KVCache(dr.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv, device,
                                 dr.k_scale, dr.v_scale, dr.k_inv_scale, dr.v_inv_scale)
        k_hist, v_hist = _to(dr.k_hist, device), _to(dr.v_hist, device)
        P = wl.prefix_len
        if P:
            one = lambda v, dt: torch.tensor([v], dtype=dt, device=device)
            api.kv_write_prompt(self.cache, k_hist, v_hist, one(0, torch.int64), one(0, torch.int32),
                                one(P, torch.int32), _to(sc.prefix_table, device), P)
            if len(sc.hist_pairs):
                api.copy_blocks(self.cache, _to(sc.hist_pairs, device))
        if k_hist.shape[0] > P:
            api.kv_write_prompt(self.cache, k_hist, v_hist, _to(dr.hist_row, device), _to(dr.hist_start, device),
                                _to(dr.hist_count, device), _to(sc.hist_tables, device), int(dr.hist_count.max()))
        del k_hist, v_hist
        self.q = _to(dr.q, device)
        self.k_new = _to(dr.k_new, device)
        self.v_new = _to(dr.v_new, device)
        self.tables = _to(sc.tables, device)
        self.ctx = _to(sc.ctx, device)
        self.step_pairs = _to(sc.step_pairs, device) if len(sc.step_pairs) else None
        self.max_ctx = int(sc.ctx.max())
        self.sm_scale = float(np.float32(1.0 / math.sqrt(wl.head_dim)))
        self.out = torch.empty_like(self.q)
        self.workspace = api.new_workspace(wl.batch, wl.num_q_heads, wl.head_dim, self.max_ctx, device)
        # full prefix blocks: every sequence's table starts with them (a
        # partial last prefix block is each sequence's own after copy-on-write)
        self.shared_blocks = P // wl.block_size
        self.shared_workspace = None
        if self.shared_blocks:
            assert (sc.tables[:, : self.shared_blocks] == sc.tables[0, : self.shared_blocks]).all()
            need = api.shared_workspace_size(wl.batch, wl.num_q_heads, wl.head_dim, self.max_ctx,
                                             self.shared_blocks * wl.block_size)
            self.shared_workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=device)

    def run(self, cache=None, stream=None, fused=True, shared=False):
        """One step: copy-on-write copies, then append + decode (one launch when fused;
        a prefix pass first when shared and the workload has a shared prefix)."""
        c = cache or self.cache
        if self.step_pairs is not None:
            api.copy_blocks(c, self.step_pairs, stream)
        if shared and self.shared_blocks:
            B = self.q.shape[0]
            if not fused:
                api.kv_append(c, self.k_new, self.v_new, self.tables, self.ctx, stream)
            api.decode_shared_prefix(c, self.q, self.tables, self.ctx, self.max_ctx, self.sm_scale, [0, B],
                                     [self.shared_blocks], self.k_new if fused else None,
                                     self.v_new if fused else None, self.out, self.shared_workspace, stream)
        elif fused:
            api.decode_step(c, self.q, self.k_new, self.v_new, self.tables, self.ctx, self.max_ctx, self.sm_scale,
                            self.out, self.workspace, stream)
        else:
            api.kv_append(c, self.k_new, self.v_new, self.tables, self.ctx, stream)
            api.decode(c, self.q, self.tables, self.ctx, self.max_ctx, self.sm_scale, self.out, self.workspace,
                       stream)
        return self.out
