"""One decode step on the CPU reference — TEST INFRASTRUCTURE ONLY.

Takes a workload draw and the block tables the reference allocator produced
for it (both passed in; this module imports nothing from the product), builds
the pool with the oracle's own prompt write, copy and append, and decodes.
"""
import math

import numpy as np

from . import append, copy_blocks, decode, decode_pairs, write_tokens

_POOL_DTYPE = {"f32": np.float32, "f16": np.float16, "e4m3": np.uint8}


class ReferenceStep:
    def __init__(self, dr, scenario):
        wl = dr.wl
        self.dr, self.sc = dr, scenario
        shape = (dr.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
        self.k = np.zeros(shape, dtype=_POOL_DTYPE[wl.kv])
        self.v = np.zeros_like(self.k)
        ki, vi = dr.k_inv_scale, dr.v_inv_scale
        P = wl.prefix_len
        if P:
            write_tokens(self.k, self.v, dr.k_hist, dr.v_hist, [0], [0], [P], scenario.prefix_table, ki, vi)
            if len(scenario.hist_pairs):
                copy_blocks(self.k, self.v, scenario.hist_pairs)
        write_tokens(self.k, self.v, dr.k_hist, dr.v_hist, dr.hist_row, dr.hist_start, dr.hist_count,
                     scenario.hist_tables, ki, vi)
        self.history_k, self.history_v = self.k.copy(), self.v.copy()
        self.sm_scale = float(np.float32(1.0 / math.sqrt(wl.head_dim)))

    def append(self):
        """The step's copy-on-write copies, then the new token's K/V."""
        dr, sc = self.dr, self.sc
        if len(sc.step_pairs):
            copy_blocks(self.k, self.v, sc.step_pairs)
        append(self.k, self.v, dr.k_new, dr.v_new, sc.tables, sc.ctx, dr.wl.block_size, dr.k_inv_scale,
               dr.v_inv_scale)

    def decode(self):
        dr = self.dr
        return decode(self.k, self.v, dr.q, self.sc.tables, self.sc.ctx, self.sm_scale, dr.k_scale, dr.v_scale)

    def decode_pairs(self, seqs, heads):
        dr = self.dr
        return decode_pairs(self.k, self.v, dr.q, self.sc.tables, self.sc.ctx, self.sm_scale, seqs, heads,
                            dr.k_scale, dr.v_scale)
