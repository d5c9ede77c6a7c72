"""One decode step on the CPU reference — TEST INFRASTRUCTURE ONLY.

Takes a workload draw and the block tables the reference allocator produced
for it (both passed in; this module imports nothing from the product), builds
the pool with the oracle's own prompt write, copy and append, and decodes.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

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

    def decode_threaded(self, threads=None):
        """decode() with the (sequence, head) pairs spread over host threads:
        each thread runs the unchanged decode_pairs routine (a C call, which
        runs without the interpreter lock) on its own share, dealt longest
        context first.  Returns the same values as decode()."""
        threads = threads or host_threads()
        B, hq, d = self.dr.q.shape
        ctx = np.asarray(self.sc.ctx)
        pairs = sorted(((s, h) for s in range(B) for h in range(hq)), key=lambda p: (-int(ctx[p[0]]), p))
        shares = [pairs[i::threads] for i in range(threads)]
        out = np.zeros((B, hq, d), dtype=np.float64)

        def work(share):
            if share:
                seqs, heads = zip(*share)
                out[list(seqs), list(heads)] = self.decode_pairs(list(seqs), list(heads))

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, shares))
        return out


def host_threads():
    """Host threads to spread the reference over: the CPUs this process may
    run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))
