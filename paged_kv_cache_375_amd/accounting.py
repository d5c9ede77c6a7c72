"""Byte and flop accounting for one decode step (used by the benchmark).

The cache of B sequences over L layers with N positions each holds
B * L * N * 2 * H_kv * d_head * bytes_per_element bytes: one K and one V
vector per KV head, layer and position [AIF level-1 card]; the same count for
one token of OPT-13B is 2 * 5120 * 40 * 2 = 819,200 bytes [F55 §一个词元 800 KB].

Algorithmic bytes of one step (what the method must move, not counting any
implementation's partial results):
  every cached K/V vector of every sequence is read once (the new token's
  included), the new token's K/V are read from the caller and written into
  the pool, q is read and the output written, the block-table entries and
  lengths are read, and copy-on-write copies read and write whole blocks.
"""
from dataclasses import dataclass

import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "e4m3": 1}


def kv_bytes(batch, layers, tokens, kv_heads, head_dim, bytes_per_element):
    return batch * layers * tokens * 2 * kv_heads * head_dim * bytes_per_element


@dataclass
class StepBytes:
    kv_read: int
    kv_read_unique: int
    append: int
    q_out: int
    tables: int
    cow: int

    @property
    def total(self):
        return self.kv_read + self.append + self.q_out + self.tables + self.cow

    @property
    def total_unique(self):
        return self.kv_read_unique + self.append + self.q_out + self.tables + self.cow


def step_bytes(ctx, tables, num_q_heads, num_kv_heads, head_dim, block_size, act, kv, n_pairs=0):
    """Algorithmic bytes for one step over the realised lengths and tables.

    kv_read counts every sequence's reads (shared blocks once per reader);
    kv_read_unique counts each physical (block, slot) once.
    """
    ctx = np.asarray(ctx, dtype=np.int64)
    ea, ek = ELEM_BYTES[act], ELEM_BYTES[kv]
    per_token = 2 * num_kv_heads * head_dim * ek
    kv_read = int(ctx.sum()) * per_token
    slots = set()
    tables = np.asarray(tables)
    for s, n in enumerate(ctx.tolist()):
        for t in range(n):
            slots.add((int(tables[s, t // block_size]), t % block_size))
    kv_read_unique = len(slots) * per_token
    B = len(ctx)
    append = B * 2 * num_kv_heads * head_dim * (ea + ek)
    q_out = 2 * B * num_q_heads * head_dim * ea
    blocks = int(sum(-(-n // block_size) for n in ctx.tolist()))
    tab = 4 * blocks + 4 * B
    cow = 2 * n_pairs * num_kv_heads * block_size * head_dim * ek * 2
    return StepBytes(kv_read, kv_read_unique, append, q_out, tab, cow)


def step_flops(ctx, num_q_heads, head_dim):
    """Multiply-adds of the scores and the weighted sum, two flops each."""
    return 4 * head_dim * num_q_heads * int(np.asarray(ctx, dtype=np.int64).sum())
