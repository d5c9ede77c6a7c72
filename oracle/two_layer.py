"""The two-layer cached-vs-recomputed model — TEST INFRASTRUCTURE ONLY.

The "KV 缓存" topic page (aiinfact.com), level-3 script, runs one small model
two ways and requires the same result:
  * recompute: every step runs the whole prefix through every layer, and a
    layer finishes all positions before the next layer starts (position i
    attends over positions 0..i);
  * cached: every step projects only the new position's K and V, appends them
    to the layer's cache, and attends over the cache.
Layers have square q/k/v projections only; a layer's output at a position is
its attention output, which feeds the next layer.  The page warns that a
version updating only the last position per layer passed with one layer and
diverged with two, so the model here has two layers.

Here the cached path keeps each layer's K/V in a paged pool (block size 4,
shuffled physical placement) and reads it through the C oracle's append and
paged decode, so the equivalence ties the paged decode to the recomputed
contiguous attention.

Multiply-accumulates are counted where they happen: one per multiply-add in
the projection loops, in the recomputed attention loops, and (returned by the
C oracle) in the paged decode's two dot-product loops.  Account A counts the
K and V projections only; account B counts the q/k/v projections plus the
score and weighted-sum loops [AIF level-2 knob, level-3 account table].
"""
import math

import numpy as np

from . import F64, append as paged_append, decode as paged_decode
from .allocator import OracleAllocator


class Counter:
    def __init__(self):
        self.q = self.k = self.v = self.attn = 0

    @property
    def account_a(self):
        return self.k + self.v

    @property
    def account_b(self):
        return self.q + self.k + self.v + self.attn


def matvec(W, x, counter=None, kind=None):
    out = []
    for row in W:
        acc = 0.0
        for a, b in zip(row, x):
            acc += a * b
        out.append(acc)
    if counter is not None:
        setattr(counter, kind, getattr(counter, kind) + len(W) * len(x))
    return out


def attend(q, keys, values, scale, counter=None):
    scores = []
    for k in keys:
        acc = 0.0
        for a, b in zip(q, k):
            acc += a * b
        scores.append(scale * acc)
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = sum(w)
    out = [0.0] * len(values[0])
    for t, v in enumerate(values):
        for i, vi in enumerate(v):
            out[i] += w[t] * vi
    if counter is not None:
        counter.attn += len(keys) * len(q) + len(values) * len(values[0])
    return [o / z for o in out]


def forward_all_layers(weights, tokens, counter=None):
    """Recompute path: returns per-layer outputs for every position of the prefix."""
    dim = len(tokens[0])
    scale = 1.0 / math.sqrt(dim)
    layer_in = [list(t) for t in tokens]
    per_layer = []
    for Wq, Wk, Wv in weights:
        keys = [matvec(Wk, t, counter, "k") for t in layer_in]
        values = [matvec(Wv, t, counter, "v") for t in layer_in]
        out = []
        for i, t in enumerate(layer_in):
            q = matvec(Wq, t, counter, "q")
            out.append(attend(q, keys[: i + 1], values[: i + 1], scale, counter))
        per_layer.append(out)
        layer_in = out  # the whole layer is done before the next starts
    return per_layer


class PagedCache:
    """One paged pool per layer (float64, block size 4, shuffled placement)."""

    def __init__(self, layers, dim, max_tokens, block_size=4, seed=0):
        nb = 2 * -(-max_tokens // block_size)
        order = np.random.Generator(np.random.PCG64(seed)).permutation(nb)
        self.alloc = [OracleAllocator(nb, block_size, order) for _ in range(layers)]
        for a in self.alloc:
            a.allocate(0, 0)
        self.k = [np.zeros((nb, 1, block_size, dim)) for _ in range(layers)]
        self.v = [np.zeros((nb, 1, block_size, dim)) for _ in range(layers)]
        self.max_blocks = -(-max_tokens // block_size)
        self.block_size = block_size


def gen_with_cache(weights, new_token, cache: PagedCache, counter=None):
    """Cached path: one new position through every layer."""
    dim = len(new_token)
    scale = 1.0 / math.sqrt(dim)
    x = list(new_token)
    for li, (Wq, Wk, Wv) in enumerate(weights):
        k = matvec(Wk, x, counter, "k")
        v = matvec(Wv, x, counter, "v")
        a = cache.alloc[li]
        a.append_slot(0)
        tables, ctx = a.export([0], cache.max_blocks)
        paged_append(cache.k[li], cache.v[li], np.array([[k]]), np.array([[v]]), tables, ctx, cache.block_size)
        q = matvec(Wq, x, counter, "q")
        out, macs = paged_decode(cache.k[li], cache.v[li], np.array([[q]], dtype=np.float64), tables, ctx,
                                 scale, count_macs=True)
        if counter is not None:
            counter.attn += macs
        x = list(out[0, 0])
    return x


def run_both(tokens, weights):
    """Returns (max abs difference over every prefix, recompute counter, cached counter, occupancy)."""
    positions, dim = len(tokens), len(tokens[0])
    layers = len(weights)
    rc, cc = Counter(), Counter()
    cache = PagedCache(layers, dim, positions)
    worst = 0.0
    occupancy = []
    for n in range(1, positions + 1):
        full = forward_all_layers(weights, tokens[:n], rc)[-1][-1]
        step = gen_with_cache(weights, tokens[n - 1], cache, cc)
        worst = max(worst, max(abs(a - b) for a, b in zip(full, step)))
        # numbers the caches hold: every layer keeps a K and a V vector per position
        occupancy.append(sum(a.ctx[0] for a in cache.alloc) * 2 * dim)
    return worst, rc, cc, occupancy
