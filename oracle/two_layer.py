"""The two-layer cached-vs-recomputed model — TEST INFRASTRUCTURE ONLY.

The "KV 缓存" topic page (aiinfact.com), level-3 script, describes one small
attention model (two layers of width 32, 40 positions) computed two ways that
must agree:

  * without a cache, producing position n means running the whole prefix
    0..n through both layers again; inside a layer every position is brought
    up to date before the next layer begins, and position i only looks at
    positions 0..i;
  * with a cache, only the newest position's K and V are projected in each
    layer and added to that layer's store; the query of the new position then
    attends over everything the store holds.

A layer has square query, key and value projections and nothing else; what it
hands to the next layer at a position is its attention output there.  The
page retracted an earlier version whose uncached path refreshed only the last
position per layer: with one layer it agreed, with two it did not.

Written here in matrix form.  The uncached path of one layer is

    Q = X Wq^T,  K = X Wk^T,  V = X Wv^T          (X: [n][D], one row per position)
    S = (Q K^T) / sqrt(D),  S[i][j] = -inf for j > i   (the causal mask)
    Y = softmax_rows(S) V                          (max-subtracted, float64)

and Y becomes the next layer's X.  The cached path keeps each layer's K and V
in a paged pool (block size 4, shuffled physical placement) written by the C
oracle's append and read by its paged decode, so the agreement of the two
paths also ties the paged decode to plain causal attention.

Multiply-accumulates are counted as the page's two accounts do
[AIF level-2 knob, level-3 account table]: account A is the K and V
projections; account B adds the Q projection, the scores and the weighted
sums.  A product of an [n][D] matrix by a [D][D] one is n * D * D of them;
causal attention costs D for the score and D for the weighted sum of every
(query, key) pair the mask lets through; the paged decode reports its own
count.  Softmax, scaling and the mask itself are not counted.
"""
import numpy as np

from . import append as paged_append, decode as paged_decode
from .allocator import OracleAllocator


class MacCount:
    """Multiply-accumulates per kind: projections (q, k, v) and attention."""

    def __init__(self):
        self.proj = {"q": 0, "k": 0, "v": 0}
        self.attention = 0

    @property
    def account_a(self):
        return self.proj["k"] + self.proj["v"]

    @property
    def account_b(self):
        return sum(self.proj.values()) + self.attention


def project(W, X, count=None, kind=None):
    """Rows of X mapped by W: X W^T, float64."""
    W = np.asarray(W, dtype=np.float64)
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    if count is not None:
        count.proj[kind] += X.shape[0] * W.shape[0] * W.shape[1]
    return X @ W.T


def causal_attention(Q, K, V, first_pos=0, count=None):
    """Scaled dot-product attention of query rows at positions first_pos,
    first_pos + 1, ... over key/value rows 0..len(K)-1; the query at
    position p sees keys 0..p only."""
    Q, K, V = (np.atleast_2d(np.asarray(a, dtype=np.float64)) for a in (Q, K, V))
    dim = Q.shape[1]
    pos = first_pos + np.arange(Q.shape[0])[:, None]
    allowed = np.arange(K.shape[0])[None, :] <= pos
    S = np.where(allowed, (Q @ K.T) / np.sqrt(dim), -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    if count is not None:
        count.attention += int(allowed.sum()) * dim * 2
    return P @ V


def recompute(weights, tokens, count=None):
    """Uncached path: the outputs of the last layer at every position of the
    prefix `tokens`, each layer brought fully up to date before the next."""
    X = np.asarray(tokens, dtype=np.float64)
    for Wq, Wk, Wv in weights:
        Q = project(Wq, X, count, "q")
        K = project(Wk, X, count, "k")
        V = project(Wv, X, count, "v")
        X = causal_attention(Q, K, V, 0, count)
    return X


class PagedStores:
    """One paged K/V pool per layer (float64, 1 head, block size 4), each
    with its own allocator whose free list is a seeded shuffle, holding one
    sequence (id 0)."""

    def __init__(self, layers, dim, max_positions, block_size=4, seed=0):
        self.block_size = block_size
        self.max_blocks = -(-max_positions // block_size)
        nblocks = 2 * self.max_blocks
        self.layers = []
        for _ in range(layers):
            order = np.random.Generator(np.random.PCG64(seed)).permutation(nblocks)
            alloc = OracleAllocator(nblocks, block_size, order)
            alloc.allocate(0, 0)
            pools = (np.zeros((nblocks, 1, block_size, dim)), np.zeros((nblocks, 1, block_size, dim)))
            self.layers.append((alloc, pools))

    def numbers_held(self):
        """How many numbers the stores hold: a K and a V vector per position per layer."""
        return sum(alloc.ctx[0] * 2 * pools[0].shape[-1] for alloc, pools in self.layers)


def cached_step(weights, token, stores: PagedStores, count=None):
    """Cached path: the newest position through every layer; returns the last
    layer's output there.  Each layer reserves the slot, stores the new K and
    V through the block table, then decodes over the whole table."""
    x = np.asarray(token, dtype=np.float64)[None, :]
    for (Wq, Wk, Wv), (alloc, (kpool, vpool)) in zip(weights, stores.layers):
        k_row = project(Wk, x, count, "k")
        v_row = project(Wv, x, count, "v")
        alloc.append_slot(0)
        table, lens = alloc.export([0], stores.max_blocks)
        paged_append(kpool, vpool, k_row[:, None, :], v_row[:, None, :], table, lens, stores.block_size)
        q_row = project(Wq, x, count, "q")
        y, macs = paged_decode(kpool, vpool, q_row[:, None, :], table, lens, 1.0 / np.sqrt(x.shape[1]),
                               count_macs=True)
        if count is not None:
            count.attention += macs
        x = y[:, 0, :]
    return x[0]


def run_both(tokens, weights):
    """Both paths over every prefix of `tokens`.  Returns (largest absolute
    difference seen, uncached MAC count, cached MAC count, numbers held by the
    caches after each position)."""
    tokens = np.asarray(tokens, dtype=np.float64)
    weights = np.asarray(weights, dtype=np.float64)
    uncached, cached = MacCount(), MacCount()
    stores = PagedStores(len(weights), tokens.shape[1], len(tokens))
    worst, held = 0.0, []
    for n in range(1, len(tokens) + 1):
        want = recompute(weights, tokens[:n], uncached)[-1]
        got = cached_step(weights, tokens[n - 1], stores, cached)
        worst = max(worst, float(np.max(np.abs(want - got))))
        held.append(stores.numbers_held())
    return worst, uncached, cached, held
