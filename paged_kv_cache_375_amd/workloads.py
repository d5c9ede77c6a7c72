"""Seeded synthetic inputs for paged decode — shared by the tests, the bench
and the CPU reference; it holds random draws, sizes and the order of block
allocator calls, and none of the decode's arithmetic.

Every draw uses numpy's PCG64 through ``SeedSequence(seed).spawn``, one child
stream per kind of draw, so that changing the block size (the block-size
sweep) leaves every length and every K/V number unchanged:

  stream 0: context lengths (inclusive uniform integers)
  stream 1: the pool's initial free-list order (a random permutation, i.e.
            random physical placement of every logical block)
  stream 2: q, then the cached K history, V history, then the new token's
            K and V — standard normal float32, rounded to the activation dtype

Context lengths count the token appended in the step (the new token attends
to itself); a sequence with context length n holds n - 1 tokens before the
step and appends token n - 1 during it.

Workloads (the shapes the pages discuss; lengths are uniform because the
request-length datasets the paper measured on are not available here):

  toy            the plate's machine: 44 blocks x 4 slots, 1 head, d 32, fp32,
                 6 sequences of 1..20 tokens [F55 §实验台, §模型省略了什么]
  opt13b         OPT-13B layer: 40 heads x 128 (hidden 5120), fp16, block 16,
                 30 sequences of 128..2048 [F55 §一个词元 800 KB, §快了多少]
  llama70b_gqa   Llama-2-70B layer: 64 q heads, 8 KV heads, d 128, fp16,
                 block 16, 64 sequences of 1024..4096 [F55 §后来的做法]
  falcon7b_mqa   Falcon-7B layer: 71 q heads on 1 KV head, d 64, fp16,
                 block 16, 128 sequences of 256..2048 [F55 §后来的做法]
  opt13b_fp8_prefix  OPT-13B layer, K/V stored as FP8 E4M3 with one fp32
                 scale per tensor, 64 sequences forked from one 512-token
                 prefix, each with 1..1536 further tokens
                 [F55 §后来的做法]; [IPX §同一提示生成两个回答的假想例子]
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    batch: int
    ctx_lo: int          # inclusive bounds of the post-append context length
    ctx_hi: int          # (for prefix workloads: of the per-sequence suffix)
    act: str = "f16"     # dtype of q, new K/V and the output
    kv: str = "f16"      # dtype stored in the pool
    fixed_pool: int = 0  # >0: exactly this many physical blocks
    prefix_len: int = 0  # tokens of a prefix shared by every sequence

    def with_block_size(self, bs):
        return replace(self, block_size=bs, name=f"{self.name}_bs{bs}")

    def scaled(self, batch=None, ctx_lo=None, ctx_hi=None, prefix_len=None, name=None):
        """A smaller instance of the same shape, for tests the CPU reference finishes fast."""
        return replace(self, batch=self.batch if batch is None else batch,
                       ctx_lo=self.ctx_lo if ctx_lo is None else ctx_lo,
                       ctx_hi=self.ctx_hi if ctx_hi is None else ctx_hi,
                       prefix_len=self.prefix_len if prefix_len is None else prefix_len,
                       name=name or self.name + "_small")


WORKLOADS = {
    "toy": Workload("toy", 1, 1, 32, 4, 6, 1, 20, act="f32", kv="f32", fixed_pool=44),
    "opt13b": Workload("opt13b", 40, 40, 128, 16, 30, 128, 2048),
    "llama70b_gqa": Workload("llama70b_gqa", 64, 8, 128, 16, 64, 1024, 4096),
    "falcon7b_mqa": Workload("falcon7b_mqa", 71, 1, 64, 16, 128, 256, 2048),
    "opt13b_fp8_prefix": Workload("opt13b_fp8_prefix", 40, 40, 128, 16, 64, 1, 1536,
                                  kv="e4m3", prefix_len=512),
    # correctness-only variant: the shared prefix ends inside a block, so the
    # first write of every sequence hits a partially filled shared block
    "opt13b_fp8_prefix505": Workload("opt13b_fp8_prefix505", 40, 40, 128, 16, 64, 1, 1536,
                                     kv="e4m3", prefix_len=505),
    # one GPU's share under tensor parallelism over 8 GPUs (heads split, the
    # same sequences, lengths and block tables on every GPU)
    "llama70b_gqa_tp8": Workload("llama70b_gqa_tp8", 8, 1, 128, 16, 64, 1024, 4096),
    "opt13b_tp8": Workload("opt13b_tp8", 5, 5, 128, 16, 30, 128, 2048),
}

BLOCK_SIZE_SWEEP = (1, 2, 4, 8, 16, 32, 64)

NP_DTYPE = {"f32": np.float32, "f16": np.float16, "e4m3": np.uint8}


@dataclass
class Draw:
    wl: Workload
    ctx: np.ndarray          # int32 [B], post-append context length
    num_blocks: int
    free_order: np.ndarray   # int32 [num_blocks]
    q: np.ndarray            # [B][Hq][d] act dtype
    k_hist: np.ndarray       # [rows][Hkv][d] act dtype: prefix rows, then each sequence's own rows
    v_hist: np.ndarray
    hist_row: np.ndarray     # int64 [B]: first row of sequence s's own history
    hist_start: np.ndarray   # int32 [B]: logical position of that row
    hist_count: np.ndarray   # int32 [B]: number of own history rows
    k_new: np.ndarray        # [B][Hkv][d] act dtype
    v_new: np.ndarray
    k_scale: float = 1.0     # FP8 pools: stored = e4m3(x * inv_scale), value = code * scale
    v_scale: float = 1.0
    k_inv_scale: float = 1.0
    v_inv_scale: float = 1.0

    @property
    def max_blocks(self):
        return int(max(1, -(-int(self.ctx.max()) // self.wl.block_size)))


def _normal(rng, shape, dtype):
    return rng.standard_normal(size=shape, dtype=np.float32).astype(dtype)


def _fp8_scale(hist, new):
    amax = max(float(np.abs(hist.astype(np.float32)).max(initial=0.0)),
               float(np.abs(new.astype(np.float32)).max(initial=0.0)))
    scale = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    return float(scale), float(np.float32(1.0 / np.float64(scale)))


def draw(wl: Workload, seed: int = 0) -> Draw:
    s_len, s_place, s_val, _ = np.random.SeedSequence(seed).spawn(4)
    r_len = np.random.Generator(np.random.PCG64(s_len))
    B, bs, P = wl.batch, wl.block_size, wl.prefix_len
    lens = r_len.integers(wl.ctx_lo, wl.ctx_hi, size=B, endpoint=True).astype(np.int64)
    ctx = (lens + P).astype(np.int32)

    if wl.fixed_pool:
        num_blocks = wl.fixed_pool
    else:
        # twice the blocks the step needs; with a shared prefix, its full blocks
        # count once and every sequence may need its own copy of a partial one
        shared_full = P // bs
        need = shared_full + (1 if P % bs else 0) + int(sum(-(-int(c) // bs) - shared_full for c in ctx))
        num_blocks = 2 * need
    r_place = np.random.Generator(np.random.PCG64(s_place))
    free_order = r_place.permutation(num_blocks).astype(np.int32)

    r_val = np.random.Generator(np.random.PCG64(s_val))
    act = NP_DTYPE[wl.act]
    hkv, d = wl.num_kv_heads, wl.head_dim
    q = _normal(r_val, (B, wl.num_q_heads, d), act)
    own = (ctx.astype(np.int64) - 1 - P)
    rows = P + int(own.sum())
    k_hist = _normal(r_val, (rows, hkv, d), act)
    v_hist = _normal(r_val, (rows, hkv, d), act)
    k_new = _normal(r_val, (B, hkv, d), act)
    v_new = _normal(r_val, (B, hkv, d), act)
    hist_row = (P + np.concatenate([[0], np.cumsum(own)[:-1]])).astype(np.int64)
    dr = Draw(wl, ctx, num_blocks, free_order, q, k_hist, v_hist, hist_row,
              np.full(B, P, dtype=np.int32), own.astype(np.int32), k_new, v_new)
    if wl.kv == "e4m3":
        dr.k_scale, dr.k_inv_scale = _fp8_scale(k_hist, k_new)
        dr.v_scale, dr.v_inv_scale = _fp8_scale(v_hist, v_new)
    return dr


@dataclass
class Scenario:
    """Block tables produced by one allocator for one draw."""
    prefix_table: np.ndarray   # int32 [1][max_blocks] (only for prefix workloads)
    hist_tables: np.ndarray    # int32 [B][max_blocks], the state before the step
    hist_pairs: np.ndarray     # int32 [n][2] copy-on-write copies made while building that state
    tables: np.ndarray         # int32 [B][max_blocks], after the step's slot reservation
    ctx: np.ndarray            # int32 [B]
    step_pairs: np.ndarray     # int32 [n][2] copy-on-write copies the step needs


def run_scenario(dr: Draw, alloc) -> Scenario:
    """Drive an allocator (any object with allocate / fork / append_slot /
    export) through the workload's history and one decode step.

    Plain workloads: each sequence arrives with its ctx - 1 cached tokens.
    Prefix workloads: a holder sequence (id = batch) takes the prefix, every
    sequence forks it and then reserves its own history tokens one by one.
    Then every sequence reserves the slot of the step's new token.
    """
    wl, B, P = dr.wl, dr.wl.batch, dr.wl.prefix_len
    mb = dr.max_blocks
    ids = list(range(B))
    hist_pairs = []
    prefix_table = np.zeros((0, mb), dtype=np.int32)
    if P:
        alloc.allocate(B, P)
        prefix_table, _ = alloc.export([B], mb)
        for s in ids:
            alloc.fork(B, s)
        for s in ids:
            for _ in range(int(dr.hist_count[s])):
                pr = alloc.append_slot(s)
                if pr[0] >= 0:
                    hist_pairs.append(pr)
    else:
        for s in ids:
            alloc.allocate(s, int(dr.ctx[s]) - 1)
    hist_tables, _ = alloc.export(ids, mb)
    step_pairs = []
    for s in ids:
        pr = alloc.append_slot(s)
        if pr[0] >= 0:
            step_pairs.append(pr)
    tables, ctx = alloc.export(ids, mb)
    assert np.array_equal(ctx, dr.ctx)
    as_pairs = lambda ps: np.array(ps, dtype=np.int32).reshape(-1, 2)
    return Scenario(prefix_table, hist_tables, as_pairs(hist_pairs), tables, ctx, as_pairs(step_pairs))


def two_layer_inputs(seed=0, layers=2, dim=32, positions=40):
    """Inputs of the small two-layer model (tokens, then q/k/v weights per layer).

    Weights are N(0, 1/dim) so activations stay of order one; the page prints
    neither its weight distribution nor its inputs, so these are this
    library's own draws [AIF level-3 script].
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    tokens = rng.standard_normal((positions, dim))
    weights = rng.standard_normal((layers, 3, dim, dim)) / np.sqrt(dim)
    return tokens, weights
