"""Pins of the oracle's pool operations and paged decode (CPU only).

The paged decode is compared with contiguous, unpaged brute-force attention
on logical token lists (oracle/brute.py), under random physical placement;
placement and block-size invariance, special cases and copy-on-write
behaviour are checked as properties.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute
from oracle.allocator import OracleAllocator


def _build(rng, ctx, hq, hkv, d, bs, kv_dtype=np.float32, act=np.float32, extra_blocks=3, place_rng=None):
    """Random logical K/V per sequence, placed into a shuffled pool token by token."""
    B = len(ctx)
    keys = [rng.standard_normal((c, hkv, d)).astype(act) for c in ctx]
    vals = [rng.standard_normal((c, hkv, d)).astype(act) for c in ctx]
    q = rng.standard_normal((B, hq, d)).astype(act)
    need = sum(-(-c // bs) for c in ctx)
    nb = need + extra_blocks
    alloc = OracleAllocator(nb, bs, (place_rng or rng).permutation(nb))
    mb = max(1, max(-(-c // bs) for c in ctx))
    kp = np.zeros((nb, hkv, bs, d), dtype=kv_dtype)
    vp = np.zeros_like(kp)
    for s in range(B):
        alloc.allocate(s, 0)
    # generation order: one token per step for every sequence still growing
    for t in range(max(ctx)):
        live = [s for s in range(B) if ctx[s] > t]
        for s in live:
            assert alloc.append_slot(s) == (-1, -1)
        tables, lens = alloc.export(list(range(B)), mb)
        kn = np.stack([keys[s][t] if ctx[s] > t else np.zeros((hkv, d), act) for s in range(B)])
        vn = np.stack([vals[s][t] if ctx[s] > t else np.zeros((hkv, d), act) for s in range(B)])
        idx = np.array(live)
        oracle.append(kp, vp, kn[idx], vn[idx], tables[idx], lens[idx], bs)
    tables, lens = alloc.export(list(range(B)), mb)
    assert list(lens) == list(ctx)
    return dict(kp=kp, vp=vp, q=q, keys=keys, vals=vals, tables=tables, ctx=lens, alloc=alloc)


def _brute(case, group, scale):
    q = case["q"].astype(np.float64).tolist()
    keys = [k.astype(np.float64).tolist() for k in case["keys"]]
    vals = [v.astype(np.float64).tolist() for v in case["vals"]]
    return np.array(brute.decode_contiguous(q, keys, vals, scale, group))


@pytest.mark.parametrize("bs", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("group", [1, 2, 8])
def test_paged_decode_equals_contiguous_brute_force(bs, group):
    rng = np.random.default_rng(100 * bs + group)
    hkv, d = (2 if group < 8 else 1), 8
    hq = hkv * group
    ctx = [1, 2, bs, bs + 1, 17, 40]
    case = _build(rng, ctx, hq, hkv, d, bs)
    scale = 1.0 / math.sqrt(d)
    got = oracle.decode(case["kp"], case["vp"], case["q"], case["tables"], case["ctx"], scale)
    want = _brute(case, group, scale)
    assert np.max(np.abs(got - want)) < 1e-12


def test_prompt_write_equals_token_by_token_append():
    rng = np.random.default_rng(7)
    bs, hkv, d = 4, 2, 8
    ctx = [3, 9, 12, 1]
    case = _build(rng, ctx, 2, hkv, d, bs)
    kp2 = np.zeros_like(case["kp"])
    vp2 = np.zeros_like(case["vp"])
    rows = np.concatenate(case["keys"])
    vrows = np.concatenate(case["vals"])
    start_row = np.concatenate([[0], np.cumsum(ctx)[:-1]])
    oracle.write_tokens(kp2, vp2, rows, vrows, start_row, np.zeros(4), np.array(ctx), case["tables"])
    assert np.array_equal(kp2, case["kp"]) and np.array_equal(vp2, case["vp"])


def test_append_touches_exactly_the_target_slots():
    rng = np.random.default_rng(8)
    bs, hkv, d = 4, 3, 8
    case = _build(rng, [5, 8, 2], 3, hkv, d, bs)
    kp = case["kp"].copy()
    before = kp.copy()
    vp = case["vp"].copy()
    kn = rng.standard_normal((3, hkv, d)).astype(np.float32) + 10.0  # values no slot holds yet
    oracle.append(kp, vp, kn, kn, case["tables"], case["ctx"], bs)
    changed = np.argwhere(np.any(kp != before, axis=-1))
    assert len(changed) == 3 * hkv  # every (sequence, head) wrote one slot, nothing else moved
    # the decode now sees the new token as the last key of each sequence
    for s, c in enumerate(case["ctx"]):
        case["keys"][s][c - 1] = kn[s]
        case["vals"][s][c - 1] = kn[s]
    got = oracle.decode(kp, vp, case["q"], case["tables"], case["ctx"], 0.3)
    case2 = dict(case, kp=kp, vp=vp)
    assert np.max(np.abs(got - _brute(case2, 1, 0.3))) < 1e-12


def test_placement_invariance_is_bit_exact():
    rng = np.random.default_rng(9)
    bs = 4
    case = _build(rng, [7, 13, 20, 1], 4, 2, 16, bs)
    out = oracle.decode(case["kp"], case["vp"], case["q"], case["tables"], case["ctx"], 0.25)
    nb = case["kp"].shape[0]
    for trial in range(3):
        perm = rng.permutation(nb)  # physical block b moves to perm[b]
        kp = np.empty_like(case["kp"]); kp[perm] = case["kp"]
        vp = np.empty_like(case["vp"]); vp[perm] = case["vp"]
        tables = np.where(case["tables"] >= 0, perm[np.maximum(case["tables"], 0)], -1).astype(np.int32)
        got = oracle.decode(kp, vp, case["q"], tables, case["ctx"], 0.25)
        assert np.array_equal(got, out)


def test_block_size_invariance_is_bit_exact():
    rng = np.random.default_rng(10)
    ctx = [1, 5, 16, 33]
    base = None
    for bs in (1, 2, 4, 8, 16, 32, 64):
        r = np.random.default_rng(11)  # same logical data at every block size
        case = _build(r, ctx, 4, 1, 16, bs, extra_blocks=bs, place_rng=np.random.default_rng(bs))
        out = oracle.decode(case["kp"], case["vp"], case["q"], case["tables"], case["ctx"], 0.25)
        if base is None:
            base = out
        assert np.array_equal(out, base), bs


def test_special_cases():
    rng = np.random.default_rng(12)
    d = 16
    # one token: its weight is exactly one, so the output is V_0 exactly
    case = _build(rng, [1, 1], 2, 2, d, 4)
    out = oracle.decode(case["kp"], case["vp"], case["q"], case["tables"], case["ctx"], 0.25)
    for s in range(2):
        assert np.array_equal(out[s], case["vals"][s][0].astype(np.float64))
    # q = 0: uniform weights, the output is the mean of V
    case = _build(rng, [9, 30], 2, 2, d, 4)
    q0 = np.zeros_like(case["q"])
    out = oracle.decode(case["kp"], case["vp"], q0, case["tables"], case["ctx"], 0.25)
    for s in range(2):
        assert np.allclose(out[s], case["vals"][s].astype(np.float64).mean(axis=0), atol=1e-14, rtol=0)
    # a dominant score: the output is that token's V
    case = _build(rng, [12], 1, 1, d, 4)
    kp = case["kp"]
    t_dom = 5
    blk = case["tables"][0, t_dom // 4]
    kp[blk, 0, t_dom % 4] = case["q"][0, 0] * 100.0
    out = oracle.decode(kp, case["vp"], case["q"], case["tables"], case["ctx"], 1.0)
    assert np.allclose(out[0, 0], case["vals"][0][t_dom, 0].astype(np.float64), atol=1e-12, rtol=0)
    # a zero-length context writes zeros
    out = oracle.decode(kp, case["vp"], case["q"], case["tables"], np.array([0], np.int32), 1.0)
    assert np.array_equal(out, np.zeros_like(out))


def test_f16_and_fp8_pools_decode_their_stored_values():
    rng = np.random.default_rng(13)
    ctx = [3, 17]
    case16 = _build(rng, ctx, 2, 1, 16, 4, kv_dtype=np.float16, act=np.float16)
    out = oracle.decode(case16["kp"], case16["vp"], case16["q"], case16["tables"], case16["ctx"], 0.25)
    assert np.max(np.abs(out - _brute(case16, 2, 0.25))) < 1e-12
    # FP8: the brute force sees the dequantised stored values
    k_scale, v_scale = np.float32(0.01), np.float32(0.02)
    k_inv, v_inv = np.float32(1 / np.float64(k_scale)), np.float32(1 / np.float64(v_scale))
    kp = np.zeros(case16["kp"].shape, np.uint8)
    vp = np.zeros_like(kp)
    rows_k = np.concatenate(case16["keys"])
    rows_v = np.concatenate(case16["vals"])
    oracle.write_tokens(kp, vp, rows_k, rows_v, [0, 3], [0, 0], ctx, case16["tables"], k_inv, v_inv)
    deq = lambda x, inv, sc: np.array([oracle.e4m3_to_f64(oracle.e4m3_quantize(v, inv)) * float(sc)
                                       for v in x.ravel().tolist()]).reshape(x.shape)
    case8 = dict(case16, keys=[deq(k, k_inv, k_scale) for k in case16["keys"]],
                 vals=[deq(v, v_inv, v_scale) for v in case16["vals"]])
    out8 = oracle.decode(kp, vp, case16["q"], case16["tables"], case16["ctx"], 0.25,
                         k_scale=float(k_scale), v_scale=float(v_scale))
    assert np.max(np.abs(out8 - _brute(case8, 2, 0.25))) < 1e-12


def test_fork_and_copy_on_write_keep_each_history():
    """Two answers from one prompt: shared blocks, then a private copy of the
    partially filled last block before the first write [IPX example]."""
    rng = np.random.default_rng(14)
    bs, hkv, d = 4, 1, 8
    nb = 16
    alloc = OracleAllocator(nb, bs, rng.permutation(nb))
    prompt = rng.standard_normal((6, hkv, d)).astype(np.float32)  # 6 tokens: last block 2/4 full
    kp = np.zeros((nb, hkv, bs, d), np.float32)
    vp = np.zeros_like(kp)
    alloc.allocate(0, 6)
    t, c = alloc.export([0], 4)
    oracle.write_tokens(kp, vp, prompt, prompt, [0], [0], [6], t)
    alloc.fork(0, 1)
    hist = {0: list(prompt), 1: list(prompt)}
    for step in range(5):
        for s in (1, 0):
            tok = rng.standard_normal((1, hkv, d)).astype(np.float32)
            src, dst = alloc.append_slot(s)
            if src >= 0:
                oracle.copy_blocks(kp, vp, [[src, dst]])
            t, c = alloc.export([s], 4)
            oracle.append(kp, vp, tok, tok, t, c, bs)
            hist[s].append(tok[0])
    tables, lens = alloc.export([0, 1], 4)
    q = rng.standard_normal((2, 1, d)).astype(np.float32)
    got = oracle.decode(kp, vp, q, tables, lens, 0.5)
    case = dict(q=q, keys=[np.array(hist[0]), np.array(hist[1])], vals=[np.array(hist[0]), np.array(hist[1])])
    assert np.max(np.abs(got - _brute(case, 1, 0.5))) < 1e-12
    # the first logical block stayed shared, the second was copied once
    assert tables[0, 0] == tables[1, 0] and tables[0, 1] != tables[1, 1]
