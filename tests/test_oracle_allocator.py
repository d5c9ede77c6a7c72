"""Invariants of the reference allocator on random operation traces (CPU only)."""
import numpy as np
import pytest

from oracle.allocator import OracleAllocator, OutOfBlocks, UnknownSeq


def check_invariants(a: OracleAllocator):
    counts = [0] * a.num_blocks
    for table in a.tables.values():
        for b in table:
            counts[b] += 1
    # refcount(b) = number of tables holding b
    assert counts == a.refcount
    # free + referenced = all blocks, and free blocks are unreferenced
    referenced = sum(1 for c in counts if c > 0)
    assert referenced + len(a.free) == a.num_blocks
    assert all(counts[b] == 0 for b in a.free)
    assert len(set(a.free)) == len(a.free)
    for s, table in a.tables.items():
        # blocks exactly cover the context
        assert len(table) == -(-a.ctx[s] // a.block_size)


def snapshot(a):
    return (list(a.free), list(a.refcount), {s: list(t) for s, t in a.tables.items()}, dict(a.ctx), list(a.arrival),
            dict(a.swapped))


def random_trace(a, rng, steps, max_seq=12, swaps=False):
    live, out = [], []
    nxt = 0
    for _ in range(steps):
        op = rng.integers(0, 13 if swaps else 10)
        before = snapshot(a)
        try:
            if op == 10 and live:
                s = int(rng.choice(live))
                rc_before, held = list(a.refcount), list(a.tables[s])
                assert a.swap_out(s) == held
                live.remove(s); out.append(s)
                # every block drops one reference; the length is kept
                assert all(a.refcount[b] == rc_before[b] - held.count(b) for b in set(held))
                assert a.swapped[s] == before[3][s] and s not in a.tables
                check_invariants(a)
                continue
            if op >= 11 and out:
                s = int(rng.choice(out))
                got = a.swap_in(s)
                out.remove(s); live.append(s)
                # fresh, unshared blocks that exactly cover the kept length
                assert len(got) == -(-a.ctx[s] // a.block_size) and a.ctx[s] == before[5][s]
                assert all(a.refcount[b] == 1 for b in got) and len(set(got)) == len(got)
                assert all(b in before[0] for b in got)
                check_invariants(a)
                continue
            if op >= 10:
                continue
            if op < 2 or not live:
                a.allocate(nxt, int(rng.integers(0, 3 * a.block_size + 1)))
                live.append(nxt); nxt += 1
            elif op < 3:
                a.fork(int(rng.choice(live)), nxt)
                live.append(nxt); nxt += 1
            elif op < 9:
                s = int(rng.choice(live))
                table_before = list(a.tables[s])
                rc_before = list(a.refcount)
                src, dst = a.append_slot(s)
                last = (a.ctx[s] - 1) // a.block_size
                target = a.tables[s][last]
                # the write target is never shared
                assert a.refcount[target] == 1
                if src >= 0:
                    assert rc_before[src] > 1 and a.refcount[src] == rc_before[src] - 1
                    assert table_before[last] == src and target == dst
            elif out and rng.integers(0, 2):
                s = int(rng.choice(out))
                a.free_seq(s)  # a swapped-out sequence may finish without resuming
                out.remove(s)
                assert s not in a.swapped and s not in a.arrival
            else:
                s = int(rng.choice(live))
                a.free_seq(s)
                live.remove(s)
        except OutOfBlocks:
            assert snapshot(a) == before  # a failed call changes nothing
        check_invariants(a)
        assert a.latest_arrival() == next((q for q in reversed(a.arrival) if q in a.tables), None)
        if len(live) > max_seq:
            s = live.pop(0)
            a.free_seq(s)
    for s in out:
        a.free_seq(s)
    return live


@pytest.mark.parametrize("bs", [1, 4, 16])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_traces_keep_invariants(bs, seed):
    rng = np.random.default_rng(seed)
    nb = 24
    a = OracleAllocator(nb, bs, rng.permutation(nb))
    live = random_trace(a, rng, 400)
    for s in list(live):
        a.free_seq(s)
    # freeing every sequence restores every block
    assert sorted(a.free) == list(range(nb)) and all(c == 0 for c in a.refcount)


@pytest.mark.parametrize("bs", [1, 4, 16])
@pytest.mark.parametrize("seed", [3, 4])
def test_random_traces_with_swapping_keep_invariants(bs, seed):
    rng = np.random.default_rng(seed)
    nb = 24
    a = OracleAllocator(nb, bs, rng.permutation(nb))
    live = random_trace(a, rng, 600, swaps=True)
    for s in list(live):
        a.free_seq(s)
    assert sorted(a.free) == list(range(nb)) and all(c == 0 for c in a.refcount)
    assert not a.swapped and not a.arrival


def test_preemption_by_swapping_latest_arrival_first():
    """Blocks run out: the latest arrival gives up all of its blocks, the
    earlier one proceeds, and the preempted one resumes whole once blocks
    are back [F55 §放不下的时候]."""
    a = OracleAllocator(4, 2, [0, 1, 2, 3])
    a.allocate(0, 3)                   # blocks [0, 1]
    a.allocate(1, 4)                   # blocks [2, 3]
    a.append_slot(0)                   # ctx 4: still two blocks
    with pytest.raises(OutOfBlocks):
        a.append_slot(0)               # ctx 5 needs a third block
    victim = a.latest_arrival()
    assert victim == 1
    assert a.swap_out(1) == [2, 3] and a.num_free() == 2
    assert a.latest_arrival() == 0     # a swapped-out sequence is not preempted again
    assert a.append_slot(0) == (-1, -1) and a.table(0) == [0, 1, 2]
    with pytest.raises(OutOfBlocks):
        a.swap_in(1)                   # needs 2 blocks, 1 free: all or none
    assert a.swapped == {1: 4} and a.num_free() == 1
    with pytest.raises(ValueError):
        a.allocate(1, 1)               # the id is still taken
    a.free_seq(0)
    assert a.swap_in(1) == [3, 0] and a.ctx[1] == 4 and a.latest_arrival() == 1
    with pytest.raises(UnknownSeq):
        a.swap_in(1)
    # a fork's shared blocks stay with the other holder
    a.fork(1, 2)
    assert a.swap_out(2) == [3, 0] and a.refcount[3] == 1 and a.refcount[0] == 1
    a.free_seq(2)
    assert 2 not in a.arrival


def test_fifo_order_and_all_or_nothing():
    a = OracleAllocator(5, 4, [3, 1, 4, 0, 2])
    a.allocate(0, 8)
    assert a.table(0) == [3, 1]
    with pytest.raises(OutOfBlocks):
        a.allocate(1, 13)  # needs 4 blocks, 3 free
    assert a.num_free() == 3 and 1 not in a.tables
    a.allocate(1, 4)
    assert a.table(1) == [4]
    a.free_seq(0)
    assert list(a.free) == [0, 2, 3, 1]  # freed blocks join the tail in logical order
    assert a.latest_arrival() == 1
    with pytest.raises(UnknownSeq):
        a.fork(7, 8)
    with pytest.raises(UnknownSeq):
        a.append_slot(7)


def test_fork_shares_full_blocks_and_copies_partial_last_block_once():
    a = OracleAllocator(8, 4)
    a.allocate(0, 6)           # blocks [0, 1], the second holds 2 of 4
    a.fork(0, 1)
    assert a.refcount[:2] == [2, 2]
    assert a.append_slot(1) == (1, 2)  # the child copies the shared partial block
    assert a.refcount[:3] == [2, 1, 1]
    assert a.append_slot(0) == (-1, -1)  # the parent now holds block 1 alone
    a.append_slot(0)
    assert a.append_slot(0) == (-1, -1)  # ctx 8 -> 9: a fresh block
    assert a.table(0) == [0, 1, 3]
    # a full shared block stays shared
    a.fork(0, 2)
    a.allocate(3, 0)
    assert a.table(2)[:2] == [0, 1] and a.refcount[0] == 3


def test_prefix_cache_reuses_blocks_of_a_matching_prefix_only():
    """Full blocks are keyed by their tokens and everything before them
    [F55 §后来的做法]; the same tokens at another position are other content
    [F55 §模型省略了什么]."""
    a = OracleAllocator(16, 4)
    toks = list(range(10))                                  # 2 full blocks + 2 tokens
    assert a.allocate_cached(0, toks) == 0 and a.table(0) == [0, 1, 2]
    assert a.allocate_cached(1, toks) == 8 and a.table(1) == [0, 1, 3]   # the partial block is never shared
    assert a.refcount[:4] == [2, 2, 1, 1]
    assert a.allocate_cached(2, toks[:4] + [99] * 6) == 4 and a.table(2) == [0, 4, 5]
    assert a.allocate_cached(3, [99] * 4 + toks[4:8]) == 0   # block 1's tokens, but another prefix
    assert a.allocate_cached(4, [0, 1, 2, 3] * 2) == 4       # the repeat sits at another position
    check_invariants(a)


def test_prefix_cache_survives_free_until_blocks_are_taken_again():
    a = OracleAllocator(6, 2, [0, 1, 2, 3, 4, 5])
    a.allocate_cached(0, [7, 8, 9, 10, 11])                  # blocks 0, 1 keyed; 2 partial
    a.free_seq(0)
    assert list(a.free) == [3, 4, 5, 0, 1, 2]
    assert a.allocate_cached(1, [7, 8, 9, 10]) == 4 and a.table(1) == [0, 1]  # claimed back from the free list
    assert list(a.free) == [3, 4, 5, 2]
    a.free_seq(1)
    a.allocate(2, 8)                                          # takes 3, 4, 5, 2: no key is lost yet
    # block 0 is claimed back; the partial block is the free list's head, block 1,
    # whose key (7, 8, 9, 10) is dropped as it is taken for other content
    assert a.allocate_cached(3, [7, 8, 1]) == 2 and a.table(3) == [0, 1]
    assert a.cache == {(7, 8): 0}
    a.free_seq(3)
    a.free_seq(2)
    assert list(a.free) == [0, 1, 3, 4, 5, 2]
    a.allocate(4, 2)                                          # takes block 0: the key (7, 8) goes too
    assert a.allocate_cached(5, [7, 8, 9, 10]) == 0 and a.table(5) == [1, 3]
    assert a.cache == {(7, 8): 1, (7, 8, 9, 10): 3}
    with pytest.raises(OutOfBlocks):
        a.allocate_cached(6, [7, 8] + [0] * 30)               # all or none
    assert a.refcount[1] == 1 and 6 not in a.tables
    check_invariants(a)


@pytest.mark.parametrize("bs", [1, 2, 4, 16])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefix_cache_keeps_every_sequence_reading_its_own_tokens(bs, seed):
    """A ghost pool holds token ids in place of K/V: prompts write only their
    uncached tail, appends write a fresh token, copy-on-write copies blocks.
    Every live sequence must read back exactly its own tokens through its
    table, whatever it reused."""
    rng = np.random.default_rng(seed)
    nb = 40
    a = OracleAllocator(nb, bs, rng.permutation(nb))
    content = [[None] * bs for _ in range(nb)]
    hist = {}
    systems = [rng.integers(0, 5, 3 * bs + 1).tolist() for _ in range(3)]
    live, nxt = [], 0
    for _ in range(500):
        op = int(rng.integers(0, 10))
        try:
            if op < 3 or not live:
                toks = list(systems[int(rng.integers(0, 3))])[: int(rng.integers(0, 3 * bs + 2))]
                toks += rng.integers(0, 5, int(rng.integers(0, 2 * bs))).tolist()
                cached = a.allocate_cached(nxt, toks)
                assert cached % bs == 0 and toks[:cached] == [
                    content[a.tables[nxt][p // bs]][p % bs] for p in range(cached)]
                for p in range(cached, len(toks)):
                    content[a.tables[nxt][p // bs]][p % bs] = toks[p]
                hist[nxt] = toks
                live.append(nxt); nxt += 1
            elif op < 4:
                p = int(rng.choice(live))
                a.fork(p, nxt)
                hist[nxt] = list(hist[p])
                live.append(nxt); nxt += 1
            elif op < 9:
                s = int(rng.choice(live))
                src, dst = a.append_slot(s)
                if src >= 0:
                    content[dst] = list(content[src])
                pos = a.ctx[s] - 1
                t = int(rng.integers(0, 5))
                content[a.tables[s][pos // bs]][pos % bs] = t
                hist[s].append(t)
            else:
                s = int(rng.choice(live))
                a.free_seq(s)
                live.remove(s)
        except OutOfBlocks:
            pass
        check_invariants(a)
        for k, b in a.cache.items():
            assert a.key[b] == k and len(k) % bs == 0
            assert content[b] == list(k[-bs:])                 # a keyed block holds its key's last tokens
        for s in live:
            assert [content[a.tables[s][p // bs]][p % bs] for p in range(a.ctx[s])] == hist[s]
        if len(live) > 10:
            s = live.pop(0)
            a.free_seq(s)
