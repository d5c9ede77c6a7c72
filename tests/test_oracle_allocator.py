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
    return (list(a.free), list(a.refcount), {s: list(t) for s, t in a.tables.items()}, dict(a.ctx), list(a.arrival))


def random_trace(a, rng, steps, max_seq=12):
    live = []
    nxt = 0
    for _ in range(steps):
        op = rng.integers(0, 10)
        before = snapshot(a)
        try:
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
            else:
                s = int(rng.choice(live))
                a.free_seq(s)
                live.remove(s)
        except OutOfBlocks:
            assert snapshot(a) == before  # a failed call changes nothing
        check_invariants(a)
        if len(live) > max_seq:
            s = live.pop(0)
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
