"""Block allocator bookkeeping in plain Python — TEST INFRASTRUCTURE ONLY.

The rules, in the pages' words restated:
  * The cache is cut into equal blocks; a sequence's logical blocks may sit in
    any physical blocks of one shared pool [F55 §像内存分页]; each sequence
    has its own block table [F55 §块表]; [IPX §分离逻辑顺序与实际存储位置].
  * A new physical block is taken only when the sequence's earlier blocks are
    full, so a sequence wastes less than one block [F55 §块表].
  * Blocks are granted first come, first served; a sequence holds all of its
    blocks or none [F55 §放不下的时候].  Here: a request that cannot be met
    whole changes nothing.
  * A finished sequence returns its blocks to the pool [F55 §块表].
  * When blocks run out, the latest arrival is preempted first, and a
    sequence keeps all of its blocks or gives all of them up; given-up blocks
    may be moved to host memory and moved back when the sequence resumes
    [F55 §放不下的时候].  Here: swap_out releases every block of the sequence
    (their contents are to be copied out first) and keeps its length;
    swap_in takes fresh blocks for the whole length, all or none.
  * Two sequences may point at the same physical blocks (a fork of one prompt,
    or a shared prefix) [F55 §后来的做法]; [IPX §同一提示生成两个回答的假想例子].
    Blocks carry a reference count.  Before a write into a partially filled
    block that another sequence still references, the block is copied, the
    write goes to the copy, and the original's count drops by one; full shared
    blocks stay shared; blocks nobody references are reclaimed
    [F55 §常见问题 (copy-on-write)]; [IPX §同一提示生成两个回答的假想例子].

  * Automatic prefix caching: every full block is keyed by its tokens and
    all the content before it; a new sequence whose beginning matches reuses
    the existing blocks, which saves prompt processing, not generation
    [F55 §后来的做法].  The same tokens at another position are other
    content and are not shared [F55 §模型省略了什么].  Here the key is the
    whole token prefix up to the block's end, compared exactly (no hash).
    Reuse stops at the first block that misses; only full prompt blocks are
    keyed; a block keeps its key after its last holder frees it and loses it
    when it is taken for other content (first in, first out, so the least
    recently freed block goes first); a key already held by another block is
    not taken over.

Readings where the pages are silent:
  * free list order: first in, first out (allocation pops the head, a freed
    block joins the tail); blocks freed together join in logical order.
  * fill counts: only the last block of a sequence can be partial, so one
    context length per sequence determines every entry's fill,
    min(block_size, ctx - j * block_size).
"""
from collections import deque


class OutOfBlocks(Exception):
    pass


class UnknownSeq(Exception):
    pass


class OracleAllocator:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks < 0 or block_size < 1:
            raise ValueError("bad allocator size")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.refcount = [0] * num_blocks
        self.tables = {}   # seq -> list of physical ids
        self.ctx = {}      # seq -> tokens held
        self.arrival = []  # sequences in first-come order (swapped-out ones keep their place)
        self.swapped = {}  # seq -> tokens of a sequence preempted by swapping
        self.cache = {}    # full token prefix (tuple) -> block holding its last bs tokens
        self.key = {}      # block -> its prefix key, while it keeps one

    # -- helpers
    def _take(self):
        b = self.free.popleft()
        self.refcount[b] = 1
        if b in self.key:  # taken for other content: its cached prefix is gone
            del self.cache[self.key.pop(b)]
        return b

    def _release(self, b):
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    def num_free(self):
        return len(self.free)

    # -- operations
    def allocate(self, seq, num_tokens):
        """A new sequence whose prompt holds num_tokens: ceil(n / bs) blocks, all or none."""
        if seq in self.tables or seq in self.swapped:
            raise ValueError("sequence exists")
        if num_tokens < 0:
            raise ValueError("negative length")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks()
        self.tables[seq] = [self._take() for _ in range(need)]
        self.ctx[seq] = num_tokens
        self.arrival.append(seq)

    def allocate_cached(self, seq, tokens):
        """A new sequence with prompt `tokens`, reusing cached full blocks
        whose whole prefix matches.  All or none.  Returns the number of
        leading tokens whose K/V are already in the reused blocks."""
        if seq in self.tables or seq in self.swapped:
            raise ValueError("sequence exists")
        tokens = tuple(int(t) for t in tokens)
        bs, n = self.block_size, len(tokens)
        need = -(-n // bs)
        hits = []
        while len(hits) < n // bs:
            b = self.cache.get(tokens[: (len(hits) + 1) * bs])
            if b is None:
                break
            hits.append(b)
        claimed = sum(1 for b in hits if self.refcount[b] == 0)
        if need - len(hits) + claimed > len(self.free):
            raise OutOfBlocks()
        table = []
        for b in hits:
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
            table.append(b)
        for j in range(len(hits), need):
            b = self._take()
            table.append(b)
            k = tokens[: (j + 1) * bs]
            if (j + 1) * bs <= n and k not in self.cache:
                self.cache[k] = b
                self.key[b] = k
        self.tables[seq] = table
        self.ctx[seq] = n
        self.arrival.append(seq)
        return len(hits) * bs

    def fork(self, parent, child):
        """The child's table points at every block of the parent's."""
        if parent not in self.tables:
            raise UnknownSeq()
        if child in self.tables or child in self.swapped:
            raise ValueError("sequence exists")
        self.tables[child] = list(self.tables[parent])
        self.ctx[child] = self.ctx[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1
        self.arrival.append(child)

    def append_slot(self, seq):
        """Reserve the slot for one more token; returns (cow_src, cow_dst) or (-1, -1)."""
        if seq not in self.tables:
            raise UnknownSeq()
        table, n, bs = self.tables[seq], self.ctx[seq], self.block_size
        if n % bs == 0:
            if not self.free:
                raise OutOfBlocks()
            table.append(self._take())
            self.ctx[seq] = n + 1
            return (-1, -1)
        last = table[-1]
        if self.refcount[last] > 1:
            if not self.free:
                raise OutOfBlocks()
            dst = self._take()
            self.refcount[last] -= 1
            table[-1] = dst
            self.ctx[seq] = n + 1
            return (last, dst)
        self.ctx[seq] = n + 1
        return (-1, -1)

    def free_seq(self, seq):
        if seq in self.swapped:
            del self.swapped[seq]
            self.arrival.remove(seq)
            return
        if seq not in self.tables:
            raise UnknownSeq()
        for b in self.tables.pop(seq):
            self._release(b)
        del self.ctx[seq]
        self.arrival.remove(seq)

    def swap_out(self, seq):
        """Preempt by swapping: the sequence gives up every block (released
        like a free; the caller copies their contents to host memory first)
        and keeps its length.  Returns its blocks in logical order."""
        if seq not in self.tables:
            raise UnknownSeq()
        blocks = self.tables.pop(seq)
        for b in blocks:
            self._release(b)
        self.swapped[seq] = self.ctx.pop(seq)
        return blocks

    def swap_in(self, seq):
        """Resume a swapped-out sequence: fresh blocks for its whole length,
        all or none.  Returns them in logical order (the copy-back targets)."""
        if seq not in self.swapped:
            raise UnknownSeq()
        need = -(-self.swapped[seq] // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks()
        self.tables[seq] = [self._take() for _ in range(need)]
        self.ctx[seq] = self.swapped.pop(seq)
        return list(self.tables[seq])

    def table(self, seq):
        return list(self.tables[seq])

    def export(self, seqs, max_blocks):
        """Padded int32 tables ([n][max_blocks], -1 past the end) and lengths."""
        import numpy as np
        t = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        c = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            row = self.tables[s]
            if len(row) > max_blocks:
                raise ValueError("table longer than max_blocks")
            t[i, :len(row)] = row
            c[i] = self.ctx[s]
        return t, c

    def latest_arrival(self):
        """The sequence preempted first when blocks run out: the latest to
        arrive among those holding blocks."""
        for s in reversed(self.arrival):
            if s in self.tables:
                return s
        return None

    def utilisation(self):
        """Tokens held / (blocks in use * block_size), each shared block counted once."""
        used = self.num_blocks - len(self.free)
        if used == 0:
            return 1.0
        slots = set()
        for s, table in self.tables.items():
            for t in range(self.ctx[s]):
                slots.add((table[t // self.block_size], t % self.block_size))
        return len(slots) / (used * self.block_size)
