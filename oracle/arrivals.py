"""The toy machine's arrival simulator in plain Python — TEST INFRASTRUCTURE ONLY.

The "KV 缓存与分页注意力" page (world.lapla.si, plate F55), section 实验台,
runs a toy memory of 44 blocks x 4 slots: sequences of at most 20 tokens
arrive one after another, write one token per round, leave when done, and
wait when they do not fit.  The reservation is either paged (blocks of 1, 2,
4, 8 or 16 tokens) or a whole row of the maximum length per sequence.  It
reads out the most sequences written at once, the average share of reserved
memory that holds tokens, and the rounds needed to finish them all.  The
page prints no values for these readouts.

Readings where the page is silent (each a plain choice):
  * Time runs in rounds.  In a round every running sequence writes one token.
  * Arrival round and length of every sequence are inputs.
  * A round runs in four steps:
      1. Growth.  Running sequences take this round's slot, earliest arrival
         first.  When no block is free, the latest arrival among the running
         sequences is preempted [F55 §放不下的时候].  It gives up all of its
         blocks, keeps its tokens (swap) and returns to the queue.  If it is
         the sequence asking, that sequence writes nothing this round.
      2. Admission.  If nothing was preempted this round, queued sequences are
         admitted strictly first come, first served.  The head is admitted
         only when blocks for all of its tokens, this round's included, are
         free; otherwise it and everyone behind it wait.
      3. Readout.  Running sequences, tokens held, and slots reserved
         (blocks in use x block size) are counted.
      4. Departure.  Sequences that have written all of their tokens free
         their blocks.
  * "Row" mode, where each sequence reserves the maximum length on arrival,
    is the allocator with one block of max_len slots per sequence.  The
    pool is then floor(total slots / max_len) blocks.
  * Utilisation is the mean, over rounds that reserve anything, of tokens
    held / slots reserved.

The simulator drives ``OracleAllocator``.  Its readouts are "parity
unpinned": the page prints none.  The tests pin the simulator itself with
closed forms: unlimited memory, one-token blocks, the row mode's
concurrency bound, and small cases worked by hand.
"""
from .allocator import OracleAllocator, OutOfBlocks


def simulate(num_blocks, block_size, arrivals, lengths):
    """Run the toy to completion.

    Returns dict(max_concurrent, utilisation, rounds, preemptions, trace).
    trace[r] = (running, tokens held, slots reserved) after the writes of
    round r.
    """
    n = len(lengths)
    if len(arrivals) != n or any(x < 1 for x in lengths) or any(a < 0 for a in arrivals):
        raise ValueError("every sequence needs an arrival round >= 0 and a length >= 1")
    if n and -(-max(lengths) // block_size) > num_blocks:
        raise ValueError("a sequence longer than the whole pool can never finish")
    alloc = OracleAllocator(num_blocks, block_size)
    order = sorted(range(n), key=lambda i: (arrivals[i], i))  # first come, first served
    rank = {s: k for k, s in enumerate(order)}
    written = [0] * n
    queue = []      # waiting sequences (new or preempted), kept in arrival order
    running = []    # in arrival order
    arrived = 0
    done = 0
    r = 0
    trace = []
    preemptions = 0
    while done < n:
        while arrived < n and arrivals[order[arrived]] <= r:
            queue.append(order[arrived])
            arrived += 1
        queue.sort(key=rank.get)

        # 1. growth, earliest arrival first
        preempted = False
        for s in list(running):
            if s not in running:  # preempted earlier in this round
                continue
            while True:
                try:
                    alloc.append_slot(s)
                    written[s] += 1
                    break
                except OutOfBlocks:
                    victim = max(running, key=rank.get)
                    alloc.swap_out(victim)
                    running.remove(victim)
                    queue.append(victim)
                    queue.sort(key=rank.get)
                    preemptions += 1
                    preempted = True
                    if victim == s:
                        break

        # 2. admission, strictly first come, first served
        while queue and not preempted:
            s = queue[0]
            need = -(-(written[s] + 1) // block_size)
            if need > alloc.num_free():
                break
            if written[s] == 0:
                alloc.allocate(s, 1)
            else:
                alloc.swap_in(s)
                alloc.append_slot(s)
            written[s] += 1
            queue.pop(0)
            running.append(s)
            running.sort(key=rank.get)

        # 3. readout
        held = sum(written[s] for s in running)
        reserved = (num_blocks - alloc.num_free()) * block_size
        trace.append((len(running), held, reserved))

        # 4. departures
        for s in list(running):
            if written[s] == lengths[s]:
                alloc.free_seq(s)
                running.remove(s)
                done += 1
        r += 1

    samples = [h / v for _, h, v in trace if v > 0]
    return {
        "max_concurrent": max((c for c, _, _ in trace), default=0),
        "utilisation": sum(samples) / len(samples) if samples else 0.0,
        "rounds": len(trace),
        "preemptions": preemptions,
        "trace": trace,
    }


def toy_pool(total_slots, block_size, max_len):
    """(num_blocks, block_size) for a paged option, or for the row option (block_size None)."""
    if block_size is None:
        return total_slots // max_len, max_len
    return total_slots // block_size, block_size
