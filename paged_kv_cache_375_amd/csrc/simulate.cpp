// The toy machine's arrival simulator, driven by the library's own block
// allocator: sequences arrive, write one token per round, wait when they do
// not fit, are preempted latest-arrival-first by swapping when blocks run
// out, and leave when done [F55 §实验台, §放不下的时候].
//
// A round runs in four steps.
//   1. Growth: running sequences take this round's slot, earliest arrival
//      first.  When no block is free, pa_latest_arrival names the sequence
//      to swap out.  It keeps its tokens and rejoins the queue; if it is the
//      sequence asking, that one writes nothing this round.
//   2. Admission, only in a round without preemption: queued sequences
//      strictly first come, first served, while the head's whole need
//      (its tokens so far plus this round's) is free.
//   3. Readout of running sequences, tokens held and slots reserved.
//   4. Departure of sequences that have written all of their tokens.
#include <algorithm>
#include <numeric>
#include <vector>

#include "internal.h"

using pa::fail;
using pa::ok;

namespace {

struct AllocatorGuard {
  pa_allocator* a = nullptr;
  ~AllocatorGuard() { pa_allocator_destroy(a); }
};

pa_status simulate(int32_t num_blocks, int32_t block_size, const int32_t* arrivals, const int32_t* lengths,
                   int32_t n, pa_arrival_readout* out, int32_t* trace, int32_t trace_cap) {
  static const char* fn = "pa_simulate_arrivals";
  if (!out || n < 0 || num_blocks < 0 || block_size < 1 || trace_cap < 0 || (trace_cap > 0 && !trace) ||
      (n > 0 && (!arrivals || !lengths)))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: bad argument", fn);
  int64_t round_cap = 1;  // every round with a queue or a runner writes at least one token
  for (int32_t i = 0; i < n; ++i) {
    if (arrivals[i] < 0 || lengths[i] < 1)
      return fail(PA_ERR_INVALID_ARGUMENT, "%s: sequence %d has arrival %d, length %d", fn, i, arrivals[i],
                  lengths[i]);
    if ((static_cast<int64_t>(lengths[i]) + block_size - 1) / block_size > num_blocks)
      return fail(PA_ERR_INVALID_ARGUMENT, "%s: sequence %d (%d tokens) exceeds the pool", fn, i, lengths[i]);
    round_cap += lengths[i];
  }
  if (n > 0) round_cap += *std::max_element(arrivals, arrivals + n);

  AllocatorGuard g;
  if (pa_status s = pa_allocator_create(num_blocks, block_size, nullptr, &g.a)) return s;
  std::vector<int32_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return arrivals[x] < arrivals[y]; });
  std::vector<int32_t> rank(n);
  for (int32_t k = 0; k < n; ++k) rank[order[k]] = k;
  const auto by_rank = [&](int32_t x, int32_t y) { return rank[x] < rank[y]; };

  std::vector<int32_t> written(n, 0), queue, running, ids(std::max(num_blocks, 1));
  int32_t arrived = 0, done = 0, rounds = 0, max_conc = 0, preemptions = 0;
  double util_sum = 0.0;
  int32_t util_n = 0;
  int32_t cnt = 0, src = 0, dst = 0;
  while (done < n) {
    if (rounds >= round_cap) return fail(PA_ERR_INVALID_ARGUMENT, "%s: no progress after %d rounds", fn, rounds);
    while (arrived < n && arrivals[order[arrived]] <= rounds) queue.push_back(order[arrived++]);
    std::sort(queue.begin(), queue.end(), by_rank);

    // 1. growth
    bool preempted = false;
    const std::vector<int32_t> snapshot = running;
    for (int32_t s : snapshot) {
      if (std::find(running.begin(), running.end(), s) == running.end()) continue;
      for (;;) {
        const pa_status st = pa_seq_append_slot(g.a, s, &src, &dst);
        if (st == PA_OK) {
          written[s] += 1;
          break;
        }
        if (st != PA_ERR_OUT_OF_BLOCKS) return st;
        const int32_t victim = pa_latest_arrival(g.a);
        if (pa_status e = pa_seq_swap_out(g.a, victim, ids.data(), static_cast<int32_t>(ids.size()), &cnt)) return e;
        running.erase(std::find(running.begin(), running.end(), victim));
        queue.insert(std::upper_bound(queue.begin(), queue.end(), victim, by_rank), victim);
        ++preemptions;
        preempted = true;
        if (victim == s) break;
      }
    }

    // 2. admission
    while (!queue.empty() && !preempted) {
      const int32_t s = queue.front();
      const int64_t need = (static_cast<int64_t>(written[s]) + block_size) / block_size;
      if (need > pa_allocator_num_free(g.a)) break;
      if (written[s] == 0) {
        if (pa_status e = pa_seq_allocate(g.a, s, 1)) return e;
      } else {
        if (pa_status e = pa_seq_swap_in(g.a, s, ids.data(), static_cast<int32_t>(ids.size()), &cnt)) return e;
        if (pa_status e = pa_seq_append_slot(g.a, s, &src, &dst)) return e;
      }
      written[s] += 1;
      queue.erase(queue.begin());
      running.insert(std::upper_bound(running.begin(), running.end(), s, by_rank), s);
    }

    // 3. readout
    int64_t held = 0;
    for (int32_t s : running) held += written[s];
    const int64_t reserved = static_cast<int64_t>(num_blocks - pa_allocator_num_free(g.a)) * block_size;
    if (rounds < trace_cap) {
      trace[3 * rounds] = static_cast<int32_t>(running.size());
      trace[3 * rounds + 1] = static_cast<int32_t>(held);
      trace[3 * rounds + 2] = static_cast<int32_t>(reserved);
    }
    max_conc = std::max(max_conc, static_cast<int32_t>(running.size()));
    if (reserved > 0) {
      util_sum += static_cast<double>(held) / static_cast<double>(reserved);
      ++util_n;
    }

    // 4. departures
    for (size_t k = 0; k < running.size();) {
      const int32_t s = running[k];
      if (written[s] == lengths[s]) {
        if (pa_status e = pa_seq_free(g.a, s)) return e;
        running.erase(running.begin() + static_cast<std::ptrdiff_t>(k));
        ++done;
      } else {
        ++k;
      }
    }
    ++rounds;
  }
  out->max_concurrent = max_conc;
  out->rounds = rounds;
  out->preemptions = preemptions;
  out->utilisation = util_n ? util_sum / util_n : 0.0;
  return ok();
}

}  // namespace

extern "C" pa_status pa_simulate_arrivals(int32_t num_blocks, int32_t block_size, const int32_t* arrivals,
                                          const int32_t* lengths, int32_t n, pa_arrival_readout* out,
                                          int32_t* trace, int32_t trace_cap) noexcept {
  // the simulation's state is its own (vectors and an allocator it
  // destroys), so a failed host allocation only ends it
  try {
    return simulate(num_blocks, block_size, arrivals, lengths, n, out, trace, trace_cap);
  } catch (...) {
    return fail(PA_ERR_HOST_MEMORY, "pa_simulate_arrivals: out of host memory");
  }
}
