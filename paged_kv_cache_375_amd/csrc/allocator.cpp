// Host block allocator: the bookkeeping of paged KV storage.
//
// Rules (restated from [F55 §像内存分页, §块表, §放不下的时候, §常见问题] and
// [IPX §分离逻辑顺序与实际存储位置, §同一提示生成两个回答的假想例子]):
//   * one pool of equal blocks, one table of physical ids per sequence;
//   * a block is taken only when the sequence's earlier blocks are full;
//   * first come, first served; a request is met whole or not at all;
//   * finished sequences return their blocks;
//   * forks share blocks with reference counts; a write into a partially
//     filled block another sequence still references copies it first, the
//     original's count drops by one, full shared blocks stay shared;
//   * when blocks run out the latest arrival gives all of its blocks up, and
//     they may be moved to host memory and back: swap-out releases every
//     block of the sequence and keeps its length, swap-in takes fresh blocks
//     for the whole length, all or none.
//   * automatic prefix caching: a full prompt block is keyed by a hash of
//     its tokens and of everything before it (the previous block's key), and
//     a new sequence whose beginning matches reuses the keyed blocks, which
//     saves prompt processing, not generation [F55 §后来的做法].  Reuse stops
//     at the first miss.  A key lookup also compares the stored tokens and
//     previous key, so only a 64-bit collision of two whole chains could
//     give a false hit.  A block keeps its key after its last holder frees
//     it, and loses it when taken for other content.
// The free list is first in, first out (least recently freed goes first);
// blocks freed together join its tail in logical order.  It is an intrusive
// doubly linked list, so a cached block is claimed back from the middle in
// O(1).  Every operation validates before it mutates, and makes every host
// allocation it needs (vector room, map nodes) before the first change, so a
// failing call, a failed host allocation included, leaves the state
// unchanged; no exception leaves an entry point (PA_ERR_HOST_MEMORY).
#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "internal.h"

struct pa_allocator {
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t ctx = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 1;
  // free list: intrusive, first in first out
  std::vector<int32_t> fnext, fprev;
  std::vector<uint8_t> is_free;
  int32_t fhead = -1, ftail = -1, nfree = 0;
  std::vector<int32_t> refcount;
  // prefix cache
  std::unordered_map<uint64_t, int32_t> cache;  // chain hash -> block
  std::vector<uint8_t> keyed;
  std::vector<uint64_t> key_hash, key_parent;
  std::vector<int32_t> key_tokens;  // [num_blocks][block_size], filled lazily
  std::unordered_map<int32_t, Seq> seqs;
  std::unordered_map<int32_t, int32_t> swapped;  // swapped-out sequence -> its context length
  std::vector<int32_t> arrival;  // first-come order (swapped-out sequences keep their place)

  bool exists(int32_t seq) const { return seqs.count(seq) || swapped.count(seq); }

  void push_free(int32_t b) {
    fprev[b] = ftail;
    fnext[b] = -1;
    if (ftail >= 0) fnext[ftail] = b; else fhead = b;
    ftail = b;
    is_free[b] = 1;
    ++nfree;
  }
  void unlink_free(int32_t b) {
    if (fprev[b] >= 0) fnext[fprev[b]] = fnext[b]; else fhead = fnext[b];
    if (fnext[b] >= 0) fprev[fnext[b]] = fprev[b]; else ftail = fprev[b];
    is_free[b] = 0;
    --nfree;
  }
  void release(int32_t b) {
    refcount[b] -= 1;
    if (refcount[b] == 0) push_free(b);
  }
  // The free list's head, for new content: a key it kept is dropped.
  int32_t take() {
    const int32_t b = fhead;
    unlink_free(b);
    refcount[b] = 1;
    if (!keyed.empty() && keyed[b]) {
      auto it = cache.find(key_hash[b]);
      if (it != cache.end() && it->second == b) cache.erase(it);
      keyed[b] = 0;
    }
    return b;
  }
};

namespace {

// FNV-1a, 64-bit (Fowler, Noll, Vo): the chain hash of the prefix cache.
uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001b3ull;
  }
  return h;
}
constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ull;

// Key of a full block: its tokens and the key of the block before it (0 for the first).
uint64_t block_key(uint64_t parent, const int32_t* tokens, int32_t bs) {
  return fnv1a(fnv1a(kFnvBasis, &parent, sizeof parent), tokens, sizeof(int32_t) * static_cast<size_t>(bs));
}

}  // namespace

using pa::fail;
using pa::ok;

// The body of an entry point, with a failed host allocation (the only
// exception the standard containers used here throw) turned into a status.
#define PA_GUARDED(fn, ...)                                                   \
  try {                                                                       \
    __VA_ARGS__                                                               \
  } catch (const std::bad_alloc&) {                                           \
    return fail(PA_ERR_HOST_MEMORY, "%s: out of host memory", fn);            \
  } catch (...) {                                                             \
    return fail(PA_ERR_HOST_MEMORY, "%s: unexpected host failure", fn);       \
  }

extern "C" pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                                         pa_allocator** out) noexcept {
  if (!out) return fail(PA_ERR_INVALID_ARGUMENT, "pa_allocator_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_allocator_create: num_blocks %d, block_size %d", num_blocks,
                block_size);
  pa_allocator* a = new (std::nothrow) pa_allocator;
  if (!a) return fail(PA_ERR_HOST_MEMORY, "pa_allocator_create: out of host memory");
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->refcount.assign(num_blocks, 0);
    a->fnext.assign(num_blocks, -1);
    a->fprev.assign(num_blocks, -1);
    a->is_free.assign(num_blocks, 0);
    if (free_order) {
      std::vector<char> seen(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[b]) {
          delete a;
          return fail(PA_ERR_INVALID_ARGUMENT, "pa_allocator_create: free_order is not a permutation (entry %d)",
                      i);
        }
        seen[b] = 1;
        a->push_free(b);
      }
    } else {
      for (int32_t b = 0; b < num_blocks; ++b) a->push_free(b);
    }
  } catch (...) {
    delete a;
    return fail(PA_ERR_HOST_MEMORY, "pa_allocator_create: out of host memory for %d blocks", num_blocks);
  }
  *out = a;
  return ok();
}

extern "C" void pa_allocator_destroy(pa_allocator* a) noexcept { delete a; }

extern "C" int32_t pa_allocator_num_free(const pa_allocator* a) noexcept {
  return a ? a->nfree : -1;
}

extern "C" pa_status pa_seq_allocate(pa_allocator* a, int32_t seq, int32_t num_tokens) noexcept {
  if (!a || seq < 0 || num_tokens < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_allocate: bad argument (seq %d, tokens %d)", seq, num_tokens);
  if (a->exists(seq)) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_allocate: sequence %d exists", seq);
  int64_t need = (static_cast<int64_t>(num_tokens) + a->block_size - 1) / a->block_size;
  if (need > a->nfree)
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_seq_allocate: sequence %d needs %lld blocks, %d free", seq,
                static_cast<long long>(need), a->nfree);
  PA_GUARDED("pa_seq_allocate", {
    // every allocation first: the arrival slot, the table, the map node
    a->arrival.reserve(a->arrival.size() + 1);
    pa_allocator::Seq s;
    s.blocks.reserve(need);
    pa_allocator::Seq& dst = a->seqs.emplace(seq, pa_allocator::Seq{}).first->second;
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(a->take());
    s.ctx = num_tokens;
    dst = std::move(s);
    a->arrival.push_back(seq);
    return ok();
  })
}

extern "C" pa_status pa_seq_allocate_cached(pa_allocator* a, int32_t seq, const int32_t* tokens,
                                            int32_t num_tokens, int32_t* num_cached_tokens) noexcept {
  static const char* fn = "pa_seq_allocate_cached";
  if (!a || seq < 0 || num_tokens < 0 || !num_cached_tokens || (num_tokens > 0 && !tokens))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: bad argument (seq %d, tokens %d)", fn, seq, num_tokens);
  if (a->exists(seq)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: sequence %d exists", fn, seq);
  const int32_t bs = a->block_size;
  const int64_t need = (static_cast<int64_t>(num_tokens) + bs - 1) / bs;
  const int64_t full = num_tokens / bs;
  PA_GUARDED(fn, {
  // chain keys of every full block, and the leading run of cache hits
  std::vector<uint64_t> keys(full);
  std::vector<int32_t> hits;
  uint64_t parent = 0;
  bool hitting = true;
  for (int64_t j = 0; j < full; ++j) {
    const int32_t* t = tokens + j * bs;
    keys[j] = block_key(parent, t, bs);
    if (hitting) {
      auto it = a->cache.find(keys[j]);
      const int32_t b = it == a->cache.end() ? -1 : it->second;
      hitting = b >= 0 && a->key_parent[b] == parent &&
                std::memcmp(&a->key_tokens[static_cast<size_t>(b) * bs], t, sizeof(int32_t) * bs) == 0;
      if (hitting) hits.push_back(b);
    }
    parent = keys[j];
  }
  int64_t claimed = 0;
  for (int32_t b : hits) claimed += a->refcount[b] == 0;
  if (need - static_cast<int64_t>(hits.size()) + claimed > a->nfree)
    return fail(PA_ERR_OUT_OF_BLOCKS, "%s: sequence %d needs %lld new blocks, %d free", fn, seq,
                static_cast<long long>(need - static_cast<int64_t>(hits.size()) + claimed), a->nfree);
  // every allocation before the first change: the key arrays (built aside
  // and moved in whole), map nodes for the new keys (moved into the cache
  // later without allocating), the table, the arrival slot, the sequence
  if (a->keyed.empty()) {
    std::vector<uint8_t> keyed(a->num_blocks, 0);
    std::vector<uint64_t> key_hash(a->num_blocks, 0), key_parent(a->num_blocks, 0);
    std::vector<int32_t> key_tokens(static_cast<size_t>(a->num_blocks) * bs, 0);
    a->keyed = std::move(keyed);
    a->key_hash = std::move(key_hash);
    a->key_parent = std::move(key_parent);
    a->key_tokens = std::move(key_tokens);
  }
  // (a node for every new full block: taking a block below can drop a key
  // the cache holds now, and such a key is then inserted like any other)
  std::unordered_map<uint64_t, int32_t> fresh;
  for (int64_t j = static_cast<int64_t>(hits.size()); j < full; ++j) fresh.emplace(keys[j], -1);
  a->cache.reserve(a->cache.size() + fresh.size());
  a->arrival.reserve(a->arrival.size() + 1);
  pa_allocator::Seq s;
  s.blocks.reserve(need);
  pa_allocator::Seq& dst = a->seqs.emplace(seq, pa_allocator::Seq{}).first->second;
  for (int32_t b : hits) {
    if (a->refcount[b] == 0) a->unlink_free(b);
    a->refcount[b] += 1;
    s.blocks.push_back(b);
  }
  for (int64_t j = static_cast<int64_t>(hits.size()); j < need; ++j) {
    const int32_t b = a->take();
    s.blocks.push_back(b);
    if (j < full && !a->cache.count(keys[j])) {
      auto node = fresh.extract(keys[j]);  // present: one node per distinct key, used at most once
      node.mapped() = b;
      a->cache.insert(std::move(node));
      a->keyed[b] = 1;
      a->key_hash[b] = keys[j];
      a->key_parent[b] = j > 0 ? keys[j - 1] : 0;
      std::memcpy(&a->key_tokens[static_cast<size_t>(b) * bs], tokens + j * bs, sizeof(int32_t) * bs);
    }
  }
  s.ctx = num_tokens;
  dst = std::move(s);
  a->arrival.push_back(seq);
  *num_cached_tokens = static_cast<int32_t>(hits.size()) * bs;
  return ok();
  })
}

extern "C" int32_t pa_prefix_cache_size(const pa_allocator* a) noexcept {
  return a ? static_cast<int32_t>(a->cache.size()) : -1;
}

extern "C" pa_status pa_seq_fork(pa_allocator* a, int32_t parent, int32_t child) noexcept {
  if (!a || child < 0) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_fork: bad argument");
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_fork: unknown parent %d", parent);
  if (a->exists(child)) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_fork: sequence %d exists", child);
  PA_GUARDED("pa_seq_fork", {
    a->arrival.reserve(a->arrival.size() + 1);
    pa_allocator::Seq s = it->second;
    a->seqs.emplace(child, std::move(s));  // may rehash: `it` is not used after this
    for (int32_t b : a->seqs.find(child)->second.blocks) a->refcount[b] += 1;
    a->arrival.push_back(child);
    return ok();
  })
}

extern "C" pa_status pa_seq_append_slot(pa_allocator* a, int32_t seq, int32_t* cow_src, int32_t* cow_dst) noexcept {
  if (!a || !cow_src || !cow_dst) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_append_slot: NULL argument");
  *cow_src = -1;
  *cow_dst = -1;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_append_slot: unknown sequence %d", seq);
  pa_allocator::Seq& s = it->second;
  if (s.ctx == INT32_MAX) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_append_slot: context overflow");
  if (s.ctx % a->block_size == 0) {
    PA_GUARDED("pa_seq_append_slot", s.blocks.reserve(s.blocks.size() + 1);)
    // the last block is full (or there is none): lazily take a new one
    if (a->nfree == 0)
      return fail(PA_ERR_OUT_OF_BLOCKS, "pa_seq_append_slot: no free block for sequence %d", seq);
    s.blocks.push_back(a->take());
  } else {
    int32_t last = s.blocks.back();
    if (a->refcount[last] > 1) {
      // the slot lies in a partially filled block another sequence holds
      if (a->nfree == 0)
        return fail(PA_ERR_OUT_OF_BLOCKS, "pa_seq_append_slot: no free block for the copy of block %d", last);
      int32_t dst = a->take();
      a->refcount[last] -= 1;
      s.blocks.back() = dst;
      *cow_src = last;
      *cow_dst = dst;
    }
  }
  s.ctx += 1;
  return ok();
}

extern "C" pa_status pa_seq_free(pa_allocator* a, int32_t seq) noexcept {
  if (!a) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_free: NULL allocator");
  auto sw = a->swapped.find(seq);
  if (sw != a->swapped.end()) {
    a->swapped.erase(sw);
    a->arrival.erase(std::find(a->arrival.begin(), a->arrival.end(), seq));
    return ok();
  }
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_free: unknown sequence %d", seq);
  for (int32_t b : it->second.blocks) a->release(b);
  a->seqs.erase(it);
  a->arrival.erase(std::find(a->arrival.begin(), a->arrival.end(), seq));
  return ok();
}

extern "C" pa_status pa_seq_swap_out(pa_allocator* a, int32_t seq, int32_t* block_ids, int32_t cap,
                                     int32_t* num_blocks) noexcept {
  if (!a || !num_blocks || cap < 0 || (cap > 0 && !block_ids))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_swap_out: bad argument");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_swap_out: no resident sequence %d", seq);
  const auto& blocks = it->second.blocks;
  *num_blocks = static_cast<int32_t>(blocks.size());
  if (static_cast<int64_t>(blocks.size()) > cap)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_swap_out: %zu blocks, room for %d", blocks.size(), cap);
  PA_GUARDED("pa_seq_swap_out", a->swapped.emplace(seq, it->second.ctx);)
  for (size_t j = 0; j < blocks.size(); ++j) block_ids[j] = blocks[j];
  for (int32_t b : blocks) a->release(b);
  a->seqs.erase(it);
  return ok();
}

extern "C" pa_status pa_seq_swap_in(pa_allocator* a, int32_t seq, int32_t* block_ids, int32_t cap,
                                    int32_t* num_blocks) noexcept {
  if (!a || !num_blocks || cap < 0 || (cap > 0 && !block_ids))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_swap_in: bad argument");
  auto sw = a->swapped.find(seq);
  if (sw == a->swapped.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_swap_in: no swapped-out sequence %d", seq);
  const int64_t need = (static_cast<int64_t>(sw->second) + a->block_size - 1) / a->block_size;
  *num_blocks = static_cast<int32_t>(need);
  if (need > cap) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_swap_in: %lld blocks, room for %d",
                              static_cast<long long>(need), cap);
  if (need > a->nfree)
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_seq_swap_in: sequence %d needs %lld blocks, %d free", seq,
                static_cast<long long>(need), a->nfree);
  PA_GUARDED("pa_seq_swap_in", {
    pa_allocator::Seq s;
    s.blocks.reserve(need);
    s.ctx = sw->second;
    pa_allocator::Seq& dst = a->seqs.emplace(seq, pa_allocator::Seq{}).first->second;
    for (int64_t i = 0; i < need; ++i) {
      s.blocks.push_back(a->take());
      block_ids[i] = s.blocks.back();
    }
    dst = std::move(s);
    a->swapped.erase(sw);
    return ok();
  })
}

extern "C" pa_status pa_seq_get(const pa_allocator* a, int32_t seq, int32_t* block_ids, int32_t cap,
                                int32_t* num_blocks, int32_t* context_len) noexcept {
  if (!a || cap < 0 || (cap > 0 && !block_ids)) return fail(PA_ERR_INVALID_ARGUMENT, "pa_seq_get: bad argument");
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_seq_get: unknown sequence %d", seq);
  const auto& s = it->second;
  int32_t n = static_cast<int32_t>(s.blocks.size());
  for (int32_t i = 0; i < n && i < cap; ++i) block_ids[i] = s.blocks[i];
  if (num_blocks) *num_blocks = n;
  if (context_len) *context_len = s.ctx;
  return ok();
}

extern "C" pa_status pa_export_tables(const pa_allocator* a, const int32_t* seqs, int32_t n,
                                      int32_t max_blocks_per_seq, int32_t* tables_out, int32_t* context_lens_out) noexcept {
  if (!a || n < 0 || max_blocks_per_seq < 0 || (n > 0 && (!seqs || !tables_out || !context_lens_out)))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_export_tables: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "pa_export_tables: unknown sequence %d", seqs[i]);
    if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARGUMENT, "pa_export_tables: sequence %d holds %zu blocks > %d", seqs[i],
                  it->second.blocks.size(), max_blocks_per_seq);
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = a->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + static_cast<size_t>(i) * max_blocks_per_seq;
    int32_t j = 0;
    for (; j < static_cast<int32_t>(s.blocks.size()); ++j) row[j] = s.blocks[j];
    for (; j < max_blocks_per_seq; ++j) row[j] = -1;
    context_lens_out[i] = s.ctx;
  }
  return ok();
}

extern "C" int32_t pa_block_refcount(const pa_allocator* a, int32_t block) noexcept {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refcount[block];
}

extern "C" pa_status pa_allocator_get_stats(const pa_allocator* a, pa_allocator_stats* out) noexcept {
  if (!a || !out) return fail(PA_ERR_INVALID_ARGUMENT, "pa_allocator_get_stats: NULL argument");
  out->num_blocks = a->num_blocks;
  out->num_free = a->nfree;
  out->num_shared = 0;
  for (int32_t c : a->refcount) out->num_shared += (c > 1);
  out->num_seqs = static_cast<int32_t>(a->seqs.size());
  // a slot holds a token when some sequence's context covers it; count each
  // physical (block, slot) once, so shared prefixes are not double counted
  std::vector<int32_t> filled;
  PA_GUARDED("pa_allocator_get_stats", filled.assign(a->num_blocks, 0);)
  for (const auto& kv : a->seqs) {
    const auto& s = kv.second;
    for (size_t j = 0; j < s.blocks.size(); ++j) {
      int64_t f = std::min<int64_t>(a->block_size, static_cast<int64_t>(s.ctx) - static_cast<int64_t>(j) * a->block_size);
      filled[s.blocks[j]] = std::max<int32_t>(filled[s.blocks[j]], static_cast<int32_t>(f));
    }
  }
  out->tokens_held = 0;
  for (int32_t f : filled) out->tokens_held += f;
  out->slots_allocated = static_cast<int64_t>(a->num_blocks - out->num_free) * a->block_size;
  return ok();
}

extern "C" int32_t pa_latest_arrival(const pa_allocator* a) noexcept {
  if (!a) return -1;
  for (auto it = a->arrival.rbegin(); it != a->arrival.rend(); ++it)
    if (a->seqs.count(*it)) return *it;
  return -1;
}
