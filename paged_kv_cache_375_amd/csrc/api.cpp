// The C ABI of the device operations: host-side argument checks (never
// reading device memory), dispatch to the kernels, and kernel timing.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.h"
#include "launch.h"

using pa::fail;
using pa::ok;

namespace {

constexpr int kMaxGridYZ = 65535;

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

pa_status check_cache(const pa_kv_cache* c, const char* fn) {
  if (!c) return fail(PA_ERR_INVALID_ARGUMENT, "%s: cache is NULL", fn);
  if (!c->k_cache || !c->v_cache) return fail(PA_ERR_INVALID_ARGUMENT, "%s: k_cache/v_cache is NULL", fn);
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_blocks %d, num_kv_heads %d", fn, c->num_blocks, c->num_kv_heads);
  if (!is_pow2(c->block_size) || c->block_size > 64)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d is not a power of two in 1..64", fn, c->block_size);
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {32, 64, 128}", fn, c->head_dim);
  if (c->kv_dtype != PA_F32 && c->kv_dtype != PA_F16 && c->kv_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: kv_dtype %d", fn, c->kv_dtype);
  if (c->kv_dtype == PA_FP8_E4M3 &&
      !(c->k_scale > 0.f && c->v_scale > 0.f && c->k_inv_scale > 0.f && c->v_inv_scale > 0.f))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: FP8 scales must be positive", fn);
  return PA_OK;
}

pa_status check_act(const pa_kv_cache* c, int32_t act, const char* fn) {
  const bool okpair = (act == PA_F32 && (c->kv_dtype == PA_F32 || c->kv_dtype == PA_FP8_E4M3)) ||
                      (act == PA_F16 && (c->kv_dtype == PA_F16 || c->kv_dtype == PA_FP8_E4M3));
  if (!okpair) return fail(PA_ERR_UNSUPPORTED, "%s: activation dtype %d with pool dtype %d", fn, act, c->kv_dtype);
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

int32_t max_parts_for(int32_t max_context_len) {
  return max_context_len <= 0 ? 1 : (max_context_len + pa::kPartitionTokens - 1) / pa::kPartitionTokens;
}

// ---- kernel timing ----------------------------------------------------------
constexpr int kTimingSlots = 4096;
struct Timing {
  bool on = false;
  std::vector<hipEvent_t> part_ev;  // start/stop pairs around each decode kernel
  int n_part = 0;
};
Timing g_timing;

void timing_release() {
  for (hipEvent_t e : g_timing.part_ev) (void)hipEventDestroy(e);
  g_timing = Timing();
}

}  // namespace

extern "C" pa_status pa_kv_append(const pa_kv_cache* cache, const void* k_new, const void* v_new, int32_t act,
                                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_blocks_per_seq, void* stream) noexcept {
  static const char* fn = "pa_kv_append";
  if (pa_status s = check_cache(cache, fn)) return s;
  if (pa_status s = check_act(cache, act, fn)) return s;
  if (num_seqs < 0 || max_blocks_per_seq < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (num_seqs > 0 && (!k_new || !v_new || !block_tables || !context_lens))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: NULL device pointer", fn);
  return hip_status(pa::launch_append(*cache, k_new, v_new, act, block_tables, context_lens, num_seqs,
                                      max_blocks_per_seq, static_cast<hipStream_t>(stream)),
                    fn);
}

extern "C" pa_status pa_kv_write_prompt(const pa_kv_cache* cache, const void* k_src, const void* v_src, int32_t act,
                                        const int64_t* src_row, const int32_t* start_pos, const int32_t* count,
                                        const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                                        int32_t max_count, void* stream) noexcept {
  static const char* fn = "pa_kv_write_prompt";
  if (pa_status s = check_cache(cache, fn)) return s;
  if (pa_status s = check_act(cache, act, fn)) return s;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_count < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
  if (num_seqs > kMaxGridYZ) return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs %d > %d", fn, num_seqs, kMaxGridYZ);
  if (num_seqs > 0 && max_count > 0 && (!k_src || !v_src || !src_row || !start_pos || !count || !block_tables))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: NULL device pointer", fn);
  return hip_status(pa::launch_write_prompt(*cache, k_src, v_src, act, src_row, start_pos, count, block_tables,
                                            num_seqs, max_blocks_per_seq, max_count,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

extern "C" pa_status pa_copy_blocks(const pa_kv_cache* cache, const int32_t* src_dst_pairs, int32_t n,
                                    void* stream) noexcept {
  static const char* fn = "pa_copy_blocks";
  if (pa_status s = check_cache(cache, fn)) return s;
  if (n < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: negative pair count", fn);
  if (n > kMaxGridYZ) return fail(PA_ERR_UNSUPPORTED, "%s: %d pairs > %d per call", fn, n, kMaxGridYZ);
  if (n > 0 && !src_dst_pairs) return fail(PA_ERR_INVALID_ARGUMENT, "%s: pairs is NULL", fn);
  return hip_status(pa::launch_copy_blocks(*cache, src_dst_pairs, n, static_cast<hipStream_t>(stream)), fn);
}

extern "C" pa_status pa_swap_blocks(const pa_kv_cache* cache, void* host_k, void* host_v, const int32_t* block_ids,
                                    int32_t n, int32_t direction, void* stream) noexcept {
  static const char* fn = "pa_swap_blocks";
  if (pa_status s = check_cache(cache, fn)) return s;
  if (n < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: negative block count", fn);
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: direction %d", fn, direction);
  if (n == 0) return ok();
  if (!host_k || !host_v || !block_ids) return fail(PA_ERR_INVALID_ARGUMENT, "%s: NULL pointer", fn);
  // The kernel reaches host memory through its device mapping; memory the
  // runtime does not know as pinned is refused here rather than faulting.
  void* dk = nullptr;
  void* dv = nullptr;
  if (hipHostGetDevicePointer(&dk, host_k, 0) != hipSuccess || hipHostGetDevicePointer(&dv, host_v, 0) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: host buffers must be pinned host memory (hipHostMalloc)", fn);
  }
  return hip_status(pa::launch_swap_blocks(*cache, dk, dv, block_ids, n, direction == PA_SWAP_OUT,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

// Workspace: arrival counters [num_seqs][num_q_heads] int32 (padded to 256
// bytes), then (max, sum) pairs and unnormalised vectors per partition.
// A workspace starts with the arrival counters (one int32 per (sequence,
// query head) row), then the partials ((max, sum) and head_dim floats per row
// and partition).  The counters' region is sized by the workspace itself,
// for the most rows any call could use it for: a row that needs a workspace
// takes its counter and at least two partials of head_dim + 2 >= 34 floats
// (kMinRowBytes).  So on one workspace the counters of every call lie below
// the partials of every call, whatever their batch: each call leaves its
// counters at zero, and no call's partials land on a later call's counters.
constexpr size_t kMinRowBytes = sizeof(int32_t) + 2 * (32 + 2) * sizeof(float);

static size_t counters_region(size_t workspace_bytes) {
  const size_t b = workspace_bytes / kMinRowBytes * sizeof(int32_t);
  return (b + 255) & ~static_cast<size_t>(255);
}

static size_t partials_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t parts) {
  return static_cast<size_t>(num_seqs) * num_q_heads * parts * (head_dim + 2) * sizeof(float);
}

// The least size W whose room past counters_region(W) holds the partials
// with 256 bytes to spare, so that every larger size holds them too (the
// region grows 256 bytes at a time, once per 64 * kMinRowBytes bytes of W):
// W >= (partials + 512) * kMinRowBytes / (kMinRowBytes - 4) leaves W -
// counters_region(W) >= W (1 - 4 / kMinRowBytes) - 255 >= partials + 257.
static size_t workspace_bytes_for(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t parts) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || parts <= 1) return 0;
  const size_t t = partials_bytes(num_seqs, num_q_heads, head_dim, parts) + 512;
  return (t * kMinRowBytes + (kMinRowBytes - sizeof(int32_t)) - 1) / (kMinRowBytes - sizeof(int32_t));
}

// Partials per (sequence, head) of a shared-prefix decode: the prefix pass's
// (kPrefixPartTokens each) and the decode launch's (at least
// kPartitionTokens each).
static int32_t shared_parts_for(int32_t max_context_len, int32_t max_shared_tokens) {
  const int32_t pre = max_shared_tokens <= 0 ? 0 : (max_shared_tokens + pa::kPrefixPartTokens - 1) / pa::kPrefixPartTokens;
  return pre + max_parts_for(max_context_len);
}

extern "C" size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                           int32_t max_context_len) noexcept {
  return workspace_bytes_for(num_seqs, num_q_heads, head_dim, max_parts_for(max_context_len));
}

extern "C" size_t pa_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                                  int32_t max_context_len, int32_t max_shared_tokens) noexcept {
  return workspace_bytes_for(num_seqs, num_q_heads, head_dim, shared_parts_for(max_context_len, max_shared_tokens));
}

namespace pa {

int resident_slots(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({kernel, dev});
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess) return 0;
  const int n = cus * (per > 0 ? per : 1);
  try {
    cache[{kernel, dev}] = n;  // the answer stands even when it cannot be kept
  } catch (...) {
  }
  return n;
}

}  // namespace pa

namespace {

pa_status decode_common(const char* fn, const pa_kv_cache* cache, const void* q, const void* k_new, const void* v_new,
                        void* out, int32_t act, int32_t num_q_heads, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                        int32_t max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
                        void* stream, int32_t num_groups = 0, const int32_t* group_start = nullptr,
                        const int32_t* group_shared_blocks = nullptr) {
  if (pa_status s = check_cache(cache, fn)) return s;
  if (pa_status s = check_act(cache, act, fn)) return s;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq < 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: bad size (seqs %d, q heads %d, max blocks %d, max ctx %d)", fn,
                num_seqs, num_q_heads, max_blocks_per_seq, max_context_len);
  if (num_q_heads % cache->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", fn, num_q_heads,
                cache->num_kv_heads);
  if (num_seqs > kMaxGridYZ || num_q_heads > kMaxGridYZ)
    return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs %d / num_q_heads %d above %d", fn, num_seqs, num_q_heads,
                kMaxGridYZ);
  if (max_context_len > pa::kMaxContextLen)
    return fail(PA_ERR_UNSUPPORTED, "%s: max_context_len %d above %d", fn, max_context_len, pa::kMaxContextLen);
  if (!(sm_scale == sm_scale)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: sm_scale is NaN", fn);
  // shared prefixes: host arrays, checked before anything else is touched
  int32_t max_shared = 0;
  if (num_groups < 0 || num_groups > pa::kMaxPrefixGroups)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d shared-prefix groups (at most %d)", fn, num_groups, pa::kMaxPrefixGroups);
  if (num_groups > 0) {
    if (!group_start || !group_shared_blocks) return fail(PA_ERR_INVALID_ARGUMENT, "%s: NULL group array", fn);
    if (group_start[0] < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: group_start[0] = %d", fn, group_start[0]);
    for (int32_t g = 0; g < num_groups; ++g) {
      if (group_start[g + 1] < group_start[g] || group_start[g + 1] > num_seqs)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: group %d spans sequences [%d, %d) of %d", fn, g, group_start[g],
                    group_start[g + 1], num_seqs);
      const int64_t tok = static_cast<int64_t>(group_shared_blocks[g]) * cache->block_size;
      if (group_shared_blocks[g] < 0 || group_shared_blocks[g] > max_blocks_per_seq || tok > max_context_len)
        return fail(PA_ERR_INVALID_ARGUMENT, "%s: group %d shares %d blocks (max blocks %d, max context %d)", fn, g,
                    group_shared_blocks[g], max_blocks_per_seq, max_context_len);
      max_shared = std::max<int32_t>(max_shared, static_cast<int32_t>(tok));
    }
    if (max_shared > 0 && (act != PA_F16 || cache->kv_dtype == PA_F32))
      return fail(PA_ERR_UNSUPPORTED, "%s: shared prefixes need f16 activations and an f16 or FP8 pool", fn);
    if (shared_parts_for(max_context_len, max_shared) > pa::kMaxPartitions)
      return fail(PA_ERR_UNSUPPORTED, "%s: %d partials per head (at most %d)", fn,
                  shared_parts_for(max_context_len, max_shared), pa::kMaxPartitions);
  }
  if (num_seqs == 0) return ok();
  if (!q || !out || !block_tables || !context_lens || (k_new == nullptr) != (v_new == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: NULL device pointer", fn);
  const int32_t parts = max_shared > 0 ? shared_parts_for(max_context_len, max_shared) : max_parts_for(max_context_len);
  const size_t need = workspace_bytes_for(num_seqs, num_q_heads, cache->head_dim, parts);
  // (the size suffices for the layout; both conditions are checked as well)
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   counters_region(workspace_bytes) < static_cast<size_t>(num_seqs) * num_q_heads * sizeof(int32_t) ||
                   workspace_bytes - counters_region(workspace_bytes) <
                       partials_bytes(num_seqs, num_q_heads, cache->head_dim, parts)))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);

  pa::DecodeArgs a{};
  a.cache = cache;
  a.q = q;
  a.out = out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.act = act;
  a.num_q_heads = num_q_heads;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.max_parts = parts;
  a.sm_scale = sm_scale;
  if (max_shared > 0) {
    a.ngroups = num_groups;
    for (int32_t g = 0; g <= num_groups; ++g) a.gstart[g] = group_start[g];
    for (int32_t g = 0; g < num_groups; ++g) {
      a.gtok[g] = group_shared_blocks[g] * cache->block_size;
      a.gparts[g] = (a.gtok[g] + pa::kPrefixPartTokens - 1) / pa::kPrefixPartTokens;
    }
    // every sequence skips at least min_begin tokens when the groups cover
    // the whole batch (a sequence of no group skips none)
    int32_t covered = 0, min_begin = INT32_MAX;
    for (int32_t g = 0; g < num_groups; ++g) {
      const int32_t n = group_start[g + 1] - group_start[g];
      covered += n;
      if (n > 0) min_begin = std::min(min_begin, a.gtok[g]);
    }
    a.min_begin = covered == num_seqs && min_begin != INT32_MAX ? min_begin : 0;
  }
  if (need > 0) {
    char* base = static_cast<char*>(workspace);
    a.counters = reinterpret_cast<int*>(base);
    a.ws_ml = reinterpret_cast<float*>(base + counters_region(workspace_bytes));
    a.ws_o = a.ws_ml + static_cast<size_t>(num_seqs) * num_q_heads * a.max_parts * 2;
  }
  a.stream = static_cast<hipStream_t>(stream);
  const bool timed = g_timing.on && g_timing.n_part < kTimingSlots;
  if (timed) {
    a.ev[0] = g_timing.part_ev[2 * g_timing.n_part];
    a.ev[1] = g_timing.part_ev[2 * g_timing.n_part + 1];
  }
  hipError_t e = hipSuccess;
  if (a.ngroups > 0) {
    // Where the decode runs on the per-head kernel's two-wave workgroups (FP8
    // pools), the prefix pass shares its launch and a merge launch follows.
    // Otherwise the prefix pass comes first, then the decode launch, on the
    // caller's stream: the grouped decode's first partition of each head
    // starts from the prefix's partials.  (A prefix pass beside the decode on
    // a second stream was slower: its workgroups waited for slots the
    // decode's kept refilling.)  The timing events bracket everything.
    if (a.ev[0]) (void)hipEventRecord(a.ev[0], a.stream);
    a.ev[0] = nullptr;
    if (pa::prefix_fused_applies(a)) {
      e = pa::launch_decode_prefix_fused(a);
    } else {
      e = pa::launch_prefix_pass(a);
      if (e == hipSuccess) e = pa::launch_decode(a);
    }
  } else {
    e = pa::launch_decode(a);
  }
  if (e == hipErrorInvalidValue) return fail(PA_ERR_UNSUPPORTED, "%s: unsupported dtype/shape combination", fn);
  if (timed && e == hipSuccess) g_timing.n_part += 1;
  return hip_status(e, fn);
}

}  // namespace

extern "C" pa_status pa_decode(const pa_kv_cache* cache, const void* q, void* out, int32_t act, int32_t num_q_heads,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t max_context_len, float sm_scale, void* workspace,
                               size_t workspace_bytes, void* stream) noexcept {
  return decode_common("pa_decode", cache, q, nullptr, nullptr, out, act, num_q_heads, block_tables, context_lens,
                       num_seqs, max_blocks_per_seq, max_context_len, sm_scale, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_decode_step(const pa_kv_cache* cache, const void* q, const void* k_new, const void* v_new,
                                    void* out, int32_t act, int32_t num_q_heads, const int32_t* block_tables,
                                    const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                                    int32_t max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
                                    void* stream) noexcept {
  if (num_seqs > 0 && (!k_new || !v_new))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_step: k_new/v_new is NULL");
  return decode_common("pa_decode_step", cache, q, k_new, v_new, out, act, num_q_heads, block_tables, context_lens,
                       num_seqs, max_blocks_per_seq, max_context_len, sm_scale, workspace, workspace_bytes, stream);
}

extern "C" pa_status pa_decode_shared_prefix(const pa_kv_cache* cache, const void* q, const void* k_new,
                                             const void* v_new, void* out, int32_t act, int32_t num_q_heads,
                                             const int32_t* block_tables, const int32_t* context_lens,
                                             int32_t num_seqs, int32_t max_blocks_per_seq, int32_t max_context_len,
                                             float sm_scale, int32_t num_groups, const int32_t* group_start,
                                             const int32_t* group_shared_blocks, void* workspace,
                                             size_t workspace_bytes, void* stream) noexcept {
  return decode_common("pa_decode_shared_prefix", cache, q, k_new, v_new, out, act, num_q_heads, block_tables,
                       context_lens, num_seqs, max_blocks_per_seq, max_context_len, sm_scale, workspace,
                       workspace_bytes, stream, num_groups, group_start, group_shared_blocks);
}

extern "C" pa_status pa_read_probe(const pa_kv_cache* cache, const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t mode,
                                   uint32_t* sink, void* stream) noexcept {
  static const char* fn = "pa_read_probe";
  if (pa_status s = check_cache(cache, fn)) return s;
  if (mode != 0 && mode != 1) return fail(PA_ERR_INVALID_ARGUMENT, "%s: mode %d", fn, mode);
  if (!sink) return fail(PA_ERR_INVALID_ARGUMENT, "%s: sink is NULL", fn);
  if (mode == 0) {
    if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "%s: negative size", fn);
    if (num_seqs > kMaxGridYZ || (max_context_len + pa::kPartitionTokens - 1) / pa::kPartitionTokens > kMaxGridYZ)
      return fail(PA_ERR_UNSUPPORTED, "%s: grid too large", fn);
    if (num_seqs > 0 && (!block_tables || !context_lens)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: NULL table", fn);
  }
  return hip_status(pa::launch_read_probe(*cache, block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                          max_context_len, mode, sink, static_cast<hipStream_t>(stream)),
                    fn);
}

extern "C" pa_status pa_timing_enable(int32_t on) noexcept {
  timing_release();
  if (!on) return ok();
  try {
    g_timing.part_ev.resize(2 * kTimingSlots);
  } catch (...) {
    return fail(PA_ERR_HOST_MEMORY, "pa_timing_enable: out of host memory");
  }
  for (hipEvent_t& e : g_timing.part_ev) {
    // Timing only: no system-scope fence (cache writeback and invalidation)
    // when an event completes, which would otherwise add several
    // microseconds between the kernels it brackets and the next launch.
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (r != hipSuccess) {
      e = nullptr;
      timing_release();
      return fail(PA_ERR_HIP, "pa_timing_enable: %s", hipGetErrorString(r));
    }
  }
  g_timing.on = true;
  return ok();
}

extern "C" pa_status pa_timing_read(double* decode_ms, int32_t* decode_launches) noexcept {
  if (!decode_ms || !decode_launches) return fail(PA_ERR_INVALID_ARGUMENT, "pa_timing_read: NULL argument");
  *decode_ms = 0.0;
  *decode_launches = g_timing.n_part;
  for (int i = 0; i < g_timing.n_part; ++i) {
    float ms = 0.f;
    hipError_t r = hipEventSynchronize(g_timing.part_ev[2 * i + 1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_timing.part_ev[2 * i], g_timing.part_ev[2 * i + 1]);
    if (r != hipSuccess) return fail(PA_ERR_HIP, "pa_timing_read: %s", hipGetErrorString(r));
    *decode_ms += ms;
  }
  g_timing.n_part = 0;
  return ok();
}
