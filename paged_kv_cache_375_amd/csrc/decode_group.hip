// Launches of the grouped-query decode kernel (decode_group.h): the
// partition length and wave count per launch, and the prefix pass of a
// shared-prefix decode.
#include "decode_group.h"

#include <hip/hip_runtime.h>

#include <algorithm>

namespace pa {
namespace {

template <typename KV, int D, int HT, int NW, bool UNI, bool PREFIX>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(group_occupancy<D, HT>()))) void decode_group_kernel(
    const DecodeParams P, int groups_per_kv) {
  decode_group_body<KV, D, HT, NW, UNI, PREFIX>(P, groups_per_kv, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Head tiles per workgroup: as many as the group needs, up to a register
// budget that depends on head_dim.
template <int D>
constexpr int max_head_tiles() {
  return D >= 128 ? 2 : 5;
}

// The shortest partition length (a multiple of kPartitionTokens, doubling,
// up to the table slice's kTabEntries blocks) whose worst-case workgroup
// count fits `slots` resident workgroups, so that the launch runs as one
// round; 0 if none does.
inline int one_round_part(int64_t units, int slots, int64_t span, int64_t cap) {
  for (int64_t pp = kPartitionTokens; pp <= cap; pp *= 2) {
    const int64_t parts = (span + pp - 1) / pp;
    if (units * (parts > 0 ? parts : 1) <= slots) return static_cast<int>(pp);
    if (pp >= span) break;
  }
  return 0;
}

using GroupKernel = void (*)(const DecodeParams, int);

template <typename KV, int D, int HT, int NW>
GroupKernel group_kernel(const pa_kv_cache& c) {
  return tile_addressing(c) ? decode_group_kernel<KV, D, HT, NW, true, false>
                            : decode_group_kernel<KV, D, HT, NW, false, false>;
}

template <int NW>
hipError_t launch_group(const DecodeArgs& a, int groups, GroupKernel kern, int part, int slots, int64_t units) {
  DecodeParams P = make_decode_params(a);
  P.part_tokens = part;
  const int grid_parts = decode_grid_parts(a, part);
  // one partition per unit, all resident at once: balance CUs by length
  P.fold_order = grid_parts == 1 && a.num_seqs >= 2 && a.num_seqs <= kFoldMaxSeqs &&
                 units <= static_cast<int64_t>(slots);
  // Dispatch order runs over (KV head, group), then sequences, then
  // partitions: consecutive workgroups go to different XCDs, so every
  // partition index (the first ones are the longest and the only ones
  // every sequence has) spreads evenly over the XCDs, and workgroups past a
  // sequence's last partition come last.
  const dim3 grid(static_cast<unsigned>(a.cache->num_kv_heads * groups), static_cast<unsigned>(a.num_seqs),
                  static_cast<unsigned>(grid_parts));
  if (a.ev[0]) (void)hipEventRecord(a.ev[0], a.stream);
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), 0, a.stream, P, groups);
  const hipError_t e = hipGetLastError();
  if (a.ev[1]) (void)hipEventRecord(a.ev[1], a.stream);
  return e;
}

// Waves per workgroup and partition length, per launch.  A launch runs as
// one round if it can: partitions as short as the GPU's resident slots
// allow (see one_round_part).  Eight-wave workgroups hold a CU alone (the
// accumulators leave room for no second one), so where an eight-wave launch
// fits in one round its partitions are at least twice as long as a
// four-wave launch's would be: fewer workgroups leave partials and each is
// served by twice the waves (Falcon-7B MQA layer 20.0 against 22.0 us, the
// Llama-2-70B layer's share under tensor parallelism over 8 GPUs 22.9
// against 24.6 us).  Where it does not fit (the whole Llama-2-70B layer:
// 512 units, one 4,096-token partition each on four-wave workgroups, two
// per CU), four waves; when even those need several rounds, 512-token
// partitions balance best.
template <typename KV, int D, int HT>
hipError_t launch_ht(const DecodeArgs& a, int groups) {
  const int64_t units = static_cast<int64_t>(a.cache->num_kv_heads) * groups * a.num_seqs;
  const int64_t cap = static_cast<int64_t>(kTabEntries) * a.cache->block_size;
  const int64_t span = a.max_ctx - a.min_begin;  // the longest run of a sequence's own tokens
  const GroupKernel k8 = group_kernel<KV, D, HT, 8>(*a.cache);
  const int s8 = resident_slots(reinterpret_cast<const void*>(k8), 8 * 64);
  if (const int p8 = one_round_part(units, s8, span, cap)) return launch_group<8>(a, groups, k8, p8, s8, units);
  const GroupKernel k4 = group_kernel<KV, D, HT, 4>(*a.cache);
  const int s4 = resident_slots(reinterpret_cast<const void*>(k4), 4 * 64);
  const int p4 = one_round_part(units, s4, span, cap);
  return launch_group<4>(a, groups, k4, p4 ? p4 : kPartitionTokens, s4, units);
}

template <typename KV, int D>
hipError_t launch_d(const DecodeArgs& a) {
  constexpr int HTMAX = max_head_tiles<D>();
  const int G = a.num_q_heads / a.cache->num_kv_heads;
  const int tiles = (G + 15) / 16;
  const int groups = (tiles + HTMAX - 1) / HTMAX;
  const int ht = (tiles + groups - 1) / groups;
  switch (ht) {
    case 1: return launch_ht<KV, D, 1>(a, groups);
    case 2: return launch_ht<KV, D, 2>(a, groups);
  }
  if constexpr (HTMAX >= 5) {
    switch (ht) {
      case 3: return launch_ht<KV, D, 3>(a, groups);
      case 4: return launch_ht<KV, D, 4>(a, groups);
      case 5: return launch_ht<KV, D, 5>(a, groups);
    }
  }
  return hipErrorInvalidValue;
}

// The prefix pass: rows = (sequence, query head) pairs of a group per KV
// head, in tiles of 16 * HT.
template <typename KV, int D, int HT>
hipError_t launch_prefix_ht(const DecodeArgs& a) {
  constexpr int NW = group_waves<HT>();
  auto kern = tile_addressing(*a.cache) ? decode_group_kernel<KV, D, HT, NW, true, true>
                                        : decode_group_kernel<KV, D, HT, NW, false, true>;
  DecodeParams P = make_decode_params(a);
  int max_parts = 0;
  const int cols = prefix_grid(a, HT, P, &max_parts);
  if (cols == 0 || max_parts == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(cols), static_cast<unsigned>(max_parts), 1);
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), 0, a.stream, P, 1);
  return hipGetLastError();
}

template <typename KV, int D>
hipError_t launch_prefix_d(const DecodeArgs& a) {
  constexpr int HTMAX = max_head_tiles<D>();
  const int G = a.num_q_heads / a.cache->num_kv_heads;
  int rows = 0;
  for (int g = 0; g < a.ngroups; ++g) rows = std::max(rows, (a.gstart[g + 1] - a.gstart[g]) * G);
  const int ht = std::min(HTMAX, std::max(1, (rows + 15) / 16));
  switch (ht) {
    case 1: return launch_prefix_ht<KV, D, 1>(a);
    case 2: return launch_prefix_ht<KV, D, 2>(a);
  }
  if constexpr (HTMAX >= 5) {
    switch (ht) {
      case 3: return launch_prefix_ht<KV, D, 3>(a);
      case 4: return launch_prefix_ht<KV, D, 4>(a);
      case 5: return launch_prefix_ht<KV, D, 5>(a);
    }
  }
  return hipErrorInvalidValue;
}

template <typename KV>
hipError_t launch_prefix_kv(const DecodeArgs& a) {
  switch (a.cache->head_dim) {
    case 32: return launch_prefix_d<KV, 32>(a);
    case 64: return launch_prefix_d<KV, 64>(a);
    case 128: return launch_prefix_d<KV, 128>(a);
  }
  return hipErrorInvalidValue;
}

template <typename KV>
hipError_t launch_kv(const DecodeArgs& a) {
  switch (a.cache->head_dim) {
    case 32: return launch_d<KV, 32>(a);
    case 64: return launch_d<KV, 64>(a);
    case 128: return launch_d<KV, 128>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool group_decode_applies(const DecodeArgs& a) {
  const int kv = a.cache->kv_dtype;
  return a.act == PA_F16 && (kv == PA_F16 || kv == PA_FP8_E4M3) && a.num_q_heads > a.cache->num_kv_heads;
}

hipError_t launch_decode_group(const DecodeArgs& a) {
  if (a.cache->kv_dtype == PA_F16) return launch_kv<half_t>(a);
  if (a.cache->kv_dtype == PA_FP8_E4M3) return launch_kv<fp8_t>(a);
  return hipErrorInvalidValue;
}

hipError_t launch_prefix_pass(const DecodeArgs& a) {
  if (a.act != PA_F16) return hipErrorInvalidValue;
  if (a.cache->kv_dtype == PA_F16) return launch_prefix_kv<half_t>(a);
  if (a.cache->kv_dtype == PA_FP8_E4M3) return launch_prefix_kv<fp8_t>(a);
  return hipErrorInvalidValue;
}

}  // namespace pa
