// Host-side launchers of the HIP kernels (defined in the .hip files).
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "pa.h"

namespace pa {

// Tokens per split-context partition of the decode kernels.
#ifndef PA_PARTITION_TOKENS
#define PA_PARTITION_TOKENS 512
#endif
constexpr int kPartitionTokens = PA_PARTITION_TOKENS;
// Partitions one exact merge handles, hence the longest context a decode call
// accepts: kMaxPartitions * kPartitionTokens tokens.
constexpr int kMaxPartitions = 1024;
constexpr int kMaxContextLen = kMaxPartitions * kPartitionTokens;

hipError_t launch_append(const pa_kv_cache& c, const void* k_new, const void* v_new, int act, const int32_t* tables,
                         const int32_t* ctx, int num_seqs, int max_blocks, hipStream_t st);
hipError_t launch_write_prompt(const pa_kv_cache& c, const void* k_src, const void* v_src, int act,
                               const int64_t* src_row, const int32_t* start_pos, const int32_t* count,
                               const int32_t* tables, int num_seqs, int max_blocks, int max_count, hipStream_t st);
hipError_t launch_copy_blocks(const pa_kv_cache& c, const int32_t* pairs, int n, hipStream_t st);
hipError_t launch_swap_blocks(const pa_kv_cache& c, void* host_k, void* host_v, const int32_t* ids, int n,
                              bool to_host, hipStream_t st);

// Measurement only (pa_read_probe): read the pools with the decode's load
// pattern (mode 0) or start to end (mode 1), folding into a sink of
// kProbeSinkWords words.
constexpr int kProbeSinkWords = 1024;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;  // a lane stores its fold only when it equals this
// The per-head decode kernel's loads alone (paged mode of pa_read_probe).
struct DecodeArgs;
hipError_t launch_decode_loads(const DecodeArgs& a, uint32_t* sink);
hipError_t launch_read_probe(const pa_kv_cache& c, const int32_t* tables, const int32_t* ctx, int num_seqs,
                             int max_blocks, int max_ctx, int mode, uint32_t* sink, hipStream_t st);

// Shared prefixes (see pa_decode_shared_prefix): at most this many groups
// per call; the prefix pass splits each prefix into partitions of
// kPrefixPartTokens tokens.
constexpr int kMaxPrefixGroups = 16;
#ifndef PA_PREFIX_PART_TOKENS
#define PA_PREFIX_PART_TOKENS 256
#endif
constexpr int kPrefixPartTokens = PA_PREFIX_PART_TOKENS;

struct DecodeArgs {
  const pa_kv_cache* cache;
  const void* q;
  void* out;
  const void* k_new;  // non-null: append the step's new K/V in the same launch
  const void* v_new;
  int act;
  int num_q_heads;
  const int32_t* tables;
  const int32_t* ctx;
  int num_seqs;
  int max_blocks;
  int max_ctx;
  int max_parts;   // partitions the workspace holds per (sequence, head)
  float sm_scale;
  int* counters;   // [num_seqs][num_q_heads] arrival counters, zero between calls
  float* ws_ml;    // [num_seqs][num_q_heads][max_parts][2]: running max (log2 units), sum
  float* ws_o;     // [num_seqs][num_q_heads][max_parts][head_dim]: unnormalised output
  hipStream_t stream;
  hipEvent_t ev[2];  // optional timing events around the kernel (or null)
  // shared prefixes: sequences [gstart[g], gstart[g+1]) share their first
  // gtok[g] tokens (whole blocks), whose partials a prefix pass leaves in
  // workspace slots [0, gparts[g]); ngroups = 0 for plain decode
  int ngroups;
  int gstart[kMaxPrefixGroups + 1];
  int gtok[kMaxPrefixGroups];
  int gparts[kMaxPrefixGroups];
  int min_begin;  // the fewest shared tokens of any sequence (0 if one is in no group)
};

// Partitions of `part` tokens the decode grid needs: the longest context
// less the shared tokens every sequence skips.
inline int decode_grid_parts(const DecodeArgs& a, int part) {
  const int span = a.max_ctx - a.min_begin;
  return span <= 0 ? 1 : (span + part - 1) / part;
}

// Table entries a decode workgroup stages in LDS: a partition spans at most
// kTabEntries blocks.
constexpr int kTabEntries = 1024;

// Most sequences a grouped decode launch dispatches in folded length order
// (each workgroup ranks every context length in LDS).
constexpr int kFoldMaxSeqs = 256;

// Workgroups of `threads` threads of `kernel` the current device holds at
// once (compute units x workgroups per unit; cached per kernel and device);
// 0 if the device cannot be queried.
int resident_slots(const void* kernel, int threads);

// Returns hipErrorInvalidValue for an unsupported dtype/shape combination.
hipError_t launch_decode(const DecodeArgs& a);

// The grouped-query kernel (matrix cores) serves f16 activations over f16 or
// FP8 pools when several query heads share each KV head.
bool group_decode_applies(const DecodeArgs& a);
hipError_t launch_decode_group(const DecodeArgs& a);
// The prefix pass of a shared-prefix decode (f16 activations; f16 or FP8
// pools): every group's shared tokens, read once per KV head for all of the
// group's query rows, leave partials in the workspace.
hipError_t launch_prefix_pass(const DecodeArgs& a);
// A shared-prefix decode whose decode runs on the per-head kernel's two-wave
// workgroups (f16 activations, FP8 pools, one query head per KV head, blocks
// of 16 or more tokens): the prefix pass and the decode in one launch, then
// the merge launch.
bool prefix_fused_applies(const DecodeArgs& a);
hipError_t launch_decode_prefix_fused(const DecodeArgs& a);

}  // namespace pa
