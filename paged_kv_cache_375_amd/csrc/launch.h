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
};

// Table entries a decode workgroup stages in LDS: a partition spans at most
// kTabEntries blocks.
constexpr int kTabEntries = 1024;

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

}  // namespace pa
