// Measurement only (pa_read_probe): how fast this GPU reads the pools with
// none of the decode's arithmetic, so that the decode kernels can be judged
// against what their access pattern allows.
//
// Paged mode runs the per-head decode kernel itself with its arithmetic
// compiled out (decode_kernel<..., LOADS_ONLY = true>): the same grid, table
// staging, 16-byte non-temporal K and V loads and loads in flight, blocks
// fetched through the table in logical order [F55 §块表].  Linear mode reads
// both pools from start to end: each workgroup streams one contiguous span
// with every lane keeping 16 loads in flight.  Each lane folds its loaded
// words with XOR and stores the result only if it equals a fixed value: the
// loads cannot be dropped, and the sink adds no traffic (atomics into a
// small sink from every wave had slowed both modes by a fifth).
#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kLinearThreads = 256;
constexpr int kLinearLoads = 16;                                     // per lane, in flight
constexpr int64_t kLinearSpan = int64_t{kLinearThreads} * kLinearLoads;  // 16-byte chunks per workgroup

// Chunks [blockIdx.x * kLinearSpan, + kLinearSpan) of the pool, lane-major in
// each load so that a wave load reads 1 KiB contiguously.
__global__ __launch_bounds__(kLinearThreads) void read_probe_linear(const char* __restrict__ pool, int64_t chunks,
                                                                     uint32_t* sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kLinearSpan + threadIdx.x;
  Vec16 x[kLinearLoads];
#pragma unroll
  for (int u = 0; u < kLinearLoads; ++u) {
    const int64_t i = min(base + u * kLinearThreads, chunks - 1);
    x[u] = load16_stream(pool + i * 16);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kLinearLoads; ++u) acc ^= x[u].w[0] ^ x[u].w[1] ^ x[u].w[2] ^ x[u].w[3];
  if (acc == kProbeMagic) sink[(blockIdx.x + threadIdx.x) & (kProbeSinkWords - 1)] = acc;
}

}  // namespace

hipError_t launch_read_probe(const pa_kv_cache& c, const int32_t* tables, const int32_t* ctx, int num_seqs,
                             int max_blocks, int max_ctx, int mode, uint32_t* sink, hipStream_t st) {
  if (mode == 0) {
    DecodeArgs a{};
    a.cache = &c;
    a.q = nullptr;
    a.out = sink;
    a.act = c.kv_dtype == PA_F32 ? PA_F32 : PA_F16;
    a.num_q_heads = c.num_kv_heads;  // every KV head read once
    a.tables = tables;
    a.ctx = ctx;
    a.num_seqs = num_seqs;
    a.max_blocks = max_blocks;
    a.max_ctx = max_ctx;
    a.max_parts = 1;
    a.sm_scale = 1.f;
    a.stream = st;
    return launch_decode_loads(a, sink);
  }
  const int row_bytes = c.head_dim * (c.kv_dtype == PA_F32 ? 4 : c.kv_dtype == PA_F16 ? 2 : 1);
  const int64_t chunks = static_cast<int64_t>(c.num_blocks) * c.num_kv_heads * c.block_size * row_bytes / 16;
  const unsigned grid = static_cast<unsigned>((chunks + kLinearSpan - 1) / kLinearSpan);
  for (const void* pool : {c.k_cache, c.v_cache})
    hipLaunchKernelGGL(read_probe_linear, dim3(grid), dim3(kLinearThreads), 0, st, static_cast<const char*>(pool),
                       chunks, sink);
  return hipGetLastError();
}

}  // namespace pa
