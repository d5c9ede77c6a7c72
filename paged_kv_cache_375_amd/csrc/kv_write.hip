// Kernels that write the paged pool: append of the new token, the prompt's
// bulk write, the block copy of copy-on-write, and the block moves between
// the pool and host memory of preemption by swapping.
//
// Pool layout: [num_blocks][num_kv_heads][block_size][head_dim] for K and V.
// Each thread moves one 16-byte chunk of the source vector (4 f32 or 8 f16
// numbers) into the pool, converting to E4M3 when the pool stores FP8.
#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// Store EPT = 16 / sizeof(ACT) numbers from src into dst (pool dtype KV).
template <typename ACT, typename KV>
struct ChunkStore;

template <typename T>
struct ChunkStore<T, T> {  // same dtype: a 16-byte copy
  static __device__ __forceinline__ void run(void* dst, const void* src, float) { store16(dst, load16(src)); }
};

template <>
struct ChunkStore<half_t, fp8_t> {  // 8 f16 -> 8 bytes
  static __device__ __forceinline__ void run(void* dst, const void* src, float inv) {
    *reinterpret_cast<uint2*>(dst) = f16x8_to_e4m3(load16(src), inv);
  }
};

template <>
struct ChunkStore<float, fp8_t> {  // 4 f32 -> 4 bytes
  static __device__ __forceinline__ void run(void* dst, const void* src, float inv) {
    *reinterpret_cast<uint32_t*>(dst) = f32x4_chunk_to_e4m3(load16(src), inv);
  }
};

// Byte offset of (block, head, slot, element) in the pool.
template <typename KV>
__device__ __forceinline__ size_t pool_offset(int64_t blk, int h, int slot, int elem, int hkv, int bs, int d) {
  return static_cast<size_t>(((blk * hkv + h) * bs + slot) * d + elem) * Elem<KV>::bytes;
}

// One thread per (sequence, KV head, 16-byte source chunk).
template <typename ACT, typename KV>
__global__ __launch_bounds__(kThreads) void append_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const char* __restrict__ k_new, const char* __restrict__ v_new,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ ctx_lens, int num_seqs, int max_blocks,
    int num_blocks, int log2_bs, int hkv, int d, float k_inv, float v_inv) {
  constexpr int EPT = 16 / Elem<ACT>::bytes;
  const int chunks = d / EPT;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= static_cast<int64_t>(num_seqs) * hkv * chunks) return;
  const int c = static_cast<int>(idx % chunks);
  const int h = static_cast<int>((idx / chunks) % hkv);
  const int s = static_cast<int>(idx / (static_cast<int64_t>(chunks) * hkv));
  const int pos = ctx_lens[s] - 1;
  if (pos < 0 || (pos >> log2_bs) >= max_blocks) return;
  const int blk = tables[static_cast<int64_t>(s) * max_blocks + (pos >> log2_bs)];
  if (blk < 0 || blk >= num_blocks) return;
  const int bs = 1 << log2_bs;
  const size_t dst = pool_offset<KV>(blk, h, pos & (bs - 1), c * EPT, hkv, bs, d);
  const size_t src = static_cast<size_t>(idx) * 16;  // [s][h][d] is contiguous in chunk order
  ChunkStore<ACT, KV>::run(kc + dst, k_new + src, k_inv);
  ChunkStore<ACT, KV>::run(vc + dst, v_new + src, v_inv);
}

// grid.y = sequence; x covers (token j < max_count, KV head, chunk).
template <typename ACT, typename KV>
__global__ __launch_bounds__(kThreads) void write_prompt_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const char* __restrict__ k_src, const char* __restrict__ v_src,
    const int64_t* __restrict__ src_row, const int32_t* __restrict__ start_pos, const int32_t* __restrict__ count,
    const int32_t* __restrict__ tables, int max_blocks, int max_count, int num_blocks, int log2_bs, int hkv, int d,
    float k_inv, float v_inv) {
  constexpr int EPT = 16 / Elem<ACT>::bytes;
  const int chunks = d / EPT;
  const int s = blockIdx.y;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per_token = static_cast<int64_t>(hkv) * chunks;
  const int64_t j = idx / per_token;
  if (j >= count[s] || j >= max_count) return;
  const int h = static_cast<int>((idx / chunks) % hkv);
  const int c = static_cast<int>(idx % chunks);
  const int64_t pos = static_cast<int64_t>(start_pos[s]) + j;
  if (pos < 0 || (pos >> log2_bs) >= max_blocks) return;
  const int blk = tables[static_cast<int64_t>(s) * max_blocks + (pos >> log2_bs)];
  if (blk < 0 || blk >= num_blocks) return;
  const int bs = 1 << log2_bs;
  const size_t dst = pool_offset<KV>(blk, h, static_cast<int>(pos & (bs - 1)), c * EPT, hkv, bs, d);
  const size_t src = ((static_cast<size_t>(src_row[s] + j) * hkv + h) * d + c * EPT) * Elem<ACT>::bytes;
  ChunkStore<ACT, KV>::run(kc + dst, k_src + src, k_inv);
  ChunkStore<ACT, KV>::run(vc + dst, v_src + src, v_inv);
}

// grid.y = pair; x covers the block's 16-byte chunks; K and V.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                               const int32_t* __restrict__ pairs, int num_blocks,
                                                               int64_t block_bytes) {
  const int src = pairs[2 * blockIdx.y], dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;
  for (int64_t off = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * 16; off < block_bytes;
       off += static_cast<int64_t>(gridDim.x) * kThreads * 16) {
    store16(kc + dst * block_bytes + off, load16(kc + src * block_bytes + off));
    store16(vc + dst * block_bytes + off, load16(vc + src * block_bytes + off));
  }
}

// Block moves between the pool and pinned host memory, one launch for the
// whole list: entry i of the host buffers is block ids[i].  Each thread moves
// 16-byte chunks of the flattened (entry, chunk) range, so consecutive lanes
// touch consecutive host bytes whatever the block size, and the host link
// sees many requests in flight at once.
template <bool TO_HOST>
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                               char* __restrict__ hk, char* __restrict__ hv,
                                                               const int32_t* __restrict__ ids, int64_t n,
                                                               int num_blocks, int64_t chunks) {
  const int64_t total = n * chunks;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; idx < total; idx += stride) {
    const int64_t i = idx / chunks;
    const int blk = ids[i];
    if (blk < 0 || blk >= num_blocks) continue;
    const int64_t pool = (static_cast<int64_t>(blk) * chunks + (idx - i * chunks)) * 16;
    const int64_t host = idx * 16;
    if (TO_HOST) {
      store16(hk + host, load16(kc + pool));
      store16(hv + host, load16(vc + pool));
    } else {
      store16(kc + pool, load16(hk + host));
      store16(vc + pool, load16(hv + host));
    }
  }
}

template <typename ACT, typename KV>
hipError_t append_t(const pa_kv_cache& c, const void* k_new, const void* v_new, const int32_t* tables,
                    const int32_t* ctx, int num_seqs, int max_blocks, hipStream_t st) {
  constexpr int EPT = 16 / Elem<ACT>::bytes;
  const int64_t threads = static_cast<int64_t>(num_seqs) * c.num_kv_heads * (c.head_dim / EPT);
  const int64_t grid = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((append_kernel<ACT, KV>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, st,
                     static_cast<char*>(c.k_cache), static_cast<char*>(c.v_cache),
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), tables, ctx, num_seqs,
                     max_blocks, c.num_blocks, __builtin_ctz(c.block_size), c.num_kv_heads, c.head_dim,
                     c.k_inv_scale, c.v_inv_scale);
  return hipGetLastError();
}

template <typename ACT, typename KV>
hipError_t write_prompt_t(const pa_kv_cache& c, const void* k_src, const void* v_src, const int64_t* src_row,
                          const int32_t* start_pos, const int32_t* count, const int32_t* tables, int num_seqs,
                          int max_blocks, int max_count, hipStream_t st) {
  constexpr int EPT = 16 / Elem<ACT>::bytes;
  const int64_t threads = static_cast<int64_t>(max_count) * c.num_kv_heads * (c.head_dim / EPT);
  const int64_t grid = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((write_prompt_kernel<ACT, KV>), dim3(static_cast<unsigned>(grid), num_seqs), dim3(kThreads),
                     0, st, static_cast<char*>(c.k_cache), static_cast<char*>(c.v_cache),
                     static_cast<const char*>(k_src), static_cast<const char*>(v_src), src_row, start_pos, count,
                     tables, max_blocks, max_count, c.num_blocks, __builtin_ctz(c.block_size), c.num_kv_heads,
                     c.head_dim, c.k_inv_scale, c.v_inv_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const pa_kv_cache& c, const void* k_new, const void* v_new, int act, const int32_t* tables,
                         const int32_t* ctx, int num_seqs, int max_blocks, hipStream_t st) {
  if (num_seqs == 0) return hipSuccess;
  if (act == PA_F32 && c.kv_dtype == PA_F32)
    return append_t<float, float>(c, k_new, v_new, tables, ctx, num_seqs, max_blocks, st);
  if (act == PA_F16 && c.kv_dtype == PA_F16)
    return append_t<half_t, half_t>(c, k_new, v_new, tables, ctx, num_seqs, max_blocks, st);
  if (act == PA_F16 && c.kv_dtype == PA_FP8_E4M3)
    return append_t<half_t, fp8_t>(c, k_new, v_new, tables, ctx, num_seqs, max_blocks, st);
  if (act == PA_F32 && c.kv_dtype == PA_FP8_E4M3)
    return append_t<float, fp8_t>(c, k_new, v_new, tables, ctx, num_seqs, max_blocks, st);
  return hipErrorInvalidValue;
}

hipError_t launch_write_prompt(const pa_kv_cache& c, const void* k_src, const void* v_src, int act,
                               const int64_t* src_row, const int32_t* start_pos, const int32_t* count,
                               const int32_t* tables, int num_seqs, int max_blocks, int max_count, hipStream_t st) {
  if (num_seqs == 0 || max_count == 0) return hipSuccess;
  if (act == PA_F32 && c.kv_dtype == PA_F32)
    return write_prompt_t<float, float>(c, k_src, v_src, src_row, start_pos, count, tables, num_seqs, max_blocks,
                                        max_count, st);
  if (act == PA_F16 && c.kv_dtype == PA_F16)
    return write_prompt_t<half_t, half_t>(c, k_src, v_src, src_row, start_pos, count, tables, num_seqs, max_blocks,
                                          max_count, st);
  if (act == PA_F16 && c.kv_dtype == PA_FP8_E4M3)
    return write_prompt_t<half_t, fp8_t>(c, k_src, v_src, src_row, start_pos, count, tables, num_seqs, max_blocks,
                                         max_count, st);
  if (act == PA_F32 && c.kv_dtype == PA_FP8_E4M3)
    return write_prompt_t<float, fp8_t>(c, k_src, v_src, src_row, start_pos, count, tables, num_seqs, max_blocks,
                                        max_count, st);
  return hipErrorInvalidValue;
}

hipError_t launch_copy_blocks(const pa_kv_cache& c, const int32_t* pairs, int n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t elem = c.kv_dtype == PA_F32 ? 4 : c.kv_dtype == PA_F16 ? 2 : 1;
  const int64_t block_bytes = static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim * elem;
  const int64_t chunks = block_bytes / 16;
  int64_t gx = (chunks + kThreads - 1) / kThreads;
  if (gx > 1024) gx = 1024;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(gx), n), dim3(kThreads), 0, st,
                     static_cast<char*>(c.k_cache), static_cast<char*>(c.v_cache), pairs, c.num_blocks,
                     block_bytes);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const pa_kv_cache& c, void* host_k, void* host_v, const int32_t* ids, int n,
                              bool to_host, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t elem = c.kv_dtype == PA_F32 ? 4 : c.kv_dtype == PA_F16 ? 2 : 1;
  const int64_t chunks = static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim * elem / 16;
  int64_t gx = (static_cast<int64_t>(n) * chunks + kThreads - 1) / kThreads;
  if (gx > 4096) gx = 4096;
  auto kern = to_host ? swap_blocks_kernel<true> : swap_blocks_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(gx)), dim3(kThreads), 0, st, static_cast<char*>(c.k_cache),
                     static_cast<char*>(c.v_cache), static_cast<char*>(host_k), static_cast<char*>(host_v), ids,
                     static_cast<int64_t>(n), c.num_blocks, chunks);
  return hipGetLastError();
}

}  // namespace pa
