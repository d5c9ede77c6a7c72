// Pieces shared by the two decode kernels (per-head VALU kernel and grouped
// MFMA kernel): launch parameters, the new token's pool-format chunks for the
// fused append, and device-coherent accesses to the split-context partials.
#pragma once
#include <cstddef>
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.h"
#include "launch.h"

namespace pa {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeParams {
  const char* kc;  // K pool
  const char* vc;  // V pool
  char* kw;        // the same pools, written by the fused append
  char* vw;
  const void* q;
  void* out;
  const char* k_new;  // [num_seqs][hkv][D] activations, or null (no append)
  const char* v_new;
  const int32_t* tables;
  const int32_t* ctx;
  int* counters;  // [num_seqs][hq] partition arrival counts (zero between calls)
  float* ws_ml;   // [num_seqs][hq][max_parts][2]
  float* ws_o;    // [num_seqs][hq][max_parts][D]
  int num_blocks, log2_bs, hkv, hq, group, max_blocks, max_ctx;
  int max_parts;    // partitions of kPartitionTokens the workspace holds per head (its stride)
  int part_tokens;  // tokens per partition in this launch: a multiple of kPartitionTokens
  int num_seqs;
  int fold_order;   // grouped decode: dispatch sequences in folded length order (see the kernel)
  // scores are kept in log2 units: score_scale = sm_scale * log2(e) (* k_scale
  // for FP8 pools); v_scale multiplies the output (FP8 pools, else 1)
  float score_scale, v_scale, k_inv, v_inv;
  // shared prefixes (DecodeArgs): a sequence of group g starts this launch's
  // tokens at gtok[g] and finds gparts[g] prefix partials in slots 0.. of
  // its workspace rows; gwg[g] = first prefix-pass workgroup of group g
  int ngroups;
  int gstart[kMaxPrefixGroups + 1];
  int gtok[kMaxPrefixGroups];
  int gparts[kMaxPrefixGroups];
  int gwg[kMaxPrefixGroups + 1];
};

// A kernel that reads its DecodeParams fields where it uses them, each read
// behind a branch waiting for its own scalar load, pays a chain of misses
// on a cold scalar cache, one per 64-byte line of the argument block.
// Reading one word of each line it needs at entry, all at once, takes that
// cost once; later field reads hit the cache.  Lines [0, lines) are read,
// and `extra`, a kernel argument past the block (its line is read too).
__device__ __forceinline__ void warm_args(const DecodeParams& P, int lines, int extra) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&P);
  uint32_t x = static_cast<uint32_t>(extra);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(DecodeParams) / 4); i += 16)
    if (i < lines * 16) x ^= w[i];
  asm volatile("" ::"s"(x));
}
// Lines holding every field before the shared-prefix arrays.
constexpr int kArgHeadLines = (offsetof(DecodeParams, gstart) + 63) / 64;
constexpr int kArgAllLines = (static_cast<int>(sizeof(DecodeParams)) + 63) / 64;

// Where sequence s's own tokens begin, and how many prefix partials precede
// its partitions' slots (both 0 outside every shared-prefix group).
struct SeqPrefix {
  int begin, pre;
};
__device__ __forceinline__ SeqPrefix seq_prefix(const DecodeParams& P, int s) {
  for (int g = 0; g < P.ngroups; ++g)
    if (s >= P.gstart[g] && s < P.gstart[g + 1]) return SeqPrefix{P.gtok[g], P.gparts[g]};
  return SeqPrefix{0, 0};
}

// A context length the launch cannot serve (negative, past max_context_len
// or the table, shorter than the sequence's shared prefix, or a new token
// inside that prefix): the sequence's output is NaN.
__device__ __forceinline__ bool seq_bad_len(const DecodeParams& P, int ctx, const SeqPrefix& pf) {
  return ctx < 0 || ctx > P.max_ctx || static_cast<int64_t>(ctx) > static_cast<int64_t>(P.max_blocks) << P.log2_bs ||
         ctx < pf.begin || (P.k_new != nullptr && pf.pre > 0 && ctx - 1 < pf.begin);
}

inline DecodeParams make_decode_params(const DecodeArgs& a) {
  const pa_kv_cache& c = *a.cache;
  DecodeParams P;
  P.kc = static_cast<const char*>(c.k_cache);
  P.vc = static_cast<const char*>(c.v_cache);
  P.kw = static_cast<char*>(c.k_cache);
  P.vw = static_cast<char*>(c.v_cache);
  P.q = a.q;
  P.out = a.out;
  P.k_new = static_cast<const char*>(a.k_new);
  P.v_new = static_cast<const char*>(a.v_new);
  P.tables = a.tables;
  P.ctx = a.ctx;
  P.counters = a.counters;
  P.ws_ml = a.ws_ml;
  P.ws_o = a.ws_o;
  P.num_blocks = c.num_blocks;
  P.log2_bs = __builtin_ctz(c.block_size);
  P.hkv = c.num_kv_heads;
  P.hq = a.num_q_heads;
  P.group = a.num_q_heads / c.num_kv_heads;
  P.max_blocks = a.max_blocks;
  P.max_ctx = a.max_ctx;
  P.max_parts = a.max_parts;
  P.part_tokens = kPartitionTokens;
  P.num_seqs = a.num_seqs;
  P.fold_order = 0;
  P.score_scale = a.sm_scale * kLog2e * (c.kv_dtype == PA_FP8_E4M3 ? c.k_scale : 1.f);
  P.v_scale = c.kv_dtype == PA_FP8_E4M3 ? c.v_scale : 1.f;
  P.k_inv = c.k_inv_scale;
  P.v_inv = c.v_inv_scale;
  P.ngroups = a.ngroups;
  for (int g = 0; g <= kMaxPrefixGroups; ++g) {
    P.gstart[g] = g <= a.ngroups ? a.gstart[g] : 0;
    P.gwg[g] = 0;
  }
  for (int g = 0; g < kMaxPrefixGroups; ++g) {
    P.gtok[g] = g < a.ngroups ? a.gtok[g] : 0;
    P.gparts[g] = g < a.ngroups ? a.gparts[g] : 0;
  }
  return P;
}

// Device-coherent (agent scope) accesses for data exchanged between
// workgroups of one launch, which may run on different XCDs.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16- and 8-byte device-coherent accesses to a window [base, base + bytes)
// of float data through a buffer resource.  The resource sits in scalar
// registers, so `base` must be the same for the whole wave; lanes pass byte
// offsets.  The accesses carry the cache policy of the 4-byte ones above
// (SC1: stores written through to memory, loads served from past this XCD's
// L2).  The hardware range check reads zeros for, and drops stores to,
// offsets at or past `bytes`.
struct CoherentWindow {
  static constexpr int kSc1 = 16;            // cache-policy operand: SC1
  static constexpr int kWord3 = 0x00020000;  // 32-bit data format, untyped access
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ CoherentWindow(const float* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, static_cast<int>(bytes), kWord3)) {}
  __device__ __forceinline__ float4_t load4(uint32_t off) const {
    return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
  }
  __device__ __forceinline__ float load1(uint32_t off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1));
  }
  __device__ __forceinline__ float2_t load2(uint32_t off) const {
    return __builtin_bit_cast(float2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSc1));
  }
  __device__ __forceinline__ void store4(uint32_t off, float4_t v) const {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kSc1);
  }
  __device__ __forceinline__ void store2(uint32_t off, float2_t v) const {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kSc1);
  }
};

// The new token's 16-byte chunk c in pool format (quantised for FP8 pools),
// read from a [head_dim] row of activations.
template <typename KV, typename ACT>
struct NewChunk;
template <typename T>
struct NewChunk<T, T> {
  static __device__ __forceinline__ Vec16 load(const char* row, int c, float) { return load16(row + c * 16); }
};
template <>
struct NewChunk<fp8_t, half_t> {  // 16 numbers = 32 bytes of f16
  static __device__ __forceinline__ Vec16 load(const char* row, int c, float inv) {
    const uint2 a = f16x8_to_e4m3(load16(row + c * 32), inv), b = f16x8_to_e4m3(load16(row + c * 32 + 16), inv);
    return Vec16{{a.x, a.y, b.x, b.y}};
  }
};
template <>
struct NewChunk<fp8_t, float> {  // 16 numbers = 64 bytes of f32
  static __device__ __forceinline__ Vec16 load(const char* row, int c, float inv) {
    Vec16 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = f32x4_chunk_to_e4m3(load16(row + c * 64 + 16 * i), inv);
    return r;
  }
};

}  // namespace pa

namespace pa {

// The merged state of a shared prefix: the prefix pass left `pre` partials
// of workspace row sh in slots 0 .. pre - 1, each (m, l) and an unnormalised
// vector times the V scale, like every partial.  Returns the running max M
// (log2 units), the weight sum L and elements [d0, d0 + N) of the vector,
// rescaled to M and without the V scale (in the pool's units, as a decode
// partition accumulates); the partition starts its online softmax from them.  Coherent loads:
// another launch wrote the partials, possibly from another XCD.
template <int D, int N>
__device__ __forceinline__ void load_prefix_state(const DecodeParams& P, int64_t sh, int pre, int d0, float& M,
                                                  float& L, float* o) {
  const float* ml = P.ws_ml + sh * P.max_parts * 2;
  M = -INFINITY;
  for (int q = 0; q < pre; ++q) M = fmaxf(M, coherent_load(ml + 2 * q));
  const float mu = M == -INFINITY ? 0.f : M;
  L = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] = 0.f;
  for (int q = 0; q < pre; ++q) {
    const float w = exp2f(coherent_load(ml + 2 * q) - mu);
    L += w * coherent_load(ml + 2 * q + 1);
    const float* src = P.ws_o + (sh * P.max_parts + q) * D + d0;
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] += w * coherent_load(src + e);
  }
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] /= P.v_scale;
}

// Floats of LDS scratch merge_partials needs (two arrays of this size); at
// least the largest partition count.
constexpr int kMergeCap = kMaxPartitions;

// The exact merge of split-context partials, run by the last workgroup of a
// (sequence, head group) to finish: heads sh0 .. sh0 + nh - 1 (rows of the
// [num_seqs * hq] workspace), nparts partitions each, in workspace slots
// slot0 .. slot0 + nparts - 1.  Every partition p
// left (m_p, l_p) (running max in log2 units and weight sum) and the
// unnormalised vector o_p; the result is
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p,
// the same rescaling the online softmax does within a partition.  Partials
// are read with device-coherent loads (other workgroups wrote them,
// possibly on another XCD), 8 or 16 bytes at a time; each thread issues
// the loads of up to U output items before it uses any, so one memory
// latency serves them all.  The sum over partitions runs in partition
// order whatever U is.  With at most four partitions the first U items'
// partials are loaded together with the (m, l) pairs, so the merge costs one
// memory latency.  mw, ww: LDS scratch of kMergeCap floats each.  NT
// threads take part; the caller synchronises before the call.
template <typename ACT, int D, int NT, int U = 1>
__device__ __forceinline__ void merge_partials(const DecodeParams& P, int64_t sh0, int nh, int slot0, int nparts,
                                               int tid, float* mw, float* ww) {
  static_assert(U >= 1 && U <= 4, "items in flight per thread");
  ACT* out = static_cast<ACT*>(P.out);
  const int64_t stride = P.max_parts;  // slots per workspace row
  // rows sh0 .. sh0 + nh - 1, slots slot0 .. slot0 + nparts - 1 (at most
  // 80 rows x kMaxPartitions slots x 512 bytes: 32-bit offsets suffice)
  const uint32_t span = static_cast<uint32_t>((nh - 1) * stride + nparts);
  const CoherentWindow wml(P.ws_ml + (sh0 * stride + slot0) * 2, span * 8u);
  const CoherentWindow wo(P.ws_o + (sh0 * stride + slot0) * D, span * (D * 4u));
  const int hb = max(1, min(nh, kMergeCap / nparts));  // heads per batch
  for (int hbase = 0; hbase < nh; hbase += hb) {
    const int nb = min(hb, nh - hbase);
    const int pairs = nb * nparts;
    // four consecutive output elements per item
    const int items = nb * (D / 4);
    auto item_off = [&](int i, int q) -> uint32_t {
      const int hh = i / (D / 4), d = (i - hh * (D / 4)) * 4;
      return static_cast<uint32_t>(((hbase + hh) * stride + q) * D + d) * 4u;
    };
    auto load_items = [&](float4_t (&x)[U][4], int i0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = min(i0 + u * NT, items - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < nparts) x[u][q] = wo.load4(item_off(i, q));
      }
    };
    const bool few = nparts <= 4;
    float4_t x0[U][4];
    if (few) load_items(x0, tid);
    for (int i0 = tid; i0 < pairs; i0 += 2 * NT) {
      float2_t x[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = min(i0 + u * NT, pairs - 1);  // past the end: re-read the last pair
        const int hh = i / nparts, q = i - hh * nparts;
        x[u] = wml.load2(static_cast<uint32_t>((hbase + hh) * stride + q) * 8u);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT;
        if (i < pairs) {
          mw[i] = x[u][0];
          ww[i] = x[u][1];
        }
      }
    }
    __syncthreads();
    for (int hh = tid; hh < nb; hh += NT) {
      float M = -INFINITY;
      for (int q = 0; q < nparts; ++q) M = fmaxf(M, mw[hh * nparts + q]);
      float L = 0.f;
      for (int q = 0; q < nparts; ++q) {
        const float f = exp2f(mw[hh * nparts + q] - M);
        mw[hh * nparts + q] = f;
        L += f * ww[hh * nparts + q];
      }
      const float inv = 1.f / L;
      for (int q = 0; q < nparts; ++q) ww[hh * nparts + q] = mw[hh * nparts + q] * inv;
    }
    __syncthreads();
    auto finish = [&](int i, const float4_t& acc) {
      const int hh = i / (D / 4), d = (i - hh * (D / 4)) * 4;
      const int64_t sh = sh0 + hbase + hh;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[sh * D + d + e] = from_f32<ACT>(acc[e]);
    };
    if (few) {
      auto combine = [&](const float4_t (&x)[U][4], int i0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * NT;
          if (i >= items) continue;
          const float* w = ww + (i / (D / 4)) * nparts;
          float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q < nparts) acc += w[q] * x[u][q];
          finish(i, acc);
        }
      };
      combine(x0, tid);
      for (int i0 = tid + U * NT; i0 < items; i0 += U * NT) {
        float4_t x[U][4];
        load_items(x, i0);
        combine(x, i0);
      }
    } else {
      for (int i = tid; i < items; i += NT) {
        const float* w = ww + (i / (D / 4)) * nparts;
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
        int q = 0;
        for (; q + 4 <= nparts; q += 4) {
          float4_t x[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] = wo.load4(item_off(i, q + u));
#pragma unroll
          for (int u = 0; u < 4; ++u) acc += w[q + u] * x[u];
        }
        for (; q < nparts; ++q) acc += w[q] * wo.load4(item_off(i, q));
        finish(i, acc);
      }
    }
    __syncthreads();
  }
}

}  // namespace pa
