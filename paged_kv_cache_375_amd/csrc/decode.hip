// Paged decode attention: split-context partition kernel + merge kernel.
//
// One workgroup per (partition of kPartitionTokens tokens, query head,
// sequence).  It stages the partition's slice of the block table in LDS,
// then every wavefront streams K/V rows with 16-byte loads: a token's
// head_dim numbers are spread over LPT consecutive lanes (16 bytes each), so
// one wave load covers TPL = 64 / LPT tokens.  The lane's partial q.k is
// summed across its LPT lanes, each lane keeps a running (max, sum, vector)
// online softmax for the tokens of its row [F55 related plate F51: the
// compute-as-you-go softmax gives the same result], and rows, wavefronts and
// finally partitions are merged with the same exact rescaling.  Scores are
// kept in log2 units (scaled by sm_scale * log2(e)) so exp2 is used.
//
// Blocks are fetched through the table in logical token order; physical
// blocks need not be adjacent [F55 §块表]; [IPX §分离逻辑顺序与实际存储位置].
#include <hip/hip_runtime.h>

#include <cmath>

#include "device.h"
#include "launch.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Per-dtype arithmetic on one lane's 16-byte K or V chunk.
template <typename KV, typename ACT>
struct Math;

template <>
struct Math<half_t, half_t> {  // f16 pool, f16 query: packed dot products
  static constexpr int EPL = 8;
  struct Q {
    uint32_t w[4];
  };
  static __device__ __forceinline__ Q load_q(const half_t* q) {
    const Vec16 v = load16(q);
    return Q{{v.w[0], v.w[1], v.w[2], v.w[3]}};
  }
  static __device__ __forceinline__ float dot(const Vec16& k, const Q& q) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, k.w[i]), __builtin_bit_cast(half2_t, q.w[i]), acc,
                                   false);
    return acc;
  }
  static __device__ __forceinline__ void axpy(float* acc, const Vec16& v, float p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += p * half_lo(v.w[i]);
      acc[2 * i + 1] += p * half_hi(v.w[i]);
    }
  }
};

template <>
struct Math<float, float> {  // f32 pool, f32 query
  static constexpr int EPL = 4;
  struct Q {
    float f[4];
  };
  static __device__ __forceinline__ Q load_q(const float* q) {
    const float4 v = *reinterpret_cast<const float4*>(q);
    return Q{{v.x, v.y, v.z, v.w}};
  }
  static __device__ __forceinline__ float dot(const Vec16& k, const Q& q) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += __builtin_bit_cast(float, k.w[i]) * q.f[i];
    return acc;
  }
  static __device__ __forceinline__ void axpy(float* acc, const Vec16& v, float p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += p * __builtin_bit_cast(float, v.w[i]);
  }
};

template <typename ACT>
struct Math<fp8_t, ACT> {  // E4M3 pool: exact hardware conversion to f32
  static constexpr int EPL = 16;
  struct Q {
    float f[16];
  };
  static __device__ __forceinline__ Q load_q(const ACT* q) {
    Q r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r.f[i] = to_f32(q[i]);
    return r;
  }
  static __device__ __forceinline__ float dot(const Vec16& k, const Q& q) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2_t lo = e4m3x2_to_f32(k.w[i], false), hi = e4m3x2_to_f32(k.w[i], true);
      acc += lo[0] * q.f[4 * i] + lo[1] * q.f[4 * i + 1] + hi[0] * q.f[4 * i + 2] + hi[1] * q.f[4 * i + 3];
    }
    return acc;
  }
  static __device__ __forceinline__ void axpy(float* acc, const Vec16& v, float p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2_t lo = e4m3x2_to_f32(v.w[i], false), hi = e4m3x2_to_f32(v.w[i], true);
      acc[4 * i] += p * lo[0];
      acc[4 * i + 1] += p * lo[1];
      acc[4 * i + 2] += p * hi[0];
      acc[4 * i + 3] += p * hi[1];
    }
  }
};

template <typename KV>
struct KVBytes {
  static constexpr int value = Elem<KV>::bytes;
};

// Merge (m, l, acc) with another state: exact rescaling to the larger max.
template <int EPL>
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float mo, float lo, const float* acco) {
  const float mn = fmaxf(m, mo);
  const float mu = (mn == -INFINITY) ? 0.f : mn;
  const float a = exp2f(m - mu), b = exp2f(mo - mu);
  l = l * a + lo * b;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * a + acco[e] * b;
  m = mn;
}

template <typename KV, typename ACT, int D, int NW, int U>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(
    const char* __restrict__ kc, const char* __restrict__ vc, const ACT* __restrict__ q, ACT* __restrict__ out,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ ctx_lens, float* __restrict__ ws_ml,
    float* __restrict__ ws_o, int num_blocks, int log2_bs, int hkv, int hq, int group, int max_blocks, int max_ctx,
    int max_parts, float score_scale, float v_scale) {
  using M = Math<KV, ACT>;
  constexpr int EPL = M::EPL;
  constexpr int LPT = D / EPL;
  constexpr int TPL = 64 / LPT;
  constexpr int PART = kPartitionTokens;
  constexpr int ROUND = NW * TPL;
  static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0, "head_dim does not fit the lane layout");

  const int p = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = lane / LPT, c = lane % LPT;
  const int bs = 1 << log2_bs;
  const int ctx = ctx_lens[s];
  const bool bad_len = ctx < 0 || ctx > max_ctx || static_cast<int64_t>(ctx) > static_cast<int64_t>(max_blocks) * bs;
  const int nparts = bad_len ? 1 : max(1, (ctx + PART - 1) / PART);
  if (p >= nparts) return;
  const int t0 = p * PART;
  const int t1 = bad_len ? t0 : min(t0 + PART, ctx);
  const int b0 = t0 >> log2_bs;
  const int nb = t1 > t0 ? ((t1 - 1) >> log2_bs) - b0 + 1 : 0;

  __shared__ int tab[PART];
  __shared__ int bad_blk;
  __shared__ float red_m[NW], red_l[NW];
  __shared__ float red_o[NW][D];
  if (tid == 0) bad_blk = 0;
  __syncthreads();
  for (int i = tid; i < nb; i += NW * 64) {
    int b = tables[static_cast<int64_t>(s) * max_blocks + b0 + i];
    if (b < 0 || b >= num_blocks) {
      bad_blk = 1;
      b = 0;
    }
    tab[i] = b;
  }
  __syncthreads();
  const int64_t sh = static_cast<int64_t>(s) * hq + h;
  if (bad_len || bad_blk) {
    if (tid < D) {
      if (nparts == 1) {
        out[sh * D + tid] = from_f32<ACT>(NAN);
      } else {
        ws_o[(sh * max_parts + p) * D + tid] = NAN;
        if (tid == 0) ws_ml[(sh * max_parts + p) * 2] = ws_ml[(sh * max_parts + p) * 2 + 1] = NAN;
      }
    }
    return;
  }

  const int g = h / group;
  const typename M::Q qr = M::load_q(q + sh * D + c * EPL);
  float m = -INFINITY, l = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  const int nrounds = (t1 - t0 + ROUND - 1) / ROUND;
  for (int r0 = 0; r0 < nrounds; r0 += U) {
    Vec16 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + (r0 + u) * ROUND + w * TPL + row;
      valid[u] = t < t1;
      const int tt = valid[u] ? t : t0;
      const int64_t blk = tab[(tt >> log2_bs) - b0];
      const int64_t tok_row = (blk * hkv + g) * bs + (tt & (bs - 1));
      const size_t off = static_cast<size_t>(tok_row * D + c * EPL) * KVBytes<KV>::value;
      if (valid[u]) {
        kr[u] = load16(kc + off);
        vr[u] = load16(vc + off);
      } else {
        kr[u] = Vec16{{0, 0, 0, 0}};
        vr[u] = Vec16{{0, 0, 0, 0}};
      }
    }
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d0 = M::dot(kr[u], qr);
#pragma unroll
      for (int o = 1; o < LPT; o <<= 1) d0 += __shfl_xor(d0, o);
      sc[u] = valid[u] ? d0 * score_scale : -INFINITY;
    }
    float mloc = sc[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mloc = fmaxf(mloc, sc[u]);
    const float m_new = fmaxf(m, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = exp2f(sc[u] - m_use);
      l += pu;
      M::axpy(acc, vr[u], pu);
    }
    m = m_new;
  }

  // merge the rows of the wave (lanes that differ in the bits above LPT)
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) {
    float acco[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acco[e] = __shfl_xor(acc[e], o);
    const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
    merge_state<EPL>(m, l, acc, mo, lo, acco);
  }
  if (lane < LPT) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) red_o[w][c * EPL + e] = acc[e];
  }
  if (lane == 0) {
    red_m[w] = m;
    red_l[w] = l;
  }
  __syncthreads();
  for (int i = tid; i < D; i += NW * 64) {
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) mx = fmaxf(mx, red_m[v]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float f = exp2f(red_m[v] - mu);
      o += f * red_o[v][i];
      L += f * red_l[v];
    }
    if (nparts == 1) {
      out[sh * D + i] = from_f32<ACT>(ctx > 0 ? o / L * v_scale : 0.f);
    } else {
      ws_o[(sh * max_parts + p) * D + i] = o * v_scale;
      if (i == 0) {
        ws_ml[(sh * max_parts + p) * 2] = mx;
        ws_ml[(sh * max_parts + p) * 2 + 1] = L;
      }
    }
  }
}

// One workgroup of D threads per (query head, sequence) with > 1 partition.
template <typename ACT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ ws_ml,
                                                         const float* __restrict__ ws_o, ACT* __restrict__ out,
                                                         const int32_t* __restrict__ ctx_lens, int hq, int max_ctx,
                                                         int max_blocks, int log2_bs, int max_parts) {
  constexpr int PART = kPartitionTokens;
  const int h = blockIdx.x, s = blockIdx.y, i = threadIdx.x;
  const int ctx = ctx_lens[s];
  const bool bad_len = ctx < 0 || ctx > max_ctx ||
                       static_cast<int64_t>(ctx) > static_cast<int64_t>(max_blocks) << log2_bs;
  if (bad_len) return;
  const int nparts = (ctx + PART - 1) / PART;
  if (nparts <= 1) return;
  const int64_t sh = static_cast<int64_t>(s) * hq + h;
  const float* ml = ws_ml + sh * max_parts * 2;
  float mx = -INFINITY;
  for (int p = 0; p < nparts; ++p) mx = fmaxf(mx, ml[2 * p]);
  float o = 0.f, L = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float f = exp2f(ml[2 * p] - mx);
    L += f * ml[2 * p + 1];
    o += f * ws_o[(sh * max_parts + p) * D + i];
  }
  out[sh * D + i] = from_f32<ACT>(o / L);
}

template <typename KV, typename ACT, int D>
hipError_t decode_t(const DecodeArgs& a, bool* merge_launched) {
  constexpr int NW = 4, U = 8;
  const pa_kv_cache& c = *a.cache;
  const int log2_bs = __builtin_ctz(c.block_size);
  const int group = a.num_q_heads / c.num_kv_heads;
  const float score_scale = a.sm_scale * kLog2e * (c.kv_dtype == PA_FP8_E4M3 ? c.k_scale : 1.f);
  const float v_scale = c.kv_dtype == PA_FP8_E4M3 ? c.v_scale : 1.f;
  const int parts = (a.max_ctx + kPartitionTokens - 1) / kPartitionTokens;
  const dim3 grid(parts > 0 ? parts : 1, a.num_q_heads, a.num_seqs);
  if (a.ev[0]) (void)hipEventRecord(a.ev[0], a.stream);
  hipLaunchKernelGGL((decode_partition_kernel<KV, ACT, D, NW, U>), grid, dim3(NW * 64), 0, a.stream,
                     static_cast<const char*>(c.k_cache), static_cast<const char*>(c.v_cache),
                     static_cast<const ACT*>(a.q), static_cast<ACT*>(a.out), a.tables, a.ctx, a.ws_ml, a.ws_o,
                     c.num_blocks, log2_bs, c.num_kv_heads, a.num_q_heads, group, a.max_blocks, a.max_ctx,
                     a.max_parts, score_scale, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev[1]) (void)hipEventRecord(a.ev[1], a.stream);
  *merge_launched = false;
  if (parts > 1) {
    if (a.ev[2]) (void)hipEventRecord(a.ev[2], a.stream);
    hipLaunchKernelGGL((decode_merge_kernel<ACT, D>), dim3(a.num_q_heads, a.num_seqs), dim3(D), 0, a.stream,
                       a.ws_ml, a.ws_o, static_cast<ACT*>(a.out), a.ctx, a.num_q_heads, a.max_ctx, a.max_blocks,
                       log2_bs, a.max_parts);
    e = hipGetLastError();
    if (a.ev[3]) (void)hipEventRecord(a.ev[3], a.stream);
    *merge_launched = true;
  }
  return e;
}

template <typename KV, typename ACT>
hipError_t decode_d(const DecodeArgs& a, bool* ml) {
  switch (a.cache->head_dim) {
    case 32: return decode_t<KV, ACT, 32>(a, ml);
    case 64: return decode_t<KV, ACT, 64>(a, ml);
    case 128: return decode_t<KV, ACT, 128>(a, ml);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool* merge_launched) {
  *merge_launched = false;
  if (a.num_seqs == 0 || a.num_q_heads == 0) return hipSuccess;
  const int kv = a.cache->kv_dtype;
  if (kv == PA_F32 && a.act == PA_F32) return decode_d<float, float>(a, merge_launched);
  if (kv == PA_F16 && a.act == PA_F16) return decode_d<half_t, half_t>(a, merge_launched);
  if (kv == PA_FP8_E4M3 && a.act == PA_F16) return decode_d<fp8_t, half_t>(a, merge_launched);
  if (kv == PA_FP8_E4M3 && a.act == PA_F32) return decode_d<fp8_t, float>(a, merge_launched);
  return hipErrorInvalidValue;
}

}  // namespace pa
