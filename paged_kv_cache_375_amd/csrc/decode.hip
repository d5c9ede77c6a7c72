// Paged decode attention: split-context partitions and optionally the
// append of the step's new token in one launch, then an exact merge of the
// partitions' partial results by a small second launch (merge_kernel).
//
// One workgroup per (partition of kPartitionTokens tokens, query head,
// sequence).  Every wavefront streams K/V rows with 16-byte loads: a token's
// head_dim numbers are spread over LPT consecutive lanes (16 bytes each), so
// one wave load covers TPL = 64 / LPT tokens, and the NW waves of the
// workgroup cover ROUND = NW * TPL consecutive tokens per round.  The lane's
// partial q.k is summed across its LPT lanes with DPP row operations, each
// lane keeps a running (max, sum, vector) online softmax for the tokens of
// its row [F55 related plate F51: the compute-as-you-go softmax gives the
// same result], and rows, wavefronts and finally partitions are merged with
// the same exact rescaling.  Scores are kept in log2 units (scaled by
// sm_scale * log2(e)) so exp2 is used.
//
// Blocks are fetched through the table in logical token order; physical
// blocks need not be adjacent [F55 §块表]; [IPX §分离逻辑顺序与实际存储位置].
// When a block holds at least TPL tokens, the TPL tokens of one wave load
// always lie in one block, so the block id is wave-uniform: the partition's
// table slice is loaded once into registers (one entry per lane) and read
// with readlane; smaller blocks stage the slice in LDS and look it up per
// lane.  Loads are never
// predicated: lanes past the context re-read the last token (a cache hit)
// and their scores are masked to -inf.
#include <hip/hip_runtime.h>

#include <cmath>

#include "decode_common.h"
#include "decode_group.h"

namespace pa {
namespace {

// Launch shape: wavefronts per workgroup (measured best: eight for f16 and
// f32 pools, two for FP8 pools, whose lanes do more arithmetic per byte) and
// wave loads per batch.
#ifndef PA_DECODE_WAVES_F16
#define PA_DECODE_WAVES_F16 8
#endif
template <typename KV>
constexpr int decode_waves() {
  return Elem<KV>::bytes == 1 ? 2 : PA_DECODE_WAVES_F16;
}
#ifndef PA_DECODE_UNROLL
#define PA_DECODE_UNROLL 8
#endif
// Grid order: 1 = query head varies fastest (the K/V tiles of neighbouring
// heads of one block are adjacent in the pool), 0 = partition fastest.
#ifndef PA_GRID_HEAD_FIRST
#define PA_GRID_HEAD_FIRST 1
#endif

// ---- cross-lane sums -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over aligned groups of N lanes; every lane of a group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<kQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kRowMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

// ---- per-dtype arithmetic on one lane's 16-byte K or V chunk ---------------

template <typename KV, typename ACT>
struct Math;

template <>
struct Math<half_t, half_t> {  // f16 pool, f16 query: packed dot products
  static constexpr int EPL = 8;
  static constexpr bool PAIRED = false;
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
  static constexpr bool PAIRED = false;
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

template <>
struct Math<fp8_t, half_t> {  // E4M3 pool, f16 query: K converted to f16 pairs (exact) for packed dots,
                               // V accumulated two tokens at a time with f16 weights
  static constexpr int EPL = 16;
  static constexpr bool PAIRED = true;
  struct Q {
    uint32_t w[8];  // the 16 query values as f16 pairs
  };
  static __device__ __forceinline__ Q load_q(const half_t* q) {
    const Vec16 a = load16(q), b = load16(q + 8);
    return Q{{a.w[0], a.w[1], a.w[2], a.w[3], b.w[0], b.w[1], b.w[2], b.w[3]}};
  }
  static __device__ __forceinline__ float dot(const Vec16& k, const Q& q) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // bytes 0, 1 and 2, 3 of the word: elements 4i, 4i + 1 and 4i + 2, 4i + 3
      const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.w[i], 1.0f, false);
      const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k.w[i], 1.0f, true);
      acc = __builtin_amdgcn_fdot2(lo, __builtin_bit_cast(half2_t, q.w[2 * i]), acc, false);
      acc = __builtin_amdgcn_fdot2(hi, __builtin_bit_cast(half2_t, q.w[2 * i + 1]), acc, false);
    }
    return acc;
  }
  // acc[e] += p.x a[e] + p.y b[e] over the lane's 16 elements of two tokens'
  // V rows a and b, the weights an f16 pair: each word's bytes of the two
  // rows are interleaved (v_perm_b32: a0 b0 a1 b1, a2 b2 a3 b3), converted
  // to f16 pairs (exact) and dotted with the weights (exact products, f32
  // accumulation): 2.5 instructions per element pair instead of 3 for a
  // conversion to f32 and two multiply-adds.  On FP8 pools the kernel does
  // about twice the vector work per byte of f16 (a wave had a VALU
  // instruction active in 27% of its cycles, at two waves per SIMD), so
  // this shows: FP8 prefix layer 98.5 -> 97.8 us, OPT-13B shape with an FP8
  // pool 66.2 -> 65.7 us.
  static __device__ __forceinline__ void axpy2(float* acc, const Vec16& a, const Vec16& b, half2_t p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x01 = __builtin_amdgcn_perm(b.w[i], a.w[i], 0x05010400u);
      const uint32_t x23 = __builtin_amdgcn_perm(b.w[i], a.w[i], 0x07030602u);
      acc[4 * i] = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x01, 1.0f, false), p, acc[4 * i], false);
      acc[4 * i + 1] =
          __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x01, 1.0f, true), p, acc[4 * i + 1], false);
      acc[4 * i + 2] =
          __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x23, 1.0f, false), p, acc[4 * i + 2], false);
      acc[4 * i + 3] =
          __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x23, 1.0f, true), p, acc[4 * i + 3], false);
    }
  }
};

template <>
struct Math<fp8_t, float> {  // E4M3 pool, f32 query: exact hardware conversion to f32
  static constexpr int EPL = 16;
  static constexpr bool PAIRED = false;
  struct Q {
    float f[16];
  };
  static __device__ __forceinline__ Q load_q(const float* q) {
    Q r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r.f[i] = q[i];
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

// BIG: block_size >= TPL (block id wave-uniform, table slice in registers).
// A head whose tokens span several partitions, or whose sequence follows a
// shared prefix (whose pass left partials in slots 0 .. pre - 1), leaves a
// partial per partition in slot pre + p for merge_kernel; a head with a
// single partial writes its output.
// LOADS_ONLY (measurement, pa_read_probe): the same grid, table staging and
// K/V loads, with the arithmetic replaced by an XOR of the loaded words into
// P.out (a uint32 sink of kProbeSinkWords words); nothing else is written.
template <typename KV, typename ACT, int D, int NW, int U, bool BIG, bool LOADS_ONLY = false>
__device__ __forceinline__ void decode_heads_body(const DecodeParams& P, const int h, const int p, const int s) {
  using M = Math<KV, ACT>;
  constexpr int EPL = M::EPL;
  constexpr int LPT = D / EPL;
  constexpr int TPL = 64 / LPT;
  constexpr int PART = kPartitionTokens;
  constexpr int ROUND = NW * TPL;
  constexpr int KVB = Elem<KV>::bytes;
  static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0, "head_dim does not fit the lane layout");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane / LPT, c = lane % LPT;
  const int log2_bs = P.log2_bs;
  const int bs = 1 << log2_bs;
  const int ctx = P.ctx[s];
  // A shared prefix's tokens [0, begin) were covered by the prefix pass, which
  // left `pre` partials; the new token may not lie in them.
  const SeqPrefix pf = seq_prefix(P, s);
  const bool bad_len = seq_bad_len(P, ctx, pf);
  // this launch's partitions; partition 0 starts from the prefix's merged
  // state, so these are all the partials to merge
  const int nparts = bad_len ? 1 : max(1, (ctx - pf.begin + PART - 1) / PART);
  if (p >= nparts) return;
  const int t0 = (bad_len ? 0 : pf.begin) + p * PART;
  const int t1 = bad_len ? t0 : min(t0 + PART, ctx);
  const int b0 = t0 >> log2_bs;
  const int64_t trow = static_cast<int64_t>(s) * P.max_blocks;
  const int g = h / P.group;
  const int64_t sh = static_cast<int64_t>(s) * P.hq + h;
  const int64_t head_rows = static_cast<int64_t>(g) * bs;      // token rows before head g in a block
  const int64_t block_rows = static_cast<int64_t>(P.hkv) * bs;  // token rows per block

  // q is loaded first, so its latency overlaps the table slice's
  typename M::Q qr{};
  if constexpr (!LOADS_ONLY) qr = M::load_q(static_cast<const ACT*>(P.q) + sh * D + c * EPL);

  __shared__ int tab[BIG ? 1 : PART];
  __shared__ float red_m[NW], red_l[NW];
  __shared__ float red_o[NW][D];
  int my_bad = bad_len ? 1 : 0;
  // BIG: the partition's table slice lives in registers, entry i in lane
  // i % 64 of tabreg[i / 64]; a wave-uniform index is read with readlane.
  constexpr int NTR = (PART / TPL + 63) / 64;
  int tabreg[NTR];
  {
    const int nb = t1 > t0 ? ((t1 - 1) >> log2_bs) - b0 + 1 : 0;
    if constexpr (BIG) {
#pragma unroll
      for (int j = 0; j < NTR; ++j) {
        const int i = lane + 64 * j;
        int b = 0;
        if (i < nb) {
          b = P.tables[trow + b0 + i];
          if (b < 0 || b >= P.num_blocks) {
            my_bad = 1;
            b = 0;
          }
        }
        tabreg[j] = b;
      }
    } else {
      for (int i = tid; i < nb; i += NW * 64) {
        int b = P.tables[trow + b0 + i];
        if (b < 0 || b >= P.num_blocks) {
          my_bad = 1;
          b = 0;
        }
        tab[i] = b;
      }
    }
  }

  // Fused append: the partition holding the new token (position ctx - 1)
  // takes its K/V from the caller's rows, not from the pool, and the kv
  // head's first query head stores them into the pool slot.  Nothing in this
  // launch reads that slot from the pool.
  const bool has_new = !LOADS_ONLY && P.k_new != nullptr && p == nparts - 1 && !bad_len && ctx >= 1;
  Vec16 knew{{0, 0, 0, 0}}, vnew{{0, 0, 0, 0}};
  if (has_new) {
    const int64_t src = (static_cast<int64_t>(s) * P.hkv + g) * D * static_cast<int64_t>(sizeof(ACT));
    knew = NewChunk<KV, ACT>::load(P.k_new + src, c, P.k_inv);
    vnew = NewChunk<KV, ACT>::load(P.v_new + src, c, P.v_inv);
    if (h % P.group == 0 && w == 0 && row == 0) {
      const int pos = ctx - 1;
      const int b = P.tables[trow + (pos >> log2_bs)];
      if (b >= 0 && b < P.num_blocks) {
        const int64_t tok_row = static_cast<int64_t>(b) * block_rows + head_rows + (pos & (bs - 1));
        const size_t off = static_cast<size_t>(tok_row * D + c * EPL) * KVB;
        store16(P.kw + off, knew);
        store16(P.vw + off, vnew);
      }
    }
  }
  const bool bad_early = __syncthreads_or(my_bad) != 0;
  float m = -INFINITY, l = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  const int nrounds = bad_early ? 0 : (t1 - t0 + ROUND - 1) / ROUND;
  uint32_t fold = 0;  // LOADS_ONLY
  for (int r0 = 0; r0 < nrounds; r0 += U) {
    Vec16 kr[U], vr[U];
    int tok[U];
    int64_t blk[U];
    // block ids of the U wave loads first ...
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tb = t0 + (r0 + u) * ROUND + w * TPL;  // first token of this wave load
      tok[u] = tb + row;
      if constexpr (BIG) {
        const int idx = (min(tb, t1 - 1) >> log2_bs) - b0;
        blk[u] = __builtin_amdgcn_readlane(tabreg[idx >> 6], idx & 63);
      } else {
        blk[u] = tab[(min(tok[u], t1 - 1) >> log2_bs) - b0];
      }
    }
    // ... then every K and V load of the batch, before any arithmetic
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(tok[u], t1 - 1);
      const int64_t tok_row = blk[u] * block_rows + head_rows + (t & (bs - 1));
      const size_t off = static_cast<size_t>(tok_row * D + c * EPL) * KVB;
      kr[u] = load16_stream(P.kc + off);
      vr[u] = load16_stream(P.vc + off);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LOADS_ONLY) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        fold ^= kr[u].w[0] ^ kr[u].w[1] ^ kr[u].w[2] ^ kr[u].w[3] ^ vr[u].w[0] ^ vr[u].w[1] ^ vr[u].w[2] ^ vr[u].w[3];
      continue;
    }
    if (has_new && r0 + U >= nrounds) {  // the batch that holds the new token
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // lanes past the context re-read the last token: they take the new
        // token too (their weight is zero, but a stale slot could hold NaN)
        if (min(tok[u], t1 - 1) == ctx - 1) {
          kr[u] = knew;
          vr[u] = vnew;
        }
      }
    }
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float d0 = group_sum<LPT>(M::dot(kr[u], qr));
      sc[u] = tok[u] < t1 ? d0 * P.score_scale : -INFINITY;
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
    if constexpr (M::PAIRED) {
      // the weights of tokens u and u + 1 as an f16 pair; the sum takes the
      // same rounded weights (a dot product with ones)
      static_assert(U % 2 == 0, "tokens in pairs");
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        const half2_t p = __builtin_convertvector(float2_t{exp2f(sc[u] - m_use), exp2f(sc[u + 1] - m_use)}, half2_t);
        l = __builtin_amdgcn_fdot2(p, half2_t{1, 1}, l, false);
        M::axpy2(acc, vr[u], vr[u + 1], p);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pu = exp2f(sc[u] - m_use);
        l += pu;
        M::axpy(acc, vr[u], pu);
      }
    }
    m = m_new;
  }

  if constexpr (LOADS_ONLY) {
    // the loads cannot be dropped: the store depends on their values (and
    // almost never happens, so the sink adds no traffic)
    if (fold == kProbeMagic)
      static_cast<uint32_t*>(P.out)[(h + 37 * p + 101 * s + tid) & (kProbeSinkWords - 1)] = fold;
    return;
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
  ACT* out = static_cast<ACT*>(P.out);
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
    if (bad_early) o = L = mx = NAN;
    // The output itself when this is the head's only partial, else a
    // partial for merge_kernel.  Plain stores: the merge runs in the next
    // launch, after this one's writes are visible device-wide.  Leaving the
    // merge to a second launch frees each workgroup as soon as its partial
    // is stored; merging in this launch (the last partition to finish, found
    // with an arrival counter) held every split workgroup for the stores'
    // completion and a counter round trip (OPT-13B layer 120.8 -> 117.2 us).
    if (bad_len || pf.pre + nparts == 1) {
      out[sh * D + i] = from_f32<ACT>(bad_early ? NAN : (ctx > 0 ? o / L * P.v_scale : 0.f));
    } else {
      const int slot = pf.pre + p;
      P.ws_o[(sh * P.max_parts + slot) * D + i] = o * P.v_scale;
      if (i == 0) {
        P.ws_ml[(sh * P.max_parts + slot) * 2] = mx;
        P.ws_ml[(sh * P.max_parts + slot) * 2 + 1] = L;
      }
    }
  }
}

template <typename KV, typename ACT, int D, int NW, int U, bool BIG, bool LOADS_ONLY = false>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeParams P) {
  decode_heads_body<KV, ACT, D, NW, U, BIG, LOADS_ONLY>(P, PA_GRID_HEAD_FIRST ? blockIdx.x : blockIdx.y,
                                                        PA_GRID_HEAD_FIRST ? blockIdx.y : blockIdx.x, blockIdx.z);
}

// A shared-prefix decode over an FP8 pool in one launch, followed by the
// merge launch.  The workgroups run the per-head decode (head fastest, then
// partition, then sequence, as decode_kernel), then, in the last prefix_wgs
// of the grid, the prefix pass (the grouped kernel's body, one head tile of
// 16 rows per workgroup, two waves, in the order described below).
// Neither reads what the other writes: the prefix pass reads the groups'
// shared blocks and q and writes workspace slots [0, pre); the decode reads
// each sequence's own blocks past its shared tokens, writes slots from pre
// on (never the output: with a prefix every head leaves partials) and
// stores the new token, which never falls in a shared block (a sequence
// whose new token would is refused, and copy on write keeps a shared block
// from being written).  Only the merge launch reads both.  The prefix pass
// is a chain of dependent round trips over few bytes; dispatched last, its
// workgroups take the slots that the decode's final round leaves idle as it
// drains (FP8 prefix layer of 64 sequences: 99.4 us per step, against 103.2
// with the prefix workgroups first in the grid and 106.1 with the prefix
// pass as a launch of its own before the decode).  Both roles fit the
// two-wave workgroup, and the prefix role's LDS leaves six workgroups per
// CU, at which the FP8 decode runs no slower than at its own eight.  Six
// need three waves per SIMD, which the register budget is held to: left
// free, the compiler gives the head_dim-128 instance 156 VGPRs and 40
// accumulation registers, two waves per SIMD (FP8 prefix layer 98.1
// against 98.5 us of launches, three runs each).
template <int D>
__global__ __launch_bounds__(2 * 64) __attribute__((amdgpu_waves_per_eu(3))) void decode_prefix_fused_kernel(
    const DecodeParams P, int prefix_cols, int prefix_wgs, int np) {
  static_assert(decode_waves<fp8_t>() == 2, "both roles use two-wave workgroups");
  const int i = blockIdx.x;
  const int ndec = static_cast<int>(gridDim.x) - prefix_wgs;
  if (i >= ndec) {
    // Each group's prefix workgroups, ordered in blocks of 8 (KV head,
    // partition) units x R row sets, so that the R row sets of one unit,
    // which read the same shared K/V, run 8 workgroups apart: consecutive
    // workgroups go to different XCDs, so these share one XCD's L2 (FP8
    // prefix layer: 13 MB less read from HBM per launch, 98.4 against
    // 99.9 us).  The map is a bijection onto (row-set column, partition).
    const int b = i - ndec;
    const int maxp = prefix_wgs / prefix_cols;
    int gi = 0;
    while (gi + 1 < P.ngroups && b >= P.gwg[gi + 1] * maxp) ++gi;  // the group's workgroups are contiguous
    const int R = (P.gwg[gi + 1] - P.gwg[gi]) / P.hkv;               // row sets per KV head (> 0 here)
    const int j = b - P.gwg[gi] * maxp, units = P.hkv * maxp;
    const int blk = j / (8 * R), in_blk = j - blk * 8 * R;
    const int width = min(8, units - blk * 8);  // units in this block (fewer in the last)
    const int unit = blk * 8 + in_blk % width, rs = in_blk / width;
    decode_group_body<fp8_t, D, 1, 2, true, true>(P, 1, P.gwg[gi] + (unit % P.hkv) * R + rs, unit / P.hkv, 0);
    return;
  }
  const int h = i % P.hq, r = i / P.hq;
  decode_heads_body<fp8_t, half_t, D, 2, PA_DECODE_UNROLL, true>(P, h, r % np, r / np);
}

// The merge after a decode launch: one wave per (q head, sequence) merges
// the head's partials, a shared prefix's included, exactly:
//   out = sum_q 2^(m_q - M) o_q / sum_q 2^(m_q - M) l_q,  M = max_q m_q
// (the online softmax's rescaling).  Heads with a single partial were
// written by the decode.  Lane q holds partial q's (m, l) (lanes stride
// over longer lists).  The (m, l) of the first 64 slots and the vectors of
// the first QB are loaded together with the context length, before the
// number of partials is known (every slot of the head's workspace row
// exists; slots past the partials are read and ignored), so a head with few
// partials costs one memory round trip.  Lane i takes elements
// E i .. E i + E - 1.
template <typename ACT, int D>
__global__ __launch_bounds__(64) void merge_kernel(const DecodeParams P) {
  constexpr int E = D >= 64 ? D / 64 : 1;  // elements per lane (head_dim 32: lanes 32..63 idle)
  constexpr int QB = 8;                    // partials per batch of vector loads
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int64_t sh = static_cast<int64_t>(s) * P.hq + h;
  // the head's workspace row (written by earlier launches; coherent loads
  // all the same)
  const int slots = P.max_parts;
  const CoherentWindow wml(P.ws_ml + sh * slots * 2, static_cast<uint32_t>(slots) * 8u);
  const CoherentWindow wo(P.ws_o + sh * slots * D, static_cast<uint32_t>(slots) * (D * 4u));
  const bool active = lane * E < D;
  auto load_o = [&](int q, float (&x)[E]) {
    const uint32_t off = static_cast<uint32_t>(q * D + lane * E) * 4u;
    if constexpr (E == 2) {
      const float2_t v = wo.load2(off);
      x[0] = v[0];
      x[1] = v[1];
    } else {
      x[0] = wo.load1(off);
    }
  };
  float x[QB][E];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    if (qb < slots && active) load_o(qb, x[qb]);
  float2_t mlq = {-INFINITY, 0.f};
  if (lane < slots) mlq = wml.load2(static_cast<uint32_t>(lane) * 8u);
  const int ctx = P.ctx[s];
  const SeqPrefix pf = seq_prefix(P, s);
  const bool bad_len = seq_bad_len(P, ctx, pf);
  const int nparts = bad_len ? 1 : max(1, (ctx - pf.begin + kPartitionTokens - 1) / kPartitionTokens);
  const int total = pf.pre + nparts;
  if (bad_len || total == 1) return;
  if (lane >= total) mlq = float2_t{-INFINITY, 0.f};
  float M = mlq[0];
  for (int q = lane + 64; q < total; q += 64) M = fmaxf(M, wml.load1(static_cast<uint32_t>(q) * 8u));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float wq = lane < total ? exp2f(mlq[0] - M) : 0.f;  // partial `lane`'s weight
  float L = wq * mlq[1];
  for (int q = lane + 64; q < total; q += 64) {
    const float2_t v = wml.load2(static_cast<uint32_t>(q) * 8u);
    L += exp2f(v[0] - M) * v[1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int q0 = 0; q0 < total; q0 += QB) {
    if (q0 > 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        if (q0 + qb < total && active) load_o(q0 + qb, x[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int q = q0 + qb;
      if (q >= total) break;
      const float w = q < 64 ? __shfl(wq, q) : exp2f(wml.load1(static_cast<uint32_t>(q) * 8u) - M);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * x[qb][e];
    }
  }
  if (active) {
    ACT* out = static_cast<ACT*>(P.out);
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < E; ++e) out[sh * D + lane * E + e] = from_f32<ACT>(acc[e] * inv);
  }
}

template <typename KV, typename ACT, int D>
hipError_t decode_t(const DecodeArgs& a) {
  constexpr int NW = decode_waves<KV>(), U = PA_DECODE_UNROLL;
  constexpr int TPL = 64 / (D / Math<KV, ACT>::EPL);
  const pa_kv_cache& c = *a.cache;
  const DecodeParams P = make_decode_params(a);
  const unsigned np = static_cast<unsigned>(decode_grid_parts(a, kPartitionTokens));
  const dim3 grid(PA_GRID_HEAD_FIRST ? a.num_q_heads : np, PA_GRID_HEAD_FIRST ? np : a.num_q_heads, a.num_seqs);
  auto kern = c.block_size >= TPL ? decode_kernel<KV, ACT, D, NW, U, true> : decode_kernel<KV, ACT, D, NW, U, false>;
  if (a.ev[0]) (void)hipEventRecord(a.ev[0], a.stream);
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), 0, a.stream, P);
  hipError_t e = hipGetLastError();
  // partials exist only where a head has more than one
  if (e == hipSuccess && (np > 1 || a.ngroups > 0)) {
    hipLaunchKernelGGL((merge_kernel<ACT, D>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0, a.stream, P);
    e = hipGetLastError();
  }
  if (a.ev[1]) (void)hipEventRecord(a.ev[1], a.stream);
  return e;
}

// Workgroups of the fused shared-prefix launch: heads x partitions x
// sequences of the decode, then prefix row sets x prefix partitions.
struct FusedGrid {
  int prefix_cols, prefix_wgs, np;
  int64_t total;
};
inline FusedGrid fused_grid(const DecodeArgs& a, DecodeParams& P) {
  FusedGrid f;
  int parts = 0;
  f.prefix_cols = prefix_grid(a, 1, P, &parts);
  f.prefix_wgs = f.prefix_cols * parts;
  f.np = decode_grid_parts(a, kPartitionTokens);
  f.total = f.prefix_wgs + static_cast<int64_t>(a.num_q_heads) * f.np * a.num_seqs;
  return f;
}

template <int D>
hipError_t decode_prefix_fused_t(const DecodeArgs& a) {
  DecodeParams P = make_decode_params(a);
  const FusedGrid f = fused_grid(a, P);
  if (a.ev[0]) (void)hipEventRecord(a.ev[0], a.stream);
  hipLaunchKernelGGL(decode_prefix_fused_kernel<D>, dim3(static_cast<unsigned>(f.total)), dim3(2 * 64), 0, a.stream,
                     P, f.prefix_cols > 0 ? f.prefix_cols : 1, f.prefix_wgs, f.np);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL((merge_kernel<half_t, D>), dim3(a.num_q_heads, a.num_seqs), dim3(64), 0, a.stream, P);
    e = hipGetLastError();
  }
  if (a.ev[1]) (void)hipEventRecord(a.ev[1], a.stream);
  return e;
}

// The per-head kernel's loads alone over a pool of element size KVB bytes
// (pa_read_probe, paged mode): every KV head decoded as if it had one query
// head, with f16 or f32 arithmetic types standing for the row length only.
template <typename KV, typename ACT, int D>
hipError_t probe_t(const DecodeArgs& a, uint32_t* sink) {
  constexpr int NW = decode_waves<KV>(), U = PA_DECODE_UNROLL;
  constexpr int TPL = 64 / (D / Math<KV, ACT>::EPL);
  DecodeParams P = make_decode_params(a);
  P.out = sink;
  P.k_new = P.v_new = nullptr;
  const unsigned np = static_cast<unsigned>(decode_grid_parts(a, kPartitionTokens));
  const dim3 grid(PA_GRID_HEAD_FIRST ? a.num_q_heads : np, PA_GRID_HEAD_FIRST ? np : a.num_q_heads, a.num_seqs);
  auto kern = a.cache->block_size >= TPL ? decode_kernel<KV, ACT, D, NW, U, true, true>
                                         : decode_kernel<KV, ACT, D, NW, U, false, true>;
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), 0, a.stream, P);
  return hipGetLastError();
}

template <typename KV, typename ACT>
hipError_t probe_d(const DecodeArgs& a, uint32_t* sink) {
  switch (a.cache->head_dim) {
    case 32: return probe_t<KV, ACT, 32>(a, sink);
    case 64: return probe_t<KV, ACT, 64>(a, sink);
    case 128: return probe_t<KV, ACT, 128>(a, sink);
  }
  return hipErrorInvalidValue;
}

template <typename KV, typename ACT>
hipError_t decode_d(const DecodeArgs& a) {
  switch (a.cache->head_dim) {
    case 32: return decode_t<KV, ACT, 32>(a);
    case 64: return decode_t<KV, ACT, 64>(a);
    case 128: return decode_t<KV, ACT, 128>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_loads(const DecodeArgs& a, uint32_t* sink) {
  if (a.num_seqs == 0 || a.num_q_heads == 0) return hipSuccess;
  const int kv = a.cache->kv_dtype;
  if (kv == PA_F32) return probe_d<float, float>(a, sink);
  if (kv == PA_F16) return probe_d<half_t, half_t>(a, sink);
  if (kv == PA_FP8_E4M3) return probe_d<fp8_t, half_t>(a, sink);
  return hipErrorInvalidValue;
}

bool prefix_fused_applies(const DecodeArgs& a) {
  const pa_kv_cache& c = *a.cache;
  if (a.ngroups == 0 || a.num_seqs == 0 || a.num_q_heads == 0 || group_decode_applies(a) || a.act != PA_F16 ||
      c.kv_dtype != PA_FP8_E4M3 || (c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128))
    return false;
  // the decode role's wave-uniform block ids (a wave load's tokens in one
  // block) and the prefix role's wave-uniform tile bases
  const int tokens_per_load = 64 / (c.head_dim / Math<fp8_t, half_t>::EPL);
  if (c.block_size < tokens_per_load || !tile_addressing(c)) return false;
  DecodeParams P = make_decode_params(a);
  return fused_grid(a, P).total * 2 * 64 <= static_cast<int64_t>(UINT32_MAX);  // work-items of a 1-D grid
}

hipError_t launch_decode_prefix_fused(const DecodeArgs& a) {
  switch (a.cache->head_dim) {
    case 32: return decode_prefix_fused_t<32>(a);
    case 64: return decode_prefix_fused_t<64>(a);
    case 128: return decode_prefix_fused_t<128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.num_seqs == 0 || a.num_q_heads == 0) return hipSuccess;
  if (group_decode_applies(a)) return launch_decode_group(a);
  const int kv = a.cache->kv_dtype;
  if (kv == PA_F32 && a.act == PA_F32) return decode_d<float, float>(a);
  if (kv == PA_F16 && a.act == PA_F16) return decode_d<half_t, half_t>(a);
  if (kv == PA_FP8_E4M3 && a.act == PA_F16) return decode_d<fp8_t, half_t>(a);
  if (kv == PA_FP8_E4M3 && a.act == PA_F32) return decode_d<fp8_t, float>(a);
  return hipErrorInvalidValue;
}

}  // namespace pa
