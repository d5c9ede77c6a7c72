// Paged decode attention for grouped- and multi-query attention, where the
// query heads of a group share one KV head [F55 §后来的做法]: the group's
// scores and weighted sums are small dense products, done on the matrix
// cores (v_mfma_f32_16x16x32_f16, f32 accumulation).
//
// One workgroup per (KV head and group of up to 16 * HT query heads,
// partition, sequence).  The partition length is chosen per launch (a
// multiple of kPartitionTokens): the shortest whose workgroups all fit on the
// GPU at once, else kPartitionTokens.  Its NW wavefronts (4, or 8 at three
// or more head tiles) take 32-token chunks of the partition in turn; a chunk
// is processed as
//
//   S^T[32 tokens][16 heads] = K[32][D] . Q^T[D][16]      (2 x D/32 MFMAs per head tile)
//   online softmax of each head's column (scores in log2 units, exp2)
//   O^T[D][16 heads] += V^T[D][32] . P^T[32][16]          (D/16 MFMAs per head tile)
//
// Computing S transposed puts the weights P^T straight into the B-operand
// layout of the second product: the lane that holds head n's scores for
// tokens {4g..4g+3, 16+4g..16+4g+3} (g = lane / 16) is the lane that feeds
// those tokens into the contraction, so P never moves between lanes.
//
// The operand layouts put each of 16 consecutive lanes on a different token,
// which the vector memory path cannot combine, so K and V rows are instead
// loaded with fully coalesced 16-byte loads (a wave load reads whole rows),
// converted to f16 if the pool is FP8, and written to the wave's slice of
// LDS with their 16-byte chunks XOR-swizzled by row.  K is read back as
// operand rows (ds_read_b128; the head_dim order of the first contraction is
// free as long as Q uses the same); V, which the second product needs as
// columns, is read back with gfx950's transposing LDS read
// (ds_read_b64_tr_b16: lane i of each 16-lane group receives element i of
// the four 8-byte rows addressed by lanes 4k..4k+3, k = 0..3), two reads per
// 16-column tile.  The loop is software-pipelined: the next chunk's K and V
// loads are issued as soon as the current ones are in LDS.
//
// Heads past the group (padding up to 16 per tile) have q = 0 and are never
// written.  The NW wavefronts' partial results are merged per head tile in a
// fixed order through LDS, and partitions by the last workgroup to finish,
// with the rescaling of the per-head kernel's merge launch (same workspace
// layout), so results are deterministic.
// Blocks are fetched through the table in logical order and need not be
// adjacent [F55 §块表]; [IPX §分离逻辑顺序与实际存储位置].
//
// The kernel body is a device function of the workgroup's grid coordinates,
// so that a launch can also run it beside other work (the prefix pass of a
// shared-prefix decode inside the per-head decode launch).
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {
namespace {

// Minimum waves per SIMD the register allocation must allow: three where
// the head tiles fit without spilling, else two.
template <int D, int HT>
constexpr int group_occupancy() {
  return D >= 128 || (D == 64 && HT >= 3) ? 2 : 3;
}

// Waves per workgroup of the prefix pass: eight with three or more head
// tiles (a wave's state is then large, about 240 VGPRs at five tiles, and
// eight waves fill a CU), else four.  The decode launch chooses per launch
// (launch_ht).
template <int HT>
constexpr int group_waves() {
  return HT >= 3 ? 8 : 4;
}

constexpr int kLdsPerCu = 160 * 1024;  // gfx950

// LDS arena of the grouped kernel (16-byte words): the fold order's lengths,
// then the main loop's K/V chunks, q rows and table slice, later the waves'
// merge exchange, sized to the LDS that each of the workgroups one CU holds
// at the kernel's occupancy may use.
template <int D, int HT, int NW>
struct GroupArena {
  static constexpr int LCH = D / 8, NDT = D / 16;
  static constexpr int kVbuf = NW * kChunk * LCH > kMergeCap / 2 ? NW * kChunk * LCH : kMergeCap / 2;
  static constexpr int kQs = HT * 16 * LCH;
  static constexpr int kLoop = kVbuf + kQs + kTabEntries / 4;
  static_assert(kVbuf * 4 >= kFoldMaxSeqs, "the fold order's lengths fit the K/V staging");
  static constexpr int exchange(int xr) { return xr * (NW - 1) * NDT * 64 + (xr * (NW - 1) * 64 + 1) / 2; }
  static constexpr int words(int xr) { return kLoop > exchange(xr) ? kLoop : exchange(xr); }
  // LDS per workgroup when the CU holds as many as the register occupancy
  // allows, less what the kernel keeps beside the arena (new token rows,
  // flags) and some slack
  static constexpr int kBudget = kLdsPerCu / (group_occupancy<D, HT>() * 4 / NW) - 2 * D * 2 - 512;
  static constexpr int pick(int xr) { return xr <= 1 || words(xr) * 16 <= kBudget ? xr : pick(xr - 1); }
  static constexpr int XR = pick(HT);
  static constexpr int kXo = XR * (NW - 1) * NDT * 64;
  static constexpr int kWords = words(XR);
};

// PREFIX = false: decode, one workgroup per (KV head and group of query
// heads, partition, sequence), as described above.
// PREFIX = true: the prefix pass of a shared-prefix decode.  The query rows
// of a workgroup are (sequence, query head) pairs of one group of sequences
// that share their first gtok tokens (whole blocks) and one KV head, up to
// 16 * HT of them; the shared blocks, read through the table of the group's
// first sequence, are loaded once for all of those rows.  Each partition of
// kPrefixPartTokens tokens leaves (m, l, o) partials in workspace slot p of
// every row (o times the V scale, like every partial).  The grouped decode
// launch that follows starts the online softmax of each head's first
// partition from their merged state; after the per-head decode, its merge
// launch takes them with the decode's own partials.
template <typename KV, int D, int HT, int NW, bool UNI, bool PREFIX>
__device__ __forceinline__ void decode_group_body(const DecodeParams& P, const int groups_per_kv, const int bx,
                                                  const int by, const int bz) {
  warm_args(P, PREFIX ? kArgAllLines : kArgHeadLines, groups_per_kv);
  using L = Layout<KV, D>;
  constexpr int KVB = L::KVB, NS = L::NS, NDT = L::NDT, NV = L::NV, LCH = L::LCH;
  constexpr int VCH = L::VCH;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  // One LDS arena serves the phases in turn.  Set-up: the fold order's
  // context lengths (at the start).  Set-up and main loop: each wave's K,
  // then V, chunk as f16 rows (vbuf), the workgroup's q rows (qs, f16, zero
  // past the group) and the partition's table slice (tab, part / block_size
  // entries).  The waves' merge (see below): per round, the states of XR head
  // tiles from the NW - 1 waves that do not own them (xo, xml: 16 and 8 bytes
  // per lane).  The split-context merge: its scratch (at the start).  XR is
  // as large as the LDS budget of the workgroups one CU holds allows, up to
  // every tile in one round.
  using A = GroupArena<D, HT, NW>;
  constexpr int kVbuf = A::kVbuf, XR = A::XR;
  static_assert(XR >= 1 && XR <= HT, "tiles per merge round");
  __shared__ uint4 arena[A::kWords];
  uint4* const vbuf = arena;
  uint4* const qs = arena + kVbuf;
  int* const tab = reinterpret_cast<int*>(arena + kVbuf + A::kQs);
  float4_t(*const xo)[64] = reinterpret_cast<float4_t(*)[64]>(arena);
  float2_t(*const xml)[64] = reinterpret_cast<float2_t(*)[64]>(arena + A::kXo);
  const int log2_bs = P.log2_bs;
  const int bs = 1 << log2_bs;
  int kvh, p, s, ctx, nparts, t0, t1, h0, nh, grp = 0;
  bool bad_len;
  SeqPrefix pf{0, 0};
  int gs = 0, r0 = 0;  // prefix pass: the group's first sequence, the workgroup's first row
  int tab0 = 0;        // table entry b0 + tid of the partition's slice, if it has one
  if constexpr (PREFIX) {
    int gi = 0;
    while (gi + 1 < P.ngroups && bx >= P.gwg[gi + 1]) ++gi;
    const int rowsets = (P.gwg[gi + 1] - P.gwg[gi]) / P.hkv;
    kvh = (bx - P.gwg[gi]) / rowsets;
    r0 = ((bx - P.gwg[gi]) % rowsets) * HT * 16;
    gs = P.gstart[gi];
    s = gs;
    p = by;
    if (p >= P.gparts[gi]) return;
    ctx = P.gtok[gi];
    bad_len = false;
    nparts = P.gparts[gi];
    t0 = p * kPrefixPartTokens;
    t1 = min(t0 + kPrefixPartTokens, ctx);
    h0 = 0;
    nh = min(HT * 16, (P.gstart[gi + 1] - gs) * P.group - r0);
  } else {
    grp = bx % groups_per_kv;
    kvh = bx / groups_per_kv;
    s = by;
    p = bz;
    int ctx_ranked = 0;
    if (P.fold_order) {
      // A launch of one partition per (sequence, KV head, group) that fills
      // two workgroups per CU in one round: workgroups i and i + (CUs) share
      // a CU, i.e. sequence positions y and y + B / 2.  Position y takes the
      // y-th longest sequence in the first half and the y-th shortest in the
      // second, so each CU holds a long and a short one and all CUs finish
      // together.  Ranks order by length, then index (a permutation).
      int* const lens = reinterpret_cast<int*>(vbuf);  // free until the main loop
      __shared__ int pick;
      const int B = P.num_seqs, half = (B + 1) / 2;
      const int want = s < half ? s : B - 1 - (s - half);
      if (threadIdx.x < B) lens[threadIdx.x] = P.ctx[threadIdx.x];
      __syncthreads();
      if (static_cast<int>(threadIdx.x) < B) {
        const int c = lens[threadIdx.x];
        int rank = 0;
        for (int u = 0; u < B; ++u) rank += lens[u] > c || (lens[u] == c && u < static_cast<int>(threadIdx.x));
        if (rank == want) pick = threadIdx.x;
      }
      __syncthreads();
      s = __builtin_amdgcn_readfirstlane(pick);
      ctx_ranked = __builtin_amdgcn_readfirstlane(lens[s]);  // no second global read
    }
    // tokens [0, begin) of a shared prefix were covered by the prefix pass
    pf = seq_prefix(P, s);
    const int part = P.part_tokens;  // a multiple of kPartitionTokens, chosen per launch
    // The table slice is read together with the context length, as if the
    // context ran to the partition's end (entries past the table row are not
    // read); entries past the real end are not used.
    {
      const int b0s = (pf.begin + p * part) >> log2_bs;
      if (static_cast<int>(threadIdx.x) < (part >> log2_bs) && b0s + static_cast<int>(threadIdx.x) < P.max_blocks)
        tab0 = P.tables[static_cast<int64_t>(s) * P.max_blocks + b0s + threadIdx.x];
    }
    ctx = P.fold_order ? ctx_ranked : P.ctx[s];
    bad_len = seq_bad_len(P, ctx, pf);
    // this launch's partitions; partition 0 starts from a shared prefix's
    // merged state, so these are all the partials to merge
    nparts = bad_len ? 1 : max(1, (ctx - pf.begin + part - 1) / part);
    if (p >= nparts) return;
    t0 = (bad_len ? 0 : pf.begin) + p * part;
    t1 = bad_len ? t0 : min(t0 + part, ctx);
    h0 = kvh * P.group + grp * HT * 16;          // first query head of the workgroup
    nh = min(HT * 16, P.group - grp * HT * 16);  // query heads of the workgroup
  }
  // workspace row of the workgroup's query row hh
  auto row_sh = [&](int hh) -> int64_t {
    if constexpr (PREFIX) {
      const int R = r0 + hh;
      return static_cast<int64_t>(gs + R / P.group) * P.hq + kvh * P.group + R % P.group;
    } else {
      return static_cast<int64_t>(s) * P.hq + h0 + hh;
    }
  };
  const int b0 = t0 >> log2_bs;
  const int64_t trow = static_cast<int64_t>(s) * P.max_blocks;
  const int64_t head_rows = static_cast<int64_t>(kvh) * bs;  // token rows before head kvh in a block
  const int64_t block_rows = static_cast<int64_t>(P.hkv) * bs;

  __shared__ int is_last;
  __shared__ Vec16 newkv[2][VCH];  // the new token's K and V rows in pool format

  // Fused append: every workgroup reading the new token takes it from the
  // caller's rows (staged in LDS in pool format) instead of the pool, and the
  // workgroup of the KV head's first query group stores it into its slot
  // after its main loop.
  const bool has_new = !PREFIX && P.k_new != nullptr && p == nparts - 1 && !bad_len && ctx >= 1;
  // Scores stay unscaled until the exponent.  A negative scale is folded
  // into q (negation is exact), so the scale applied there, |score_scale|,
  // keeps the order of the scores.
  const bool qneg = P.score_scale < 0.f;
  const float sscale = fabsf(P.score_scale);
  // The table slice, q and the new token's rows are all loaded before the
  // first of them is written to LDS, so the set-up costs one memory latency.
  // Table entries are kept as read (an entry out of range makes the
  // workgroup's result NaN and no K or V row is then loaded).
  int my_bad = bad_len ? 1 : 0;
  const int nb = t1 > t0 ? ((t1 - 1) >> log2_bs) - b0 + 1 : 0;
  if constexpr (PREFIX) tab0 = tid < nb ? P.tables[trow + b0 + tid] : 0;
  constexpr int QN = (HT * 16 * LCH + NW * 64 - 1) / (NW * 64);
  uint4 x[QN];
#pragma unroll
  for (int k = 0; k < QN; ++k) {
    const int i = tid + k * NW * 64, hh = i / LCH, ch = i % LCH;
    x[k] = make_uint4(0, 0, 0, 0);
    if (i < HT * 16 * LCH && hh < nh)
      x[k] = *reinterpret_cast<const uint4*>(static_cast<const half_t*>(P.q) + row_sh(hh) * D + ch * 8);
  }
  Vec16 nkv{{0, 0, 0, 0}};
  if (has_new && tid < 2 * VCH) {
    const int64_t src = (static_cast<int64_t>(s) * P.hkv + kvh) * D * static_cast<int64_t>(sizeof(half_t));
    const int which = tid / VCH, ch = tid % VCH;
    nkv = NewChunk<KV, half_t>::load((which ? P.v_new : P.k_new) + src, ch, which ? P.v_inv : P.k_inv);
  }
  if (tid < nb) {
    my_bad |= tab0 < 0 || tab0 >= P.num_blocks;
    tab[tid] = tab0;
  }
  for (int i = tid + NW * 64; i < nb; i += NW * 64) {  // slices longer than one entry per thread
    const int b = P.tables[trow + b0 + i];
    my_bad |= b < 0 || b >= P.num_blocks;
    tab[i] = b;
  }
#pragma unroll
  for (int k = 0; k < QN; ++k) {
    const int i = tid + k * NW * 64, hh = i / LCH, ch = i % LCH;
    if (qneg) x[k] = make_uint4(x[k].x ^ 0x80008000u, x[k].y ^ 0x80008000u, x[k].z ^ 0x80008000u, x[k].w ^ 0x80008000u);
    if (i < HT * 16 * LCH) qs[hh * LCH + (ch ^ L::swz_k(hh))] = x[k];
  }
  if (has_new && tid < 2 * VCH) newkv[tid / VCH][tid % VCH] = nkv;
  const bool bad = __syncthreads_or(my_bad) != 0;

  // B operand of the first product: q of head 16 * ht + n at head_dim
  // 32 st + 8 g .. + 7, from the workgroup's copy of q in LDS (rows swizzled
  // like K's; zero past the group), held in registers for the main loop
  half8_t qreg[HT][NS];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int hh = 16 * ht + n;
#pragma unroll
    for (int st = 0; st < NS; ++st)
      qreg[ht][st] = __builtin_bit_cast(half8_t, qs[hh * LCH + ((4 * st + g) ^ L::swz_k(hh))]);
  }
  auto q_operand = [&](int ht, int st) -> half8_t { return qreg[ht][st]; };

  float4_t o[HT][NDT];
  float m[HT], lsum[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m[ht] = -INFINITY;
    lsum[ht] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[ht][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  // A shared prefix's partials enter through wave 0 of partition 0: lane
  // (g, n) takes head column n's max and elements 16 dt + 4 g + i, and the
  // weight sum goes to the g = 0 lanes (the four lane groups' sums are added
  // at the end).
  if constexpr (!PREFIX) {
    if (p == 0 && pf.pre > 0 && !bad && w == 0) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const int hh = 16 * ht + n;
        if (hh >= nh) continue;
        const int64_t sh = row_sh(hh);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          float M, L, v[4];
          load_prefix_state<D, 4>(P, sh, pf.pre, 16 * dt + 4 * g, M, L, v);
          m[ht] = M;
          lsum[ht] = g == 0 ? L : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[ht][dt][i] = v[i];
        }
      }
    }
  }

  uint4* const vb = vbuf + w * (kChunk * LCH);
  const int nchunks = bad ? 0 : (t1 - t0 + kChunk - 1) / kChunk;
  // the chunk holding the new token (only it needs substitution); -1 if none
  const int new_chunk = has_new ? (ctx - 1 - t0) / kChunk : -1;

  // Addresses.  UNI (blocks of 16 or more tokens): a 16-token tile of a
  // chunk lies in one block, so each tile's block is one wave-uniform table
  // read and lanes add 32-bit offsets within the block.  Otherwise every
  // lane looks up its own token's block.
  const int64_t tile_bytes = static_cast<int64_t>(bs) * D * KVB;  // one (block, head) tile
  auto tile_base = [&](const char* pool, int cb, int tau) -> const char* {
    const int blk = __builtin_amdgcn_readfirstlane(tab[(min(cb + 16 * tau, t1 - 1) >> log2_bs) - b0]);
    return pool + (static_cast<int64_t>(blk) * P.hkv + kvh) * tile_bytes;
  };
  auto lane_row = [&](const char* pool, int t) -> const char* {
    return pool + (tab[(t >> log2_bs) - b0] * block_rows + head_rows + (t & (bs - 1))) * (D * KVB);
  };
  // Loads of chunk c, coalesced: load v of lane l covers 16 bytes (chunk
  // ch) of token row r = (64 v + l) / VCH, so a wave load reads whole rows.
  // K and V rows share the offsets.  The new token's slot is read like any
  // other; its pool value is replaced when the chunk is consumed.
  auto row_off = [&](int cb, int v, const char* pool) -> const char* {
    const int f = v * 64 + lane;
    const int r = f / VCH, ch = f % VCH;
    const int t = min(cb + r, t1 - 1);
    if constexpr (UNI) {
      // rows per load are 64 / VCH: a load stays within one 16-token tile
      // when that is at most 16, so its tile is known at compile time;
      // otherwise (32 rows per load) each lane picks one of the two bases
      const char* base;
      if constexpr (64 / VCH <= 16) {
        base = tile_base(pool, cb, (v * (64 / VCH)) >> 4);
      } else {
        const char* b0p = tile_base(pool, cb, 0);
        const char* b1p = tile_base(pool, cb, 1);
        base = (r >> 4) ? b1p : b0p;
      }
      // an unsigned 32-bit offset lets the load take the scalar base as is
      return base + static_cast<uint32_t>((t & (bs - 1)) * (D * KVB) + ch * 16);
    } else {
      return lane_row(pool, t) + ch * 16;
    }
  };
  // A chunk that ends inside the partition (every chunk but its last) needs
  // no clamp.  With blocks of 16 or more tokens and at most 16 rows per wave
  // load, a load's rows then lie in one 16-token tile: its address is the
  // tile's wave-uniform base (the table entry times the pool's stride per
  // block, a 32-bit product the host checks, plus the tile's first row in
  // its block) and a per-lane offset that is the same for every chunk, so
  // the K and V loads of a chunk share two table reads.
  constexpr int RPL = 64 / VCH;  // token rows per wave load
  constexpr bool FAST = UNI && RPL <= 16;
  const uint32_t block_stride = static_cast<uint32_t>(P.hkv) * static_cast<uint32_t>(tile_bytes);
  const uint32_t lane_const = static_cast<uint32_t>((lane / VCH) * (D * KVB) + (lane % VCH) * 16);
  const char* const kbase = P.kc + kvh * tile_bytes;
  const char* const vbase = P.vc + kvh * tile_bytes;
  auto chunk_tiles = [&](int c, uint64_t (&toff)[2]) {
    const int cb = t0 + c * kChunk;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tt = cb + 16 * tau;
      const uint32_t blk = __builtin_amdgcn_readfirstlane(tab[(tt >> log2_bs) - b0]);
      toff[tau] = static_cast<uint64_t>(blk) * block_stride + static_cast<uint32_t>((tt & (bs - 1)) * (D * KVB));
    }
  };
  auto load_tiles = [&](Vec16 (&x)[NV], const char* base, const uint64_t (&toff)[2]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const char* tb = base + toff[(v * RPL) >> 4];
      x[v] = load16_stream(tb + lane_const + ((v * RPL) & 15) * (D * KVB));
    }
  };
  auto load_rows = [&](Vec16 (&x)[NV], const char* pool, int c) {
    const int cb = t0 + c * kChunk;
#pragma unroll
    for (int v = 0; v < NV; ++v) x[v] = load16_stream(row_off(cb, v, pool));
  };
  // both rows of chunk c, by the fast path where it applies
  auto load_chunk = [&](Vec16 (&kx)[NV], Vec16 (&vx)[NV], int c) {
    if (FAST && t0 + (c + 1) * kChunk <= t1) {
      uint64_t toff[2];
      chunk_tiles(c, toff);
      load_tiles(kx, kbase, toff);
      load_tiles(vx, vbase, toff);
    } else {
      load_rows(kx, P.kc, c);
      load_rows(vx, P.vc, c);
    }
  };
  // The chunk holding the new token: lanes at its row (and lanes past the
  // context, which re-read it) take the caller's K/V in pool format, staged
  // in LDS at the start.
  auto substitute = [&](Vec16 (&x)[NV], int which, int c) {
    const int cb = t0 + c * kChunk;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int f = v * 64 + lane;
      const int r = f / VCH, ch = f % VCH;
      if (min(cb + r, t1 - 1) == ctx - 1) x[v] = newkv[which][ch];
    }
  };
  // Rows of a chunk into the wave's LDS slice as f16 (FP8 converted
  // exactly), 16-byte chunks swizzled by swz(row).
  auto rows_to_lds = [&](const Vec16 (&x)[NV], auto swz) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int f = v * 64 + lane;
      const int r = f / VCH, ch = f % VCH;
      if constexpr (KVB == 2) {
        vb[r * LCH + (ch ^ swz(r))] = make_uint4(x[v].w[0], x[v].w[1], x[v].w[2], x[v].w[3]);
      } else {
        const half8_t lo = e4m3x8_to_half8(x[v].w[0], x[v].w[1]);
        const half8_t hi = e4m3x8_to_half8(x[v].w[2], x[v].w[3]);
        vb[r * LCH + ((2 * ch) ^ swz(r))] = __builtin_bit_cast(uint4, lo);
        vb[r * LCH + ((2 * ch + 1) ^ swz(r))] = __builtin_bit_cast(uint4, hi);
      }
    }
  };

  // Compute chunk c from its loaded K and V.  The register copies are
  // refilled with chunk nx's loads as soon as they are in LDS, so those loads
  // fly during the rest of the chunk.  One wave's LDS accesses complete in
  // order, so the V rows may overwrite the K rows once the K reads are issued.
  //
  // Only the partition's last chunk can run past its end.  Its rows past the
  // end re-read the last token, so their scores repeat a real score and
  // leave the chunk's max as it is; their weights are set to zero.
  auto process_chunk = [&](Vec16 (&kr)[NV], Vec16 (&vr)[NV], int c, int nx) {
    const int cb = t0 + c * kChunk;
    const bool last = cb + kChunk > t1;
    const bool sub = c == new_chunk;  // wave-uniform, at most once
    // the next chunk's loads: tile offsets once for K and V on the fast path
    const bool nx_fast = FAST && nx < nchunks && t0 + (nx + 1) * kChunk <= t1;
    uint64_t toff[2] = {0, 0};
    if (nx_fast) chunk_tiles(nx, toff);
    if (sub) substitute(kr, 0, c);
    rows_to_lds(kr, L::swz_k);
    if (nx_fast) {
      load_tiles(kr, kbase, toff);
    } else if (nx < nchunks) {
      load_rows(kr, P.kc, nx);
    }

    // scores S^T (unscaled): lane (g, n) gets tokens 16 tau + 4 g + i of
    // head 16 ht + n
    float sc[HT][8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int r = 16 * tau + n;
      half8_t ka[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st) ka[st] = __builtin_bit_cast(half8_t, vb[r * LCH + ((4 * st + g) ^ L::swz_k(r))]);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NS; ++st) acc = mfma16x16x32(ka[st], q_operand(ht, st), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[ht][4 * tau + i] = acc[i];
      }
    }

    if (sub) substitute(vr, 1, c);
    rows_to_lds(vr, L::swz_v);
    if (nx_fast) {
      load_tiles(vr, vbase, toff);
    } else if (nx < nchunks) {
      load_rows(vr, P.vc, nx);
    }

    // online softmax per head column; the weights become the B operand.
    // The running max moves only when a chunk's max exceeds it by more than
    // kLazy (log2 units), so weights stay at most 2^kLazy and the rescale of
    // the accumulators is skipped by the whole wave in most chunks.  The
    // chunk's max is taken over unscaled scores and then scaled (rounding
    // is monotonic and sscale >= 0); each weight is 2^(score * sscale - m)
    // with one rounding.  A column's max exceeds the bound exactly when one
    // of its lanes' maxima does, so the max across the column's four lanes
    // is taken only in chunks where some lane's does.
    half8_t pf[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float mlane = sc[ht][0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mlane = fmaxf(mlane, sc[ht][j]);
      if (__any(mlane * sscale > m[ht] + kLazy)) {
        const float mloc = max_over_rows(mlane) * sscale;
        const bool raise = mloc > m[ht] + kLazy;  // uniform within a head column
        const float m_new = raise ? mloc : m[ht];
        const float alpha = fast_exp2(m[ht] - m_new);  // 0 on the first chunk (m = -inf)
        lsum[ht] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[ht][dt] *= alpha;
        m[ht] = m_new;
      }
      // weights as f16 pairs; their sum is taken from those same f16 values
      // (a dot product with ones: exact products, f32 accumulation)
      half2_t hp[4];
      float psum = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2_t e = {fast_exp2(fmaf(sc[ht][2 * k], sscale, -m[ht])),
                            fast_exp2(fmaf(sc[ht][2 * k + 1], sscale, -m[ht]))};
        hp[k] = __builtin_convertvector(e, half2_t);
      }
      if (last) {  // rows past the end weigh zero
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (cb + 16 * (j >> 2) + 4 * g + (j & 3) >= t1) hp[j >> 1][j & 1] = 0;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) psum = __builtin_amdgcn_fdot2(hp[k], half2_t{1, 1}, psum, false);
      pf[ht] = __builtin_bit_cast(half8_t, hp);
      lsum[ht] += psum;
    }

    // V^T tiles by transposing reads: lane (g, n) gets column 16 dt + n of
    // tokens 16 h + 4 g + k (k = 0..3) from the read of half h
    const int k4 = n >> 2, q4 = n & 3;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      half8_t va;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r = 16 * hf + 4 * g + k4;
        const int chunk = (2 * dt + (q4 >> 1)) ^ L::swz_v(r);
        // (bit-cast the whole vector: a bit-cast of one vector element is
        // lowered as element 0 by this compiler)
        const half4_t x = __builtin_bit_cast(
            half4_t, lds_read_tr16(reinterpret_cast<const char*>(vb) + r * (2 * D) + chunk * 16 + (q4 & 1) * 8));
#pragma unroll
        for (int k = 0; k < 4; ++k) va[4 * hf + k] = x[k];
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) o[ht][dt] = mfma16x16x32(va, pf[ht], o[ht][dt]);
    }
  };

  {
    Vec16 kr[NV], vr[NV];
    if (w < nchunks) load_chunk(kr, vr, w);
    for (int c = w; c < nchunks; c += NW) process_chunk(kr, vr, c, c + NW);
  }
  // the new token into its pool slot: the rows staged in LDS by the same
  // threads, the block from the table slice (skipped if out of range)
  if (has_new && grp == 0 && tid < 2 * VCH) {
    const int pos = ctx - 1;
    const int b = tab[(pos >> log2_bs) - b0];
    if (b >= 0 && b < P.num_blocks) {
      const int64_t tok_row = (static_cast<int64_t>(b) * P.hkv + kvh) * bs + (pos & (bs - 1));
      store16((tid < VCH ? P.kw : P.vw) + static_cast<size_t>(tok_row * D) * KVB + (tid % VCH) * 16,
              newkv[tid / VCH][tid % VCH]);
    }
  }

  // each head's weight sum over the wave's four lane groups
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) lsum[ht] = sum_over_rows(lsum[ht]);
  __syncthreads();  // the exchange reuses the main loop's LDS

  // Merge the waves' partial results by head tile: tile t belongs to wave
  // t % NW.  In each round of XR tiles every other wave writes its state of
  // the round's tiles to LDS at once, and each owner merges the NW - 1 states
  // of each tile it owns in a fixed order (the waves after it, cyclically), so
  // results are deterministic; every wave then stores the tiles it owns.  (A chain
  // of NW - 1 pairwise merges through one wave had each step move a whole
  // wave's state through LDS.)
  constexpr int NROUND = (HT + XR - 1) / XR;
#pragma unroll
  for (int r = 0; r < NROUND; ++r) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int t = r * XR + i;
      if (t < HT && w != t % NW) {
        const int k = (w - t % NW - 1 + NW) % NW;
        xml[i * (NW - 1) + k][lane] = float2_t{m[t], lsum[t]};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) xo[(i * (NW - 1) + k) * NDT + dt][lane] = o[t][dt];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int t = r * XR + i;
      if (t < HT && w == t % NW) {
        float2_t ml[NW - 1];
        float M = m[t];
#pragma unroll
        for (int k = 0; k < NW - 1; ++k) {
          ml[k] = xml[i * (NW - 1) + k][lane];
          M = fmaxf(M, ml[k][0]);
        }
        const float mu = (M == -INFINITY) ? 0.f : M;
        const float a = exp2f(m[t] - mu);
        float L = lsum[t] * a;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= a;
#pragma unroll
        for (int k = 0; k < NW - 1; ++k) {
          const float bk = exp2f(ml[k][0] - mu);
          L += ml[k][1] * bk;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[t][dt] += bk * xo[(i * (NW - 1) + k) * NDT + dt][lane];
        }
        lsum[t] = L;
        m[t] = M;
      }
    }
    if (r + 1 < NROUND) __syncthreads();  // the next round rewrites the exchange
  }

  half_t* out = static_cast<half_t*>(P.out);
  // the prefix pass always leaves partials (slot p); decode leaves the output
  // itself when it is the head's only partition, else partials after the
  // prefix's
  const bool direct = !PREFIX && nparts == 1;
  const int slot = PREFIX ? p : pf.pre + p;
  // decode rows are consecutive (s * hq + h0 + hh): windows from the first
  const int64_t row0 = static_cast<int64_t>(s) * P.hq + h0;
  const uint32_t rows_span = static_cast<uint32_t>((nh - 1) * static_cast<int64_t>(P.max_parts) + 1);
  const CoherentWindow wso(P.ws_o + (row0 * P.max_parts + slot) * D, rows_span * (D * 4u));
  const CoherentWindow wsml(P.ws_ml + (row0 * P.max_parts + slot) * 2, rows_span * 8u);
  {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int hh = 16 * ht + n;
      if (ht % NW != w || hh >= nh) continue;  // the owner stores its tile
      const int64_t sh = row_sh(hh);
      const float mx = bad ? NAN : m[ht];
      const float lx = bad ? NAN : lsum[ht];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + 4 * g;
        if (direct) {
          const float f = bad ? NAN : (ctx > 0 ? P.v_scale / lx : 0.f);
          half4_t r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = static_cast<_Float16>(bad ? NAN : o[ht][dt][i] * f);
          *reinterpret_cast<half4_t*>(out + sh * D + d) = r;
        } else if (PREFIX) {
          // read by a later launch: plain 16-byte stores, V-scaled like
          // every partial
          const float4_t nan4 = {NAN, NAN, NAN, NAN};
          *reinterpret_cast<float4_t*>(P.ws_o + (sh * P.max_parts + slot) * D + d) =
              bad ? nan4 : o[ht][dt] * P.v_scale;
        } else {
          const float4_t nan4 = {NAN, NAN, NAN, NAN};
          wso.store4(static_cast<uint32_t>(hh * static_cast<int64_t>(P.max_parts) * D + d) * 4u,
                     bad ? nan4 : o[ht][dt] * P.v_scale);
        }
      }
      if (!direct && g == 0) {
        if constexpr (PREFIX) {
          P.ws_ml[(sh * P.max_parts + slot) * 2] = mx;
          P.ws_ml[(sh * P.max_parts + slot) * 2 + 1] = lx;
        } else {
          wsml.store2(static_cast<uint32_t>(hh * static_cast<int64_t>(P.max_parts)) * 8u, float2_t{mx, lx});
        }
      }
    }
  }
  if (direct || PREFIX) return;

  // Split context: the last partition to finish merges every partial of the
  // workgroup's heads exactly and restores the arrival counter to zero.
  //
  // Why the last arrival sees every partial, although its workgroups may run
  // on different XCDs, each with its own L2 that is not coherent with the
  // others.  The argument rests on the gfx942/gfx950 memory model as the
  // LLVM AMDGPU backend documents it (AMDGPUUsage, "Memory Model GFX942"):
  // an access with the SC1 cache-policy bit is what that backend emits for a
  // relaxed (monotonic) atomic load or store at agent scope; it is served at
  // the agent's point of coherence, not from a cache line of this XCD.
  //  1. Every partial is written with SC1 stores (CoherentWindow::store*),
  //     so each store completes at the point of coherence.
  //  2. s_waitcnt(0) then holds each wave until all of its stores are
  //     acknowledged (on gfx9 stores count in vmcnt and are acknowledged
  //     once performed at the level their policy names), and the barrier
  //     holds the workgroup until every wave has passed that wait.  Only then
  //     does thread 0 add to the counter.
  //  3. The counter add is an agent-scope atomic, performed at the point of
  //     coherence, so all adds to one counter are ordered there.  The add
  //     that returns nparts - 1 comes after every other partition's add, and
  //     each of those was issued only after that partition's stores were
  //     acknowledged (2).  Hence every partial is at the point of coherence
  //     before the last add returns.
  //  4. The last workgroup reads the partials only after its add has
  //     returned (the barrier below and the branch on is_last; a barrier is
  //     also a compiler fence, so no load is hoisted above it), and it reads
  //     them with SC1 loads (CoherentWindow::load*), which are served at the
  //     point of coherence and cannot hit a stale line of its own L1 or L2.
  // The C++ model would ask for release/acquire on the counter; the backend
  // lowers those to a write-back of this XCD's whole L2 (buffer_wbl2) before
  // the add and an invalidation of it (buffer_inv) after, which steps 1 and
  // 4 make unnecessary: only the partials cross XCDs, and they never stay in
  // a non-coherent cache.  The counter is reset with an agent-scope store
  // after the merge; the next launch sees it through the kernel boundary.
  const int64_t cidx = static_cast<int64_t>(s) * P.hq + h0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(&P.counters[cidx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
  __syncthreads();
  if (!is_last) return;
  // the V staging buffers are free now: they hold the merge's scratch
  float* scratch = reinterpret_cast<float*>(vbuf);
  constexpr int kMergeItems = (HT * 16 * (D / 4) + NW * 64 - 1) / (NW * 64);
  merge_partials<half_t, D, NW * 64, (kMergeItems < 4 ? kMergeItems : 4)>(
      P, static_cast<int64_t>(s) * P.hq + h0, nh, pf.pre, nparts, tid, scratch, scratch + kMergeCap);
  if (tid == 0) __hip_atomic_store(&P.counters[cidx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// UNI addressing (wave-uniform tile bases): blocks of 16 or more tokens, and
// a pool stride per block (all KV heads' tiles) that fits 32 bits.
inline bool tile_addressing(const pa_kv_cache& c) {
  const int kvb = c.kv_dtype == PA_F32 ? 4 : c.kv_dtype == PA_F16 ? 2 : 1;
  return c.block_size >= 16 &&
         static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim * kvb <= static_cast<int64_t>(UINT32_MAX);
}

// The prefix pass's grid for row sets of 16 * ht rows: fills P.gwg (the
// first grid column of each group) and returns the number of columns (grid
// x); *parts receives the most prefix partitions of any group (grid y).
inline int prefix_grid(const DecodeArgs& a, int ht, DecodeParams& P, int* parts) {
  const int G = a.num_q_heads / a.cache->num_kv_heads;
  int max_parts = 0;
  P.gwg[0] = 0;
  for (int g = 0; g < a.ngroups; ++g) {
    const int rows = (a.gstart[g + 1] - a.gstart[g]) * G;
    const int rowsets = a.gparts[g] > 0 ? (rows + 16 * ht - 1) / (16 * ht) : 0;
    P.gwg[g + 1] = P.gwg[g] + a.cache->num_kv_heads * rowsets;
    max_parts = std::max(max_parts, a.gparts[g]);
  }
  *parts = max_parts;
  return P.gwg[a.ngroups];
}

}  // namespace
}  // namespace pa
