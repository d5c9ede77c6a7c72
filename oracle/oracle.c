/*
 * Reference oracle for paged KV-cache decode — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, scalar C.  Every floating-point result is computed in double.
 * It shares no code, header or table with the GPU library; only tests, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.
 *
 * Citation key used below (title of the web page, then its section):
 *   [F55 §x]  page "KV 缓存与分页注意力" (world.lapla.si, plate F55), section x
 *   [AIF x]   page "KV 缓存" (aiinfact.com topic page), part x
 *   [IPX §x]  page "读懂PagedAttention：vLLM的KV缓存与GPU显存管理"
 *             (iplexlaw.co.kr), sub-heading x
 *
 * Storage layout the oracle indexes (chosen by this library, see the public
 * header): a K pool and a V pool, each [num_blocks][num_kv_heads][block_size]
 * [head_dim] elements; element (b, h, slot, i) sits at
 * ((b * num_kv_heads + h) * block_size + slot) * head_dim + i.
 *
 * Data type codes (the oracle's own): 0 = binary32, 1 = binary16,
 * 2 = OCP FP8 E4M3, 3 = binary64 (oracle-only, for the cached/uncached
 * equivalence model).
 *
 * Parity pins: every function here is checked against something other than
 * itself by the CPU tests (brute-force contiguous attention, library
 * conversions, closed forms, printed counts).  None is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_E4M3 = 2, OR_F64 = 3 };

static size_t elem_size(int dt) {
  switch (dt) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_E4M3: return 1;
    case OR_F64: return 8;
  }
  return 0;
}

/* ---- scalar formats --------------------------------------------------- */

/* IEEE 754 binary16 -> double, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is subnormal. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24);
  } else if (e == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + m), e - 25);
  }
  return sign ? -v : v;
}

/* OCP FP8 E4M3 -> double: 1 sign bit, 4 exponent bits (bias 7), 3 fraction
 * bits, no infinities, S.1111.111 is NaN, exponent 0 is subnormal.  The
 * pages only say the cache may keep one byte per number [F55 §后来的做法];
 * the concrete 8-bit format is this library's reading. */
double oracle_e4m3_to_f64(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xf;
  int m = b & 0x7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) {
    v = ldexp((double)m, -9);
  } else {
    v = ldexp((double)(8 + m), e - 10);
  }
  return sign ? -v : v;
}

/* Round a non-negative double that is exactly representable to the nearest
 * integer, ties to the even integer. */
static double round_half_even(double q) {
  double fl = floor(q);
  double frac = q - fl;
  if (frac > 0.5) return fl + 1.0;
  if (frac < 0.5) return fl;
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* binary32 -> E4M3, round to nearest even, saturating: finite magnitudes and
 * infinities beyond the largest code become +-448 (code 0x7E).  Every NaN
 * becomes 0x7F: IEEE 754 does not give the sign of a NaN any meaning (an
 * arithmetic result's NaN sign is unspecified), so the store does not keep it. */
uint8_t oracle_e4m3_encode(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  if (isnan(y)) return (uint8_t)0x7f;
  if (a > 448.0) return (uint8_t)(sign | 0x7e);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: value = m * 2^-9, m = 0..8 (8 is the least normal) */
    double m = round_half_even(a * 512.0);
    return (uint8_t)(sign | (uint8_t)m);
  }
  int e = 0;
  (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) -> a in [2^(e-1), 2^e) */
  e -= 1;             /* now a in [2^e, 2^(e+1)) */
  double q = ldexp(a, 3 - e); /* in [8, 16), exact */
  double n = round_half_even(q);
  if (n == 16.0) {
    n = 8.0;
    e += 1;
  }
  int code = ((e + 7) << 3) | ((int)n - 8);
  if (code > 0x7e) code = 0x7e; /* unreachable for a <= 448 */
  return (uint8_t)(sign | code);
}

/* The quantiser applied when a number is stored in an FP8 cache: one binary32
 * multiply by the inverse scale (round to nearest even), then the encoder. */
uint8_t oracle_e4m3_quantize(float x, float inv_scale) {
  volatile float y = x * inv_scale; /* one IEEE binary32 product */
  return oracle_e4m3_encode(y);
}

/* Read element i of an array of dtype dt as a double (exact conversion). */
static double load_as_f64(const void* base, int dt, size_t i) {
  switch (dt) {
    case OR_F32: return (double)((const float*)base)[i];
    case OR_F16: return oracle_f16_to_f64(((const uint16_t*)base)[i]);
    case OR_E4M3: return oracle_e4m3_to_f64(((const uint8_t*)base)[i]);
    case OR_F64: return ((const double*)base)[i];
  }
  return NAN;
}

/* binary16 -> binary32 is exact; used to feed the quantiser. */
static float load_as_f32(const void* base, int dt, size_t i) {
  return (float)load_as_f64(base, dt, i);
}

/* ---- the pool --------------------------------------------------------- */

static size_t pool_index(int blk, int h, int slot, int i, int hkv, int bs, int d) {
  return (((size_t)blk * hkv + h) * bs + slot) * (size_t)d + i;
}

/* Store one token's vector for KV head h into (blk, slot).  Same dtype:
 * a byte copy.  E4M3 pool: quantise each number.  Any other pair: the exact
 * value must be representable (f32 <- f16, f64 <- anything). */
static int put_vector(void* pool, int kv_dt, const void* src, int act_dt, size_t src_off,
                      int blk, int h, int slot, int hkv, int bs, int d, float inv_scale) {
  size_t dst_off = pool_index(blk, h, slot, 0, hkv, bs, d);
  for (int i = 0; i < d; ++i) {
    if (kv_dt == act_dt) {
      size_t es = elem_size(kv_dt);
      memcpy((char*)pool + (dst_off + i) * es, (const char*)src + (src_off + i) * es, es);
    } else if (kv_dt == OR_E4M3) {
      ((uint8_t*)pool)[dst_off + i] = oracle_e4m3_quantize(load_as_f32(src, act_dt, src_off + i), inv_scale);
    } else if (kv_dt == OR_F32 && act_dt == OR_F16) {
      ((float*)pool)[dst_off + i] = load_as_f32(src, act_dt, src_off + i);
    } else if (kv_dt == OR_F64) {
      ((double*)pool)[dst_off + i] = load_as_f64(src, act_dt, src_off + i);
    } else {
      return 1;
    }
  }
  return 0;
}

/*
 * Append: every running sequence stores the newly generated token's K and V
 * into the free slot of its last block [F55 §一次写一个词元, §块表];
 * [IPX §分离逻辑顺序与实际存储位置] (later tokens go into the last block's
 * free slot).  ctx_lens[s] counts the new token, so its position is
 * ctx_lens[s] - 1; logical block pos / bs maps through the block table to a
 * physical block, slot pos % bs.  k_new/v_new are [num_seqs][hkv][d].
 * Returns 0, or 1 on a bad argument (nothing written for that sequence).
 */
int oracle_append(void* k_pool, void* v_pool, int kv_dt, int num_blocks, int bs, int hkv, int d,
                  const void* k_new, const void* v_new, int act_dt,
                  const int32_t* tables, int max_blocks, const int32_t* ctx_lens, int num_seqs,
                  float k_inv_scale, float v_inv_scale) {
  int bad = 0;
  for (int s = 0; s < num_seqs; ++s) {
    int pos = ctx_lens[s] - 1;
    if (pos < 0 || pos / bs >= max_blocks) { bad = 1; continue; }
    int blk = tables[(size_t)s * max_blocks + pos / bs];
    if (blk < 0 || blk >= num_blocks) { bad = 1; continue; }
    for (int h = 0; h < hkv; ++h) {
      size_t src = ((size_t)s * hkv + h) * d;
      bad |= put_vector(k_pool, kv_dt, k_new, act_dt, src, blk, h, pos % bs, hkv, bs, d, k_inv_scale);
      bad |= put_vector(v_pool, kv_dt, v_new, act_dt, src, blk, h, pos % bs, hkv, bs, d, v_inv_scale);
    }
  }
  return bad;
}

/*
 * Prompt write: the whole prompt's K/V arrive at once and go into the blocks
 * allocated for the input [F55 §一次写一个词元]; [IPX §分离逻辑顺序与实际存储位置].
 * Sequence s writes count[s] tokens at logical positions start[s] ...
 * start[s] + count[s] - 1, taken from rows src_row[s] ... of k_src/v_src,
 * which are [total_rows][hkv][d].
 */
int oracle_write_tokens(void* k_pool, void* v_pool, int kv_dt, int num_blocks, int bs, int hkv, int d,
                        const void* k_src, const void* v_src, int act_dt,
                        const int64_t* src_row, const int32_t* start, const int32_t* count,
                        const int32_t* tables, int max_blocks, int num_seqs,
                        float k_inv_scale, float v_inv_scale) {
  int bad = 0;
  for (int s = 0; s < num_seqs; ++s) {
    for (int j = 0; j < count[s]; ++j) {
      int pos = start[s] + j;
      if (pos < 0 || pos / bs >= max_blocks) { bad = 1; continue; }
      int blk = tables[(size_t)s * max_blocks + pos / bs];
      if (blk < 0 || blk >= num_blocks) { bad = 1; continue; }
      for (int h = 0; h < hkv; ++h) {
        size_t src = ((size_t)(src_row[s] + j) * hkv + h) * d;
        bad |= put_vector(k_pool, kv_dt, k_src, act_dt, src, blk, h, pos % bs, hkv, bs, d, k_inv_scale);
        bad |= put_vector(v_pool, kv_dt, v_src, act_dt, src, blk, h, pos % bs, hkv, bs, d, v_inv_scale);
      }
    }
  }
  return bad;
}

/*
 * Copy-on-write copy: before a sequence writes into a block that others still
 * reference, the block is copied and the write goes to the copy
 * [F55 §常见问题 (copy-on-write)]; [IPX §同一提示生成两个回答的假想例子].
 * pairs is [n][2] = (source block, destination block); the whole block
 * (every KV head, every slot) is copied, K and V alike.
 */
int oracle_copy_blocks(void* k_pool, void* v_pool, int kv_dt, int num_blocks, int bs, int hkv, int d,
                       const int32_t* pairs, int n) {
  size_t blk_bytes = (size_t)hkv * bs * d * elem_size(kv_dt);
  int bad = 0;
  for (int p = 0; p < n; ++p) {
    int src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) { bad = 1; continue; }
    memmove((char*)k_pool + (size_t)dst * blk_bytes, (char*)k_pool + (size_t)src * blk_bytes, blk_bytes);
    memmove((char*)v_pool + (size_t)dst * blk_bytes, (char*)v_pool + (size_t)src * blk_bytes, blk_bytes);
  }
  return bad;
}

/*
 * Decode attention for one (sequence, query head): the new token's query
 * attends over every cached key of its sequence, the token itself included,
 * fetched block by block through the block table, in logical token order
 * [F55 §块表]; [IPX §分离逻辑顺序与实际存储位置].  The attention itself is
 * the scaled dot-product softmax attention the pages cite (Vaswani et al.)
 * with the 1/sqrt(d) scale supplied as sm_scale [AIF level-3 account table].
 * Query heads map onto KV heads in contiguous groups (head h reads KV head
 * h / (hq / hkv)) [F55 §后来的做法].  E4M3 pools are dequantised as
 * code value * scale.
 *
 *   s_t   = sm_scale * sum_i q[i] * K_t[i]
 *   out[i] = sum_t exp(s_t - max_u s_u) * V_t[i] / sum_t exp(s_t - max_u s_u)
 *
 * A zero-length context writes zeros.  *macs (if non-NULL) is incremented by
 * one per multiply-accumulate of the two dot-product loops.
 */
static void decode_one(const void* k_pool, const void* v_pool, int kv_dt, int bs, int hkv, int d,
                       const void* q, int act_dt, int hq, const int32_t* table, int n,
                       int s, int h, double sm_scale, double k_scale, double v_scale,
                       double* out, double* scores, long long* macs) {
  int g = h / (hq / hkv);
  const size_t q_off = ((size_t)s * hq + h) * d;
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  if (n <= 0) return;
  double kmul = (kv_dt == OR_E4M3) ? k_scale : 1.0;
  double vmul = (kv_dt == OR_E4M3) ? v_scale : 1.0;
  double mx = -INFINITY;
  for (int t = 0; t < n; ++t) {
    int blk = table[t / bs];
    size_t base = pool_index(blk, g, t % bs, 0, hkv, bs, d);
    double dot = 0.0;
    for (int i = 0; i < d; ++i) {
      dot += load_as_f64(q, act_dt, q_off + i) * (load_as_f64(k_pool, kv_dt, base + i) * kmul);
    }
    if (macs) *macs += d;
    scores[t] = sm_scale * dot;
    if (scores[t] > mx) mx = scores[t];
  }
  double denom = 0.0;
  for (int t = 0; t < n; ++t) {
    scores[t] = exp(scores[t] - mx);
    denom += scores[t];
  }
  for (int t = 0; t < n; ++t) {
    int blk = table[t / bs];
    size_t base = pool_index(blk, g, t % bs, 0, hkv, bs, d);
    for (int i = 0; i < d; ++i) {
      out[i] += scores[t] * (load_as_f64(v_pool, kv_dt, base + i) * vmul);
    }
    if (macs) *macs += d;
  }
  for (int i = 0; i < d; ++i) out[i] /= denom;
}

/* Whole batch: out is [num_seqs][hq][d] doubles.  Returns 0, or 1 if a table
 * entry a context needs is out of range (that sequence's output is zeros). */
int oracle_decode(const void* k_pool, const void* v_pool, int kv_dt, int num_blocks, int bs, int hkv, int d,
                  const void* q, int act_dt, int hq, const int32_t* tables, int max_blocks,
                  const int32_t* ctx_lens, int num_seqs, double sm_scale, double k_scale, double v_scale,
                  double* out, long long* macs) {
  int bad = 0;
  if (hkv <= 0 || hq % hkv != 0) return 1;
  int maxn = 0;
  for (int s = 0; s < num_seqs; ++s) if (ctx_lens[s] > maxn) maxn = ctx_lens[s];
  double* scores = (double*)malloc(sizeof(double) * (size_t)(maxn > 0 ? maxn : 1));
  if (!scores) return 1;
  for (int s = 0; s < num_seqs; ++s) {
    const int32_t* table = tables + (size_t)s * max_blocks;
    int n = ctx_lens[s];
    int ok = (n >= 0) && ((n + bs - 1) / bs <= max_blocks);
    for (int j = 0; ok && j < (n + bs - 1) / bs; ++j) ok = table[j] >= 0 && table[j] < num_blocks;
    for (int h = 0; h < hq; ++h) {
      double* o = out + ((size_t)s * hq + h) * d;
      if (!ok) { for (int i = 0; i < d; ++i) o[i] = 0.0; continue; }
      decode_one(k_pool, v_pool, kv_dt, bs, hkv, d, q, act_dt, hq, table, n, s, h,
                 sm_scale, k_scale, v_scale, o, scores, macs);
    }
    if (!ok) bad = 1;
  }
  free(scores);
  return bad;
}

/* A sample of (sequence, head) pairs, for outputs of workloads too large to
 * recompute whole: out is [num_pairs][d]. */
int oracle_decode_pairs(const void* k_pool, const void* v_pool, int kv_dt, int num_blocks, int bs, int hkv, int d,
                        const void* q, int act_dt, int hq, const int32_t* tables, int max_blocks,
                        const int32_t* ctx_lens, int num_seqs, double sm_scale, double k_scale, double v_scale,
                        const int32_t* pair_seq, const int32_t* pair_head, int num_pairs, double* out) {
  int bad = 0;
  if (hkv <= 0 || hq % hkv != 0) return 1;
  for (int p = 0; p < num_pairs; ++p) {
    int s = pair_seq[p], h = pair_head[p];
    double* o = out + (size_t)p * d;
    if (s < 0 || s >= num_seqs || h < 0 || h >= hq) { bad = 1; continue; }
    int n = ctx_lens[s];
    const int32_t* table = tables + (size_t)s * max_blocks;
    int ok = (n >= 0) && ((n + bs - 1) / bs <= max_blocks);
    for (int j = 0; ok && j < (n + bs - 1) / bs; ++j) ok = table[j] >= 0 && table[j] < num_blocks;
    if (!ok) { bad = 1; for (int i = 0; i < d; ++i) o[i] = 0.0; continue; }
    double* scores = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!scores) return 1;
    decode_one(k_pool, v_pool, kv_dt, bs, hkv, d, q, act_dt, hq, table, n, s, h,
               sm_scale, k_scale, v_scale, o, scores, NULL);
    free(scores);
  }
  return bad;
}
