/*
 * pa.h — paged KV-cache decode for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels and a host-side block allocator.
 * All device entry points are asynchronous and stream-ordered; all host
 * argument checks are synchronous and never read device memory.
 *
 * Citation key (web page title, then section):
 *   [F55 §x]  "KV 缓存与分页注意力" (world.lapla.si, plate F55), section x
 *   [AIF x]   "KV 缓存" (aiinfact.com topic page), part x
 *   [IPX §x]  "读懂PagedAttention：vLLM的KV缓存与GPU显存管理" (iplexlaw.co.kr),
 *             sub-heading x
 *
 * ---------------------------------------------------------------------------
 * Memory layout of the pool (this library's choice; the pages only say that
 * storing per layer and per head performs like storing all layers together
 * [F55 §模型省略了什么]):
 *
 *   k_cache, v_cache: each [num_blocks][num_kv_heads][block_size][head_dim]
 *   element (b, h, slot, i) at ((b * num_kv_heads + h) * block_size + slot)
 *   * head_dim + i.  One (block, head) tile is contiguous.
 *
 * Block tables: int32 [num_seqs][max_blocks_per_seq], entry j = physical
 * block of logical block j [F55 §块表].  Per-entry fill counts are implied by
 * one context length per sequence: only the last block can be partial
 * [F55 §块表], so entry j holds min(block_size, ctx - j * block_size) tokens.
 * Unused entries may hold anything (conventionally -1).
 *
 * context_lens: int32 [num_seqs], tokens of each sequence INCLUDING the token
 * appended in the current step (the new token attends to itself, because its
 * K/V are appended before attention [AIF level-3 script]).
 *
 * Ownership: the caller owns every device buffer (pool, q, new K/V, output,
 * tables, lengths, workspace) and the stream; the library allocates no device
 * memory in these calls and keeps no device pointer between calls.  The
 * allocator object is the only library-owned state.
 *
 * Graph capture: the decode, append, prompt-write and block-copy calls only
 * launch kernels on the given stream (no memset, no allocation, no host
 * synchronisation), so a stream being captured into a HIP graph records
 * them, and the graph can be replayed; the workspace's arrival counters are
 * back at zero after every launch.  Timing events (pa_timing_enable) are for
 * measurement and should be off while capturing.
 *
 * Supported shapes: head_dim in {32, 64, 128}; block_size a power of two in
 * 1..64; num_q_heads a multiple of num_kv_heads; kv dtype f32, f16 or
 * FP8 E4M3; activation dtype f16 (f16 or FP8 pool) or f32 (f32 or FP8
 * pool).  Query heads sharing a KV head go to the matrix-core kernel only
 * with f16 activations; with f32 ones every head is decoded on its own.
 * Shared-prefix decode takes f16 activations only.
 * ---------------------------------------------------------------------------
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

/* Every entry point is noexcept for C++ callers: no exception leaves the
 * library.  A host memory allocation that fails inside a call returns
 * PA_ERR_HOST_MEMORY, and the call changes nothing (the allocator's state is
 * as before it). */
#ifdef __cplusplus
#define PA_NOEXCEPT noexcept
#else
#define PA_NOEXCEPT
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,
  PA_ERR_OUT_OF_BLOCKS = 2,
  PA_ERR_UNKNOWN_SEQ = 3,
  PA_ERR_WORKSPACE_TOO_SMALL = 4,
  PA_ERR_UNSUPPORTED = 5,
  PA_ERR_HIP = 6,
  PA_ERR_HOST_MEMORY = 7
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* Describes caller-owned device memory; the library keeps no pointer. */
typedef struct {
  void* k_cache;           /* device, [num_blocks][num_kv_heads][block_size][head_dim] */
  void* v_cache;           /* device, same shape and dtype */
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t kv_dtype;        /* pa_dtype */
  /* FP8 pools only: stored byte = e4m3_rne_saturate(f32(x) * inv_scale) with
   * one binary32 multiply; value read back = e4m3 value * scale.  One scale
   * per tensor (K and V separately).  Ignored for f32/f16 pools.  The pages
   * say only that the cache may keep one byte per number [F55 §后来的做法]. */
  float k_scale, v_scale, k_inv_scale, v_inv_scale;
} pa_kv_cache;

/* ============================ device operations ============================ */

/*
 * pa_kv_append — store the new token's K and V of every sequence into the
 * free slot of its last block [F55 §一次写一个词元, §块表];
 * [IPX §分离逻辑顺序与实际存储位置] (later tokens go into the last block's
 * free slot).
 *
 *   pos = context_lens[s] - 1, blk = block_tables[s][pos / block_size],
 *   k_cache[blk][h][pos % block_size][:] = k_new[s][h][:] for h < num_kv_heads
 *   (same for V); FP8 pools quantise as described above.
 *
 * k_new, v_new: device, [num_seqs][num_kv_heads][head_dim] of dtype act.
 * block_tables, context_lens: device (layouts above).  Sequences whose
 * context length is < 1, whose position needs an entry past
 * max_blocks_per_seq, or whose block id is outside [0, num_blocks) write
 * nothing.  Precondition: no two sequences target the same (block, slot) —
 * the allocator guarantees this by never letting a shared block be written
 * (copy-on-write, pa_seq_append_slot + pa_copy_blocks).  Bit-exact for
 * f32/f16 pools.  Re-running the call with the same arguments is idempotent.
 */
pa_status pa_kv_append(const pa_kv_cache* cache, const void* k_new, const void* v_new, int32_t act,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                       int32_t max_blocks_per_seq, void* stream) PA_NOEXCEPT;

/*
 * pa_kv_write_prompt — the prompt phase: a sequence's whole prompt K/V are
 * computed at once and stored into the blocks allocated for it
 * [F55 §一次写一个词元]; [IPX §分离逻辑顺序与实际存储位置] (blocks for the input
 * are allocated first).
 *
 * Sequence s stores token rows src_row[s] .. src_row[s] + count[s] - 1 of
 * k_src / v_src ([total_rows][num_kv_heads][head_dim], dtype act) at logical
 * positions start_pos[s] .. start_pos[s] + count[s] - 1, through its table.
 * src_row: device int64 [num_seqs]; start_pos, count: device int32
 * [num_seqs]; max_count >= every count[s] sizes the launch (tokens past
 * max_count are not written).  Out-of-range positions or block ids write
 * nothing.  Same precondition on distinct targets as pa_kv_append.
 */
pa_status pa_kv_write_prompt(const pa_kv_cache* cache, const void* k_src, const void* v_src, int32_t act,
                             const int64_t* src_row, const int32_t* start_pos, const int32_t* count,
                             const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                             int32_t max_count, void* stream) PA_NOEXCEPT;

/*
 * pa_copy_blocks — the copy of copy-on-write: before a sequence writes into
 * a block other sequences still reference, the block is copied and the
 * write goes to the copy [F55 §常见问题 (copy-on-write)];
 * [IPX §同一提示生成两个回答的假想例子].
 *
 * src_dst_pairs: device int32 [n][2] = (source block, destination block);
 * every KV head and slot of the block is copied, K and V.  Bit-exact.  Pairs
 * with an id outside [0, num_blocks) are skipped.  Destinations must be
 * distinct and no destination may be a source.
 */
pa_status pa_copy_blocks(const pa_kv_cache* cache, const int32_t* src_dst_pairs, int32_t n, void* stream) PA_NOEXCEPT;

/*
 * pa_swap_blocks — the copy of preemption by swapping: a preempted
 * sequence's blocks are moved to host memory and moved back when it resumes
 * [F55 §放不下的时候] (see pa_seq_swap_out / pa_seq_swap_in).
 *
 * host_k, host_v: host memory the device can access (pinned, e.g.
 * hipHostMalloc), each [n][num_kv_heads][block_size][head_dim] of the pool
 * dtype; entry i holds block block_ids[i].  block_ids: device int32 [n].
 * direction PA_SWAP_OUT copies pool -> host, PA_SWAP_IN host -> pool; every KV
 * head and slot, K and V, bit-exact.  The kernel moves 16-byte chunks over
 * the host link directly, so small blocks cost no more per byte than large
 * ones.  Ids outside [0, num_blocks) are skipped; swap-in targets must be
 * distinct.  Host buffers the runtime does not know as pinned give
 * PA_ERR_INVALID_ARGUMENT before any launch.  Asynchronous on `stream`: the
 * host buffers must stay allocated, and untouched by the host, until it
 * completes.
 */
typedef enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 } pa_swap_direction;
pa_status pa_swap_blocks(const pa_kv_cache* cache, void* host_k, void* host_v, const int32_t* block_ids, int32_t n,
                         int32_t direction, void* stream) PA_NOEXCEPT;

/*
 * pa_decode_workspace_size — bytes of device workspace pa_decode and
 * pa_decode_step need for split-context partial results: an int32 arrival
 * counter per (sequence, query head), padded to 256 bytes, then fp32
 * (max, sum) and an unnormalised vector per (sequence, query head,
 * partition).  0 when every context fits one partition (512 tokens).
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                int32_t max_context_len) PA_NOEXCEPT;

/*
 * pa_decode — one generation step's attention: for every sequence s and
 * query head h, the query attends over all context_lens[s] cached keys and
 * values of its KV head, fetched block by block through the block table
 * (blocks need not be adjacent) in logical token order [F55 §块表];
 * [IPX §分离逻辑顺序与实际存储位置].  Attention is the scaled dot-product
 * softmax attention the pages cite, with the 1/sqrt(d) scale passed as
 * sm_scale [AIF level-3 account table]:
 *
 *   s_t = sm_scale * q[s][h] . K_t,   out[s][h] = sum_t softmax(s)_t * V_t
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (grouped- and
 * multi-query attention share one KV head among contiguous query heads
 * [F55 §后来的做法]).  q, out: device [num_seqs][num_q_heads][head_dim] of
 * dtype act; fp32 accumulation; the output is rounded to act (nearest even).
 * Contexts longer than one partition are split (512 tokens for the per-head
 * kernel; for the grouped kernel a multiple of 512 chosen per launch, so
 * that its workgroups fit the GPU at once where they can); the partitions'
 * (max, sum, vector) partial results are merged exactly (the online softmax
 * gives the same result [F55 related plate F51]): by a second, small launch
 * on the same stream for the per-head kernel (MHA, and f32 activations),
 * and in the same launch, by the last partition of a (sequence, head group)
 * to finish, for the grouped kernel (GQA/MQA with f16 activations).
 *
 * max_context_len must be >= every context_lens[s] and at most 524,288
 * (1024 partitions; larger values return PA_ERR_UNSUPPORTED); workspace must hold
 * pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len)
 * bytes (NULL allowed when that size is 0).  The workspace must be
 * zero-filled before its first use.  It begins with the arrival counters,
 * one int32 per (sequence, query head) row, in a region sized by
 * workspace_bytes for the most rows such a workspace could serve; the
 * partials follow it.  Every completed call leaves its counters at zero, so
 * a workspace can be reused call after call with any sizes it is large
 * enough for (batches that grow and shrink included), provided every call on
 * it passes the same workspace_bytes.  workspace_bytes is the size of the
 * buffer itself and must not overstate it: the layout is derived from it.  Calls that overlap in time must not
 * share a workspace.  A context length of 0 yields zeros.  A
 * sequence whose context exceeds max_context_len or
 * max_blocks_per_seq * block_size, or whose table holds a block id outside
 * [0, num_blocks), yields NaN for every head (and reads nothing out of range).
 */
pa_status pa_decode(const pa_kv_cache* cache, const void* q, void* out, int32_t act, int32_t num_q_heads,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_blocks_per_seq, int32_t max_context_len, float sm_scale,
                    void* workspace, size_t workspace_bytes, void* stream) PA_NOEXCEPT;

/*
 * pa_decode_step — the whole generation step in one launch: the result of
 * pa_kv_append(cache, k_new, v_new, ...) followed by pa_decode(...) with the
 * same arguments — the new token's K/V are stored into the free slot of the
 * last block [F55 §一次写一个词元, §块表] and attended to — without a second
 * pass over memory: the workgroups that hold the new token take it from
 * k_new/v_new directly, and one of them stores it.  Same arguments, layouts,
 * workspace contract and error behaviour as the two calls; the pool ends
 * bit-identical to what pa_kv_append writes.  Copy-on-write copies
 * (pa_copy_blocks) must be issued before it on the same stream.
 */
pa_status pa_decode_step(const pa_kv_cache* cache, const void* q, const void* k_new, const void* v_new,
                         void* out, int32_t act, int32_t num_q_heads, const int32_t* block_tables,
                         const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                         int32_t max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
                         void* stream) PA_NOEXCEPT;

/*
 * pa_decode_step_noalloc — pa_decode_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  Same arguments, result and pool contents as
 * pa_decode_step, without the workspace: the split-context partials and
 * arrival counters live in a scratch array inside the library, 32 MiB on
 * each GPU it runs on (a file-scope device array, held until the process
 * ends).  The call allocates nothing and calls no allocating routine.
 *
 * A call whose pa_decode_workspace_size(num_seqs, num_q_heads, head_dim,
 * max_context_len) exceeds 32 MiB returns PA_ERR_WORKSPACE_TOO_SMALL before
 * anything else (pa_decode_step takes a workspace of any size).  The first
 * call on a device that needs the scratch clears it with a kernel on
 * `stream`, ordered before that call's decode (if `stream` is being captured,
 * the clear is captured too and the next call outside capture clears again);
 * every completed call leaves the counters at zero.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU race and
 * give undefined results, whatever their streams; the caller orders them.
 */
pa_status pa_decode_step_noalloc(const pa_kv_cache* cache, const void* q, const void* k_new, const void* v_new,
                                 void* out, int32_t act, int32_t num_q_heads, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                                 int32_t max_context_len, float sm_scale, void* stream) PA_NOEXCEPT;

/*
 * pa_decode_shared_prefix — decode (and, with k_new/v_new non-NULL, the
 * append of pa_decode_step) for batches whose sequences share a prompt
 * prefix in the same physical blocks (a fork, a common system prompt, a
 * prefix-cache hit) [F55 §后来的做法, §常见问题];
 * [IPX §同一提示生成两个回答的假想例子].  The result is the same attention as
 * pa_decode over each sequence's whole context; only the work differs.
 * Sequences [group_start[g], group_start[g+1]) (host int32, num_groups + 1
 * entries, non-decreasing, within [0, num_seqs]) hold the same first
 * group_shared_blocks[g] (host int32) table entries.  A prefix pass reads
 * those blocks once per KV head, through the table of the group's first
 * sequence, for all of the group's (sequence, query head) rows on the matrix
 * cores, and leaves per-row partials; the decode covers each sequence's own
 * tokens, and both are merged exactly.  The grouped decode runs after the
 * prefix pass and starts from its partials.  The per-head decode over an
 * FP8 pool with blocks of at least 16 tokens (and of at least
 * 64 / (head_dim / 16)) runs in the same launch as the prefix pass, whose
 * workgroups come last, and a merge launch follows; the slot of a token
 * appended by that launch must not lie in a shared block, which copy on
 * write guarantees (pa_seq_append_slot never leaves a shared block as the
 * write target).  Otherwise the prefix pass, the per-head decode and the
 * merge are three launches.  The caller guarantees the sharing: entries
 * past the first sequence's are not read for the shared range.  A sequence whose context is shorter than its group's shared
 * tokens, or (when appending) whose new token would fall inside them, gets
 * NaN output.  At most 16 groups; sequences outside every group decode
 * normally.  Needs f16 activations and an f16 or FP8 pool when any group
 * shares blocks (else PA_ERR_UNSUPPORTED).  Workspace: at least
 * pa_decode_shared_workspace_size(num_seqs, num_q_heads, head_dim,
 * max_context_len, the largest group_shared_blocks * block_size) bytes,
 * zero-filled before first use and reusable as pa_decode's.
 */
pa_status pa_decode_shared_prefix(const pa_kv_cache* cache, const void* q, const void* k_new, const void* v_new,
                                  void* out, int32_t act, int32_t num_q_heads, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                                  int32_t max_context_len, float sm_scale, int32_t num_groups,
                                  const int32_t* group_start, const int32_t* group_shared_blocks, void* workspace,
                                  size_t workspace_bytes, void* stream) PA_NOEXCEPT;
size_t pa_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t max_shared_tokens) PA_NOEXCEPT;

/* ============================== host allocator ============================= */
/*
 * The block allocator keeps the bookkeeping of [F55 §像内存分页, §块表,
 * §放不下的时候] and [IPX §同一提示生成两个回答的假想例子]:
 *   - equal-size physical blocks in one pool, one table per sequence;
 *   - a block is taken only when the sequence's earlier blocks are full;
 *   - first come, first served, and a request is met whole or not at all
 *     (a failing call changes nothing);
 *   - a finished sequence returns its blocks;
 *   - forks share blocks with reference counts; a write into a partially
 *     filled block that others still reference copies it first.
 * Free list: first in, first out (pop the head, freed blocks join the tail in
 * logical order).  Not thread-safe: one owner at a time.  Sequence ids are
 * any non-negative int32.
 */
typedef struct pa_allocator pa_allocator;

typedef struct {
  int32_t num_blocks;
  int32_t num_free;
  int32_t num_shared;       /* blocks with reference count > 1 */
  int32_t num_seqs;
  int64_t tokens_held;      /* distinct (block, slot) pairs holding a token */
  int64_t slots_allocated;  /* blocks in use * block_size */
} pa_allocator_stats;

/* free_order: host int32 [num_blocks], a permutation giving the initial free
 * list order (NULL = 0, 1, ..., num_blocks - 1). */
pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                              pa_allocator** out) PA_NOEXCEPT;
void pa_allocator_destroy(pa_allocator* a) PA_NOEXCEPT;
int32_t pa_allocator_num_free(const pa_allocator* a) PA_NOEXCEPT;
/* A new sequence holding num_tokens (>= 0) tokens: ceil(n / block_size) blocks. */
pa_status pa_seq_allocate(pa_allocator* a, int32_t seq, int32_t num_tokens) PA_NOEXCEPT;
/*
 * Automatic prefix caching [F55 §后来的做法]: allocate a sequence whose
 * prompt is tokens[0, num_tokens) (host int32 token ids), reusing blocks
 * that already hold the same beginning.  Every full block is keyed by its
 * tokens and by everything before it, through a chained 64-bit hash (the
 * FNV-1a hash of the previous block's key and the block's tokens).  A
 * lookup also compares the stored tokens and previous key.  The same
 * tokens at another position are another key.  Reuse stops at the first
 * full block that misses.  A reused block gains one reference (one that
 * had been freed is taken back off the free list); the other blocks are
 * new, and the new full ones become keys unless the key is already held.
 * A block keeps its key after its last holder frees it, and loses it when
 * the free list hands it out for other content (least recently freed
 * first).  *num_cached_tokens receives the number of leading tokens whose
 * K/V the reused blocks already hold: the caller writes only
 * [*num_cached_tokens, num_tokens) (pa_kv_write_prompt with that start).
 * This saves prompt processing; it does not change decode.  All or none:
 * PA_ERR_OUT_OF_BLOCKS changes nothing.  Blocks filled later by appends
 * are not keyed.
 */
pa_status pa_seq_allocate_cached(pa_allocator* a, int32_t seq, const int32_t* tokens, int32_t num_tokens,
                                 int32_t* num_cached_tokens) PA_NOEXCEPT;
/* Number of blocks that currently hold a prefix-cache key (-1 if a is NULL). */
int32_t pa_prefix_cache_size(const pa_allocator* a) PA_NOEXCEPT;
/* child shares every block of parent (reference counts + 1). */
pa_status pa_seq_fork(pa_allocator* a, int32_t parent, int32_t child) PA_NOEXCEPT;
/* Reserve the slot of one more token.  *cow_src / *cow_dst receive the block
 * copy the caller must perform (pa_copy_blocks) before writing, or -1 / -1. */
pa_status pa_seq_append_slot(pa_allocator* a, int32_t seq, int32_t* cow_src, int32_t* cow_dst) PA_NOEXCEPT;
/* Release the sequence: reference counts - 1, unreferenced blocks are freed
 * (a swapped-out sequence is simply forgotten). */
pa_status pa_seq_free(pa_allocator* a, int32_t seq) PA_NOEXCEPT;
/*
 * Preemption by swapping: when blocks run out, the latest arrival gives up
 * all of its blocks, which may be moved to host memory and moved back when
 * it resumes [F55 §放不下的时候].
 * pa_seq_swap_out releases every block of a resident sequence (reference
 * counts - 1, unreferenced blocks join the free list; shared blocks stay with
 * their other holders) and keeps its context length; block_ids (host, room
 * for cap entries) receives its former blocks in logical order, whose K/V the
 * caller copies out with pa_swap_blocks(PA_SWAP_OUT) before any later write
 * can reuse them (issuing the copy first on the same stream suffices).
 * pa_seq_swap_in takes ceil(ctx / block_size) fresh blocks, all or none
 * (PA_ERR_OUT_OF_BLOCKS changes nothing), and returns them in logical order
 * for pa_swap_blocks(PA_SWAP_IN).  Both set *num_blocks to the number of
 * blocks and fail with PA_ERR_INVALID_ARGUMENT, changing nothing, when cap is
 * smaller.  A swapped-out sequence keeps its place in arrival order but is
 * not a preemption candidate; pa_seq_get, append and fork do not see it.
 */
pa_status pa_seq_swap_out(pa_allocator* a, int32_t seq, int32_t* block_ids, int32_t cap, int32_t* num_blocks) PA_NOEXCEPT;
pa_status pa_seq_swap_in(pa_allocator* a, int32_t seq, int32_t* block_ids, int32_t cap, int32_t* num_blocks) PA_NOEXCEPT;
/* Copy the table (up to cap entries) and report its length and context. */
pa_status pa_seq_get(const pa_allocator* a, int32_t seq, int32_t* block_ids, int32_t cap,
                     int32_t* num_blocks, int32_t* context_len) PA_NOEXCEPT;
/* Host int32 tables [n][max_blocks_per_seq] (padding -1) and lengths [n]. */
pa_status pa_export_tables(const pa_allocator* a, const int32_t* seqs, int32_t n,
                           int32_t max_blocks_per_seq, int32_t* tables_out, int32_t* context_lens_out) PA_NOEXCEPT;
int32_t pa_block_refcount(const pa_allocator* a, int32_t block) PA_NOEXCEPT;
pa_status pa_allocator_get_stats(const pa_allocator* a, pa_allocator_stats* out) PA_NOEXCEPT;
/* The sequence to preempt first when blocks run out: the latest arrival
 * among those holding blocks [F55 §放不下的时候]; -1 if none. */
int32_t pa_latest_arrival(const pa_allocator* a) PA_NOEXCEPT;

/*
 * The toy machine's arrival simulator [F55 §实验台], run over this
 * allocator.  Sequence i arrives at round arrivals[i] and writes one token
 * per round until it has lengths[i] tokens, then leaves.  Each round:
 *   1. Growth: running sequences take this round's slot, earliest arrival
 *      first.  When no block is free, the latest arrival (pa_latest_arrival)
 *      is preempted by swapping [F55 §放不下的时候]: it keeps its tokens
 *      and rejoins the queue; if it is the sequence asking, that one writes
 *      nothing this round.
 *   2. Admission, only in a round without preemption: queued sequences
 *      strictly first come, first served (arrival round, then index) while
 *      the head's whole need, ceil((tokens + 1) / block_size) blocks, is
 *      free; the rest wait.
 *   3. Readout: running sequences, tokens held, and slots reserved (blocks
 *      in use x block_size).
 *   4. Departure of finished sequences.
 * The page's row option (each sequence reserves the maximum length on
 * arrival) is block_size = max length with floor(slots / max length) blocks.
 * Readouts: the most sequences running in one round; utilisation, the mean
 * over rounds that reserve anything of held / reserved; the rounds until
 * all have left; preemptions.  trace (host, NULL allowed) receives up to
 * trace_cap rounds of (running, held, reserved) int32 triples.
 * PA_ERR_INVALID_ARGUMENT for lengths < 1, arrivals < 0, or a sequence
 * longer than the whole pool.  Host only; allocates its own allocator.
 */
typedef struct {
  int32_t max_concurrent;
  int32_t rounds;
  int32_t preemptions;
  int32_t reserved0;
  double utilisation;
} pa_arrival_readout;
pa_status pa_simulate_arrivals(int32_t num_blocks, int32_t block_size, const int32_t* arrivals,
                               const int32_t* lengths, int32_t n, pa_arrival_readout* out, int32_t* trace,
                               int32_t trace_cap) PA_NOEXCEPT;

/* ================================ utilities ================================ */

const char* pa_status_str(pa_status s) PA_NOEXCEPT;
/* Detail of the last non-OK status returned on this thread (never NULL). */
const char* pa_last_error(void) PA_NOEXCEPT;

/*
 * Kernel timing for measurement: while enabled, every pa_decode and
 * pa_decode_step records HIP events around its kernel, on the stream the
 * kernel runs on.  pa_timing_read synchronises those events and returns the
 * summed milliseconds and the number of launches since the last read, then
 * resets the sums.  Events are created on enable (up to 4096 launches are
 * kept between reads) and destroyed on disable.  They carry no system-scope
 * memory fence, so they perturb the timed launches as little as possible;
 * they order nothing for the caller.  Not thread-safe.
 */
pa_status pa_timing_enable(int32_t on) PA_NOEXCEPT;
pa_status pa_timing_read(double* decode_ms, int32_t* decode_launches) PA_NOEXCEPT;

/*
 * pa_read_probe — measurement only: the rate at which this GPU reads the
 * pools, without any of the decode's arithmetic, so that the decode kernels
 * can be compared with what their access pattern allows.  mode 0 runs the
 * per-head decode kernel with its arithmetic compiled out, treating every KV
 * head as one query head: the same grid, table staging and 16-byte
 * non-temporal K and V loads, every sequence's rows read through its block
 * table in logical order [F55 §块表] (entries outside [0, num_blocks) make
 * that sequence read nothing).  mode 1 reads both whole pools from start to
 * end, each workgroup one contiguous span (tables and lengths are ignored).
 * Each lane folds its loaded words with XOR and writes its fold to one word
 * of sink (device, uint32 [1024], caller-owned) only if the fold equals
 * 0x9E3779B9, so the loads cannot be dropped; sink words are left as they
 * were or set to that value, and mean nothing.  Asynchronous on stream.
 */
pa_status pa_read_probe(const pa_kv_cache* cache, const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t max_blocks_per_seq, int32_t max_context_len, int32_t mode,
                        uint32_t* sink, void* stream) PA_NOEXCEPT;

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
