/*
 * pkv.h -- C ABI of libpkv.so: paged KV cache and paged decode attention on
 *          AMD Instinct MI355X (gfx950).
 *
 * What the library does, and where each part is described:
 *
 *   - A host block pool: the KV cache is cut into fixed-size blocks, each
 *     sequence owns a block table from logical block to physical block, a new
 *     block is taken only when the current one is full, finished sequences
 *     release their blocks ("PagedAttention Internals", sections "Fixed-Size
 *     KV Blocks", "The Block Table Map" and "Sharing And Dynamic Growth").
 *   - Prefix sharing: several sequences point at the same physical blocks and
 *     copy a block only when a sharer writes into it ("pagedattention" topic
 *     page, fourth paragraph and the comparison table's sharing row).
 *   - Device kernels: write new tokens' keys/values at the slots the pool
 *     handed out, copy blocks for copy-on-write, and decode attention that
 *     follows each sequence's block table to its keys and values ("The Block
 *     Table Map"; topic page, third paragraph).
 *
 * Conventions for every entry point
 *   - Return value: PKV_OK (0) or a negative PKV_ERR_* code.  On error,
 *     pkv_last_error() returns a message for the calling thread and the
 *     call has changed no pool state and launched no device work.
 *   - "host" pointers are ordinary CPU memory owned by the caller; "device"
 *     pointers are HIP device allocations owned by the caller (the library
 *     never allocates or frees device memory for caller data).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All device work is enqueued asynchronously on it, in call order.
 *   - A pool is not thread-safe: callers serialise calls on one pool.
 *   - No C++ exception crosses this boundary.
 *
 * Cache layout (the pages fix none; this library's choice):
 *   k_cache: [num_blocks, num_kv_heads, block_size, head_dim]   row-major
 *            (PKV_LAYOUT_HEAD_MAJOR), or
 *            [num_blocks, block_size, num_kv_heads, head_dim]   row-major
 *            (PKV_LAYOUT_TOKEN_MAJOR: all heads of a token together)
 *   v_cache: [num_blocks, num_kv_heads, head_dim, block_size]   row-major
 *   i.e. each block stores its keys as head_dim-contiguous rows and its values
 *   transposed (token-minor), so that the value product of decode attention
 *   reads contiguous runs of tokens of one head; the values keep that order in
 *   both layouts.  The transposed value tile departs from the plainest
 *   reading of a paged cache ([num_blocks, num_kv_heads, block_size,
 *   head_dim] for values as for keys): the matrix-core value product contracts
 *   over tokens and takes eight consecutive tokens of one head_dim element per
 *   lane, which this order turns into one 16-byte load straight from HBM.  Its
 *   cost: appending one token to a block stores each of its head_dim value
 *   elements into a different row of the tile.
 *   A block is one contiguous run of num_kv_heads * block_size * head_dim
 *   elements in each cache either way.  Slot s = block (s / block_size),
 *   offset (s % block_size).
 *   q, out:          [n_seqs, num_q_heads, head_dim]
 *   k_new, v_new:    [n_tokens, num_kv_heads, head_dim]
 *   block table:     int32 [n_seqs, max_blocks_per_seq], unused entries -1
 *   query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKV_OK                 0
#define PKV_ERR_INVALID_ARG   -1   /* malformed argument, NULL pointer, bad shape   */
#define PKV_ERR_NO_BLOCKS     -2   /* the free list cannot cover the request        */
#define PKV_ERR_BAD_SEQ       -3   /* unknown or already released sequence id       */
#define PKV_ERR_UNSUPPORTED   -4   /* shape / dtype combination not implemented     */
#define PKV_ERR_WORKSPACE     -5   /* workspace missing or too small                */
#define PKV_ERR_HIP           -6   /* a HIP runtime call or launch failed           */
#define PKV_ERR_CAPACITY      -7   /* an output buffer is too small                 */
#define PKV_ERR_DEVICE        -8   /* a kernel reported bad indices (see below)     */

/* device error bits reported by pkv_check_device_errors */
#define PKV_DEVERR_TABLE_ENTRY   1 /* block-table entry outside [0, num_blocks)     */
#define PKV_DEVERR_SLOT          2 /* cache_append slot >= num_blocks * block_size  */
#define PKV_DEVERR_COPY_PAIR     4 /* copy_blocks pair outside [0, num_blocks)      */
#define PKV_DEVERR_CONTEXT_LEN   8 /* context length < 0 or > table capacity       */
#define PKV_DEVERR_WORK_OVERFLOW 16/* more partitions than the workspace was sized */
#define PKV_DEVERR_PLAN          32/* planned decode: the workspace holds no plan for
                                       this sizing (nothing was computed)          */

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Order of the key cache inside a block (see "Cache layout" above). */
typedef enum { PKV_LAYOUT_HEAD_MAJOR = 0, PKV_LAYOUT_TOKEN_MAJOR = 1 } pkv_layout;

typedef struct pkv_pool pkv_pool;

typedef struct {
  int64_t num_blocks;
  int64_t free_blocks;
  int64_t used_blocks;      /* blocks with refcount > 0, each counted once      */
  int64_t allocated_slots;  /* used_blocks * block_size                         */
  int64_t live_tokens;      /* slots holding a token, each slot counted once    */
  int64_t wasted_slots;     /* allocated_slots - live_tokens                    */
  int64_t num_seqs;         /* live sequences                                   */
  double  fragmentation;    /* wasted_slots / allocated_slots (0 if none)       */
} pkv_stats;

/* ---- host block pool --------------------------------------------------- */

/* Create a pool of `num_blocks` blocks of `block_size` token slots: the KV
 * cache cut into equal fixed-size blocks, any of which may hold any
 * sequence's tokens ("PagedAttention Internals", "Fixed-Size KV Blocks";
 * "pagedattention" topic page, third paragraph).
 * `free_order` (host, num_blocks entries, may be NULL = 0..num_blocks-1) is
 * the initial free list, a permutation of the block ids; allocation takes its
 * head, release appends to its tail.  *out receives the handle.
 * Errors: INVALID_ARG (sizes <= 0, not a permutation, out NULL). */
int pkv_pool_create(int32_t num_blocks, int32_t block_size,
                    const int32_t* free_order, pkv_pool** out);

/* Destroy a pool (waits for its pending table uploads).  NULL is a no-op. */
int pkv_pool_destroy(pkv_pool* pool);

/* New empty sequence (no blocks, length 0).  Ids count up from 0 and are
 * never reused within a pool. */
int pkv_seq_create(pkv_pool* pool, int64_t* seq_out);

/* Append tokens: n_new[i] tokens to seqs[i], for i in call order
 * ("Fixed-Size KV Blocks": a block is taken when a token finds the current
 * one full; topic page fourth paragraph: copy-on-write on divergence).
 * For each token: if length % block_size == 0 take the free-list head as a
 * new block; else if the last block is shared (refcount > 1) take the head as
 * a private copy, report (old, new) in cow_pairs_out and drop one reference to
 * the old block; then slot = table[length / P] * P + length % P, length += 1.
 *   seqs        host int64[n_seqs], distinct live ids
 *   n_new       host int32[n_seqs], >= 0
 *   slot_mapping_out  host int32[slot_cap]: slots in call order
 *   cow_pairs_out     host int32[2 * cow_cap]: (src, dst) pairs, may be NULL
 *                     if cow_cap == 0
 *   n_cow_out   number of pairs written
 * The call is all-or-nothing.  Errors: BAD_SEQ, INVALID_ARG (duplicate id,
 * negative count), NO_BLOCKS, CAPACITY (sum(n_new) > slot_cap or more
 * copies than cow_cap). */
int pkv_seq_append_slots(pkv_pool* pool, const int64_t* seqs, const int32_t* n_new,
                         int32_t n_seqs, int32_t* slot_mapping_out, int64_t slot_cap,
                         int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out);

/* Fork: a new sequence sharing every block of `parent` (refcount + 1 each),
 * with the parent's length (topic page, fourth paragraph). */
int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t* child_out);

/* Release a sequence: a finished request gives its blocks back ("PagedAttention
 * Internals", "Sharing And Dynamic Growth"; a block shared with a fork stays
 * held by the others, "pagedattention" topic page, fourth paragraph).  Drops
 * one reference to each block in logical order; blocks reaching zero go to the
 * free-list tail in that order.  Errors: BAD_SEQ (unknown or released id; the
 * id stays unusable). */
int pkv_seq_free(pkv_pool* pool, int64_t seq);

/* Place an empty sequence on explicit free blocks `phys` (host int32[n_blocks],
 * logical order) holding `length` tokens, ceil(length / P) == n_blocks
 * ("The Block Table Map": logical blocks 0,1,2 at physical 8,3,11).  The
 * blocks leave the free list; the rest keep their order.
 * Errors: BAD_SEQ, INVALID_ARG (sequence not empty, block not free / out of
 * range / repeated, length mismatch). */
int pkv_seq_set_table(pkv_pool* pool, int64_t seq, const int32_t* phys,
                      int32_t n_blocks, int64_t length);

/* Copy a sequence's table (host int32[cap]) and length.  *n_out is the number
 * of blocks; CAPACITY if it exceeds cap (nothing written then). */
int pkv_seq_get_table(pkv_pool* pool, int64_t seq, int32_t* phys_out, int32_t cap,
                      int32_t* n_out, int64_t* len_out);

/* Occupancy and fragmentation ("inference-acceleration-pagedattention-vllm"
 * chapter: wasted = allocated but not holding a token, over allocated).
 * A shared block and its tokens count once. */
int pkv_pool_stats(pkv_pool* pool, pkv_stats* out);

/* State export for bit-exact checks: free list in order (host int32[num_blocks],
 * first *n_free_out entries valid) and every block's refcount (host
 * int32[num_blocks]).  Either output may be NULL. */
int pkv_pool_export(pkv_pool* pool, int32_t* free_order_out, int32_t* refcount_out,
                    int32_t* n_free_out);

/* Tokens each sequence holds in the same physical blocks as the one before it
 * in `seqs` (forks share blocks: "pagedattention" topic page, fourth
 * paragraph; "Sharing And Dynamic Growth"): for i >= 1, the leading table
 * entries seqs[i-1] and seqs[i] have in common times block_size, limited to
 * both lengths; entry 0 is 0.  The same counts pkv_block_table_upload writes
 * to d_shared_prev.
 *   shared_out            host int32[n_seqs], or NULL
 *   unshared_tokens_out   host, or NULL: sum over i of length_i - shared_i,
 *                         the tokens a decode that reads shared blocks once
 *                         per pack still streams (a sizing hint for
 *                         pkv_paged_attention_decode)
 * Host only.  Errors: INVALID_ARG, BAD_SEQ (nothing written then). */
int pkv_seq_shared_prefix(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs, int32_t* shared_out,
                          int64_t* unshared_tokens_out);

/* Bring a device block table, its context lengths and (optionally) a slot
 * mapping up to date with the pool ("The Block Table Map": the table records
 * each new block as the sequence grows):
 *   d_block_table   device int32[n_seqs * max_blocks_per_seq]; row i belongs
 *                   to seqs[i], entries beyond the sequence's blocks are -1
 *   d_context_lens  device int32[n_seqs]
 *   d_shared_prev   optional device int32[n_seqs] (NULL to skip): entry i >= 1
 *                   receives the number of leading tokens seqs[i] holds in
 *                   the same physical blocks as seqs[i-1] (forked sequences,
 *                   "Sharing And Dynamic Growth"): the common leading table
 *                   entries times block_size, limited to both lengths.  Entry
 *                   0 is 0.  pkv_paged_attention_decode reads it.
 *   slot_mapping / d_slot_mapping / n_slots: optional (host int32[n_slots] ->
 *                   device int32[n_slots]) copy of a slot mapping in the same
 *                   round; pass NULL/NULL/0 to skip.
 *   max_context_len_out, total_tokens_out: host outputs, may be NULL.
 *   flags  0: full upload.  The padded table is assembled on the host and
 *             copied through pool-owned pinned staging (double-buffered,
 *             reused only after the copy that last read it has completed).
 *          PKV_UPLOAD_INCREMENTAL: the caller asserts that d_block_table
 *             still holds what this pool last uploaded to that address (with
 *             the same max_blocks_per_seq), and that d_shared_prev, if it is
 *             the array passed last time, was not written since.  Rows that
 *             hold the same sequence as then, with no copy-on-write since,
 *             receive only their new entries; other rows are rewritten.
 *             Lengths, slots, entries and changed shared-token counts travel
 *             in the arguments of small patch kernels: no staging and no
 *             host-to-device copy.  Falls back to a full upload when the
 *             patch would be large (or nothing was uploaded there before).
 * The pool records, per device table address and row, what it wrote.  All
 * device work is enqueued on `stream`; the host may return before it runs.
 * Errors: BAD_SEQ, CAPACITY (a sequence has more than max_blocks_per_seq
 * blocks), INVALID_ARG (including unknown flags), HIP. */
#define PKV_UPLOAD_INCREMENTAL 1
int pkv_block_table_upload(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs,
                           int32_t max_blocks_per_seq, int32_t* d_block_table,
                           int32_t* d_context_lens, int32_t* d_shared_prev,
                           const int32_t* slot_mapping, int32_t* d_slot_mapping, int32_t n_slots,
                           int32_t* max_context_len_out, int64_t* total_tokens_out,
                           int32_t flags, void* stream);

/* ---- device kernels ---------------------------------------------------- */

/* Copy-on-write block copies: a sharer about to write into a block that
 * others still hold gets a private copy first ("pagedattention" topic page,
 * fourth paragraph and the comparison table's sharing row: shared blocks are
 * copied only where the sharers diverge; "PagedAttention Internals",
 * "Sharing And Dynamic Growth").  For each pair, every slot of block src (K
 * and V, all heads) is copied to block dst; both caches in the layout above
 * (any key layout: a block is one contiguous run either way).  `pairs` is HOST memory, int32[2*n_pairs]
 * as returned by pkv_seq_append_slots; the pairs travel in kernel arguments,
 * so no host-to-device copy is needed.  Enqueue before the cache_append that
 * writes into the new blocks.  Pairs outside [0, num_blocks) are skipped and
 * flagged (PKV_DEVERR_COPY_PAIR). */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs,
                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, pkv_dtype dtype, void* stream);

/* Write token i's keys/values (device k_new/v_new [n_tokens, Hkv, D]) into the
 * cache at slot d_slot_mapping[i] (device int32[n_tokens]) -- each generated
 * token goes into the current block ("Fixed-Size KV Blocks").  A negative
 * slot skips the token; a slot >= num_blocks * block_size is skipped and
 * flagged (PKV_DEVERR_SLOT).  Live slots must be distinct within one call.
 * k_layout is the key cache's order (PKV_LAYOUT_*; any other value is
 * INVALID_ARG); the decode and prefill calls that read the cache must pass
 * the same one.  Bit copy: no arithmetic on the values. */
int pkv_cache_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                     const int32_t* d_slot_mapping, int32_t n_tokens, int32_t num_blocks,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     pkv_dtype dtype, pkv_layout k_layout, void* stream);

/* Workspace bytes that pkv_paged_attention_decode needs for these arguments
 * (same meaning as there).  total_context_tokens may be -1 if unknown (a
 * looser bound is used). */
int pkv_decode_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t max_context_len, int64_t total_context_tokens,
                               int64_t unshared_context_tokens, pkv_dtype dtype,
                               size_t* bytes_out);

/* Paged decode attention ("The Block Table Map": attention follows each
 * sequence's table to its keys and values).  For sequence b, query head h,
 * G = Hq / Hkv, KV head g = h / G, L = d_context_lens[b]:
 *   out[b,h] = sum_{t<L} softmax_t(scale * q[b,h] . K_b[t,g]) V_b[t,g]
 * where K_b[t,g] = k_cache[table[b][t/P], g, t%P, :] and
 *       V_b[t,g] = v_cache[table[b][t/P], g, :, t%P].  L = 0 gives zeros.
 *   out, q           device [n_seqs, Hq, D], dtype
 *   k_cache, v_cache device, layout above, dtype
 *   d_block_table    device int32[n_seqs * max_blocks_per_seq]
 *   d_context_lens   device int32[n_seqs], 0 <= L <= max_blocks_per_seq * P
 *   d_shared_prev    NULL, or device int32[n_seqs]: entry b >= 1 is a number
 *                    of leading tokens that sequence b holds in the same
 *                    physical blocks as sequence b-1, as pkv_block_table_upload
 *                    writes it (entry 0 is ignored; values are clamped to
 *                    [0, min(L_b, L_{b-1})]).  The matrix-core kernel then
 *                    packs up to 16 / G consecutive sharing sequences and
 *                    reads the 32-token chunks they all share once for the
 *                    pack ("pagedattention" topic page, fourth paragraph:
 *                    forks share blocks): one unit per whole shared partition
 *                    plus one for a shared piece of the next.  With shared
 *                    lengths that are whole partitions the result is
 *                    bit-identical to a call with NULL and the same sizing
 *                    arguments (which fix T); otherwise the partition split by
 *                    the end of the shared tokens is summed as two partials.
 *                    A pack reads its shared tokens with cached loads (the
 *                    next pack over the same prefix finds them in L2); all
 *                    other keys and values stream with nontemporal loads.
 *                    The tables are not
 *                    compared: a count larger than the true shared prefix makes
 *                    that sequence read its predecessor's tokens (in bounds).
 *                    PKV_DECODE_SHARE=off ignores the array.  Runs of
 *                    more than 16 / G sharing sequences (block sizes of
 *                    8 to 64 tokens) form wide packs of up to 128 / G
 *                    sequences (at most 32) whose shared tokens are read
 *                    once for all their query rows as a dense matrix-core
 *                    product; those sum in another order, so the
 *                    bit-identity above holds for narrow packs only
 *                    (PKV_DECODE_WIDE=off keeps every pack narrow).
 *   max_context_len  >= every L (host knowledge, used for sizing)
 *   total_context_tokens  >= sum of L, or -1 if unknown (a bound from
 *                    n_seqs * max_context_len is used then).  It sizes the
 *                    work list: an underestimate that leaves the list too
 *                    small makes the plan run nothing, so no output is written
 *                    and PKV_DEVERR_WORK_OVERFLOW is set (the call itself
 *                    returns PKV_OK; pkv_check_device_errors reports it).
 *   unshared_context_tokens  sum of L minus the shared counts (as
 *                    pkv_seq_shared_prefix gives it), or -1 if unknown
 *                    (sizing only).  A value equal to total_context_tokens
 *                    (nothing shared) sizes the workspace without room for
 *                    packs, and the call then ignores d_shared_prev.
 *   scale            0 selects 1 / sqrt(head_dim) (rounded to fp32); otherwise
 *                    finite and positive
 *   workspace        device, >= pkv_decode_workspace_bytes(...) bytes,
 *                    caller-owned scratch for one call at a time: calls that
 *                    share a workspace must be ordered (same stream)
 * Work decomposition: each sequence is cut into partitions of T tokens (T a
 * power of two chosen from the batch's size, the same for every call with the
 * same sizing arguments); a workgroup of four waves takes one (partition, KV
 * head) unit and all query heads of that KV head, so every key/value byte is
 * read once.  A plan kernel orders the units longest first; sequences with
 * several partitions are combined by a merge kernel.  The summation order
 * depends only on logical positions, T and the wave split, so results do not
 * depend on where the blocks sit.  Arithmetic is fp32.  Kernel per shape:
 *   - bf16, head_dim 64/128, block_size 1, 2, 4, ..., 64, any G: matrix
 *     cores (score and value products as 16x16x32 bf16 MFMA, head group as N;
 *     G > 16 runs as ceil(G / 16) column sets of at most 16 heads, adjacent
 *     workgroups that each read the KV head's keys and values, with cached
 *     loads, and take no packs; such shapes need 16-byte aligned buffers);
 *   - fp32 (or bf16 shapes the matrix-core kernel does not take) with G <= 4,
 *     head_dim 64/128, block_size * element size a multiple of 16 bytes:
 *     vector ALU with DPP row reductions;
 *   - anything else with head_dim <= 256 and G <= 16: a generic vector-ALU
 *     kernel.
 * The environment variable PKV_DECODE_MATH = mfma | dpp | generic | valu
 * forces a kernel (UNSUPPORTED if the shape does not fit it); the matrix-core
 * and DPP kernels also need 16-byte aligned q, out and caches (otherwise the
 * generic kernel runs).  PKV_PARTITION_TOKENS forces T (rounded down to a
 * power of two, at least one chunk per wave); PKV_DECODE_SPLIT=off makes
 * every sequence a single partition.  Tuning overrides for measurement:
 * PKV_SPLIT_DIV (T is the largest power of two <= total tokens * Hkv /
 * (CUs * div); default 2 when n_seqs * Hkv >= 8 * CUs, else 4) and PKV_DECODE_WAVES=8 (matrix-core kernel: eight waves
 * per unit instead of four) change the summation order (results stay within
 * tolerance); PKV_MERGE_ELEMS = 1 | 2 | 4 (merge output elements per thread;
 * 3 counts as 2; widened where G * head_dim needs it) does not.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.  Bad table entries or
 * lengths are clamped in-bounds and flagged. */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* d_block_table,
                               const int32_t* d_context_lens, const int32_t* d_shared_prev,
                               int32_t n_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int64_t total_context_tokens, int64_t unshared_context_tokens,
                               float scale, pkv_dtype dtype,
                               pkv_layout k_layout, void* workspace, size_t workspace_bytes,
                               void* stream);

/* The decode split in two, for a step that attends several times over the
 * same block tables and lengths (one call per model layer: "The Block Table
 * Map" is per sequence, shared by every layer's cache).  pkv_decode_plan runs
 * only the plan kernel of pkv_paged_attention_decode: it reads d_context_lens
 * and d_shared_prev and writes the unit list into the workspace.
 * pkv_paged_attention_decode_planned then runs the partition and merge
 * kernels on that plan, any number of times; its result is bit-identical to
 * pkv_paged_attention_decode with the same arguments.
 *   Arguments: as pkv_paged_attention_decode.  The plan call takes the sizing
 *          arguments (n_seqs, head counts, head_dim, block_size,
 *          max_blocks_per_seq, max_context_len, total_context_tokens,
 *          unshared_context_tokens, dtype), d_context_lens, d_shared_prev
 *          (NULL or not) and the workspace; the planned call must pass the
 *          same values, the same workspace, and context lengths and shared
 *          counts unchanged since the plan ran (stream order).
 *   Checks: the plan records a stamp of its sizing in the workspace; a
 *          planned call whose sizing differs (or whose workspace holds no
 *          plan) computes nothing, leaves out unwritten and sets
 *          PKV_DEVERR_PLAN.  Changed lengths are not detected.  The planned
 *          call needs 16-byte aligned q, out and caches when the shape takes
 *          the matrix-core or DPP kernel (UNSUPPORTED otherwise).
 * Errors: as pkv_paged_attention_decode. */
int pkv_decode_plan(const int32_t* d_context_lens, const int32_t* d_shared_prev, int32_t n_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                    int64_t total_context_tokens, int64_t unshared_context_tokens,
                    pkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attention_decode_planned(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* d_block_table,
                                       const int32_t* d_context_lens,
                                       const int32_t* d_shared_prev, int32_t n_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int64_t total_context_tokens,
                                       int64_t unshared_context_tokens, float scale,
                                       pkv_dtype dtype, pkv_layout k_layout, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Decode without any device allocation, for callers that cannot allocate
 * (code under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): pkv_paged_attention_decode with every argument the same
 * except that the workspace is the library's own scratch, a static device
 * array of PKV_DECODE_SCRATCH_BYTES bytes per device (held until the process
 * ends).  The call allocates nothing.
 *   Limit: a batch whose pkv_decode_workspace_bytes(...) exceeds
 *          PKV_DECODE_SCRATCH_BYTES is refused with PKV_ERR_WORKSPACE.
 *   Sharing: every call on one device uses that device's one scratch; calls
 *          that may overlap on a device (several streams, several threads)
 *          race and must be serialised by the caller.  Nothing in the scratch
 *          needs to start at zero: each call writes what it reads.
 *   The first call on a device looks up the scratch's device address (a
 *   runtime symbol query, no allocation).
 * Errors: as pkv_paged_attention_decode, WORKSPACE as above, HIP if the
 * scratch address cannot be found. */
#define PKV_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* d_block_table,
                                       const int32_t* d_context_lens,
                                       const int32_t* d_shared_prev, int32_t n_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int64_t total_context_tokens,
                                       int64_t unshared_context_tokens, float scale,
                                       pkv_dtype dtype, pkv_layout k_layout, void* stream);

/* Paged prefill attention: causal attention of the newest tokens of each
 * sequence over everything it holds ("Fixed-Size KV Blocks": a prompt's
 * blocks are handed out as its tokens arrive; "The Block Table Map": the
 * kernel follows each table).  The new tokens must already be in the cache
 * (pkv_cache_append).  For sequence b, n_b = d_query_start[b+1] -
 * d_query_start[b] new tokens are the last n_b of its L_b = d_context_lens[b]
 * tokens; query row d_query_start[b] + i (position L_b - n_b + i) attends keys
 * 0 .. L_b - n_b + i:
 *   out[row,h] = sum_{t <= L_b-n_b+i} softmax_t(scale * q[row,h] . K_b[t,g]) V_b[t,g]
 * with K_b / V_b, g = h / G as in pkv_paged_attention_decode.
 *   out, q            device [total new tokens, Hq, D], bf16
 *   d_query_start     device int32[n_seqs + 1], nondecreasing, starting at 0
 *   d_context_lens    device int32[n_seqs], n_b <= L_b <= max_blocks_per_seq * P
 *   max_query_len     >= every n_b (host knowledge, sizes the grid); a
 *                     sequence with more new tokens has its rows past
 *                     max_query_len left unwritten and flags
 *                     PKV_DEVERR_CONTEXT_LEN
 *   scale             as in pkv_paged_attention_decode (0 = 1 / sqrt(head_dim))
 * Both products run on matrix cores; key/value chunks of 64 tokens are staged
 * once per workgroup in LDS and shared by a tile of queries: 128 query rows,
 * 128 / GW tokens of GW heads, GW the largest of 8, 4, 2, 1 dividing G.
 * Supported: bf16, head_dim 64 / 128, block_size a power of two from 8 to 256,
 * any G, fewer than 2^24 workgroups (n_seqs x Hkv x G / GW x query tiles),
 * 16-byte aligned q, out and caches.  A sequence whose length
 * is out of range is skipped (its rows unwritten) and flagged
 * (PKV_DEVERR_CONTEXT_LEN); bad table entries are clamped and flagged.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* d_block_table,
                                const int32_t* d_context_lens, const int32_t* d_query_start,
                                int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_query_len, float scale,
                                pkv_dtype dtype, pkv_layout k_layout, void* stream);

/* Synchronise `stream`, then read and clear the current device's error bits
 * (PKV_DEVERR_*) into *flags_out.  Returns PKV_ERR_DEVICE if any bit was set. */
int pkv_check_device_errors(void* stream, int32_t* flags_out);

/* Message for the last non-zero status returned on this thread ("" if none).
 * The pointer stays valid until the thread's next failing call. */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
