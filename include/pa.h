/*
 * pa.h -- C ABI of the paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * The KV cache of every sequence lives in fixed blocks of 16 token slots that
 * sit anywhere in one pool; a per-sequence block table maps the sequence's
 * logical blocks to physical ones, a block is taken only when the sequence
 * needs it and returns to the pool when released, and blocks of a common
 * prompt are shared by reference count and copied when one sharer writes
 * ("PagedAttention for the professional: how vLLM serves 2.7x more requests on
 * the same H100", sections "Beginner's example: library shelves" and "The
 * scientific explanation"; "KV Cache and PagedAttention: why your LLM server
 * slows down", sections "How PagedAttention fixes this" and "How does
 * PagedAttention work?").  Each decode step attends one new query per head
 * against the cached K/V of its sequence under grouped-query attention ("KV
 * Cache for the intermediate: why long context eats the GPU and how to cut it
 * 4x", sections "Precise scientific definition" and "Grouped Query Attention").
 *
 * Conventions
 *   - Every call returns pa_status: 0 = PA_OK, negative = error.  Nothing
 *     throws across this boundary.
 *   - Pool calls are host-only and touch no device memory.  A pool is not
 *     thread-safe; one thread owns it.
 *   - Device calls take device pointers owned by the caller and enqueue work on
 *     `stream` (a hipStream_t; NULL = the default stream).  They return as soon
 *     as the work is queued.  Arguments are checked on the host before anything
 *     is launched; an argument error launches nothing.  PA_ERR_DEVICE reports a
 *     launch failure.
 *   - q, caches and out share one dtype.  All arithmetic accumulates in fp32.
 *
 * Cache layout (per cache tensor, `num_blocks` blocks of Hkv * 16 * D elements):
 *   K: [num_blocks][Hkv][D / X][16][X], X = 16 / element bytes (8 for bf16 and
 *      fp16, 4 for fp32): token row r, dimension d of block b, head h is at
 *      ((b * Hkv + h) * (D / X) + d / X) * 16 * X + r * X + d % X.
 *   V: [num_blocks][Hkv][D][16]: at ((b * Hkv + h) * D + d) * 16 + r.
 *   Slot s is row s % 16 of block s / 16.
 *
 * INT8 cache layout (PA_I8; int8 codes, D a multiple of 64): each (block,
 * head) is D * 16 bytes at (b * Hkv + h) * D * 16, made of D / 64 slabs of
 * 1 KiB; in slab d / 64:
 *   K: token r, dimension d at ((d / 16) % 4 * 16 + r) * 16 + d % 16;
 *   V: token r, dimension d at ((r / 4) * 16 + d % 16) * 16 + (d / 16) % 4 * 4 + r % 4.
 * Either way one 16-byte load per lane of a 64-lane wave reads a contiguous
 * KiB that feeds the matrix cores directly.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
#define PA_OK 0
#define PA_ERR_INVALID_ARG (-1)   /* bad shape, pointer, position or size */
#define PA_ERR_OUT_OF_BLOCKS (-2) /* the pool cannot serve the request; nothing changed */
#define PA_ERR_BAD_BLOCK (-3)     /* block id out of range or not held */
#define PA_ERR_UNSUPPORTED (-4)   /* valid request the library does not implement */
#define PA_ERR_DEVICE (-5)        /* HIP launch or runtime error */
#define PA_ERR_WORKSPACE (-6)     /* workspace missing or too small */
#define PA_ERR_HOST_MEMORY (-7)   /* a host allocation failed; nothing changed */

/* Storage dtype of q, the caches and out. */
typedef int32_t pa_dtype;
#define PA_F32 0
#define PA_F16 1
#define PA_BF16 2
#define PA_I8 3 /* codes of an INT8 cache: pa_copy_blocks and the *_int8 calls */

#define PA_BLOCK_SIZE 16

/* partition_size values of pa_paged_attention_decode besides a positive
 * multiple of 16 */
#define PA_PARTITION_NONE 0    /* one pass over each whole sequence, no partials */
#define PA_PARTITION_AUTO (-1) /* the library picks */

/* Short English text of a status code (static storage). */
const char* pa_status_string(pa_status status);

/* ---------------------------------------------------------------------------
 * Block pool (host).  Holds block ids and reference counts only -- never device
 * memory: the caller owns the cache tensors the ids index.
 * ------------------------------------------------------------------------- */
typedef struct pa_pool pa_pool;

typedef struct {
  int32_t num_blocks;
  int32_t num_free;   /* reference count 0 */
  int32_t num_used;   /* reference count >= 1 */
  int32_t num_shared; /* reference count >= 2 */
  int64_t copies;     /* copy-on-write pairs emitted so far */
  int32_t num_cached;    /* blocks entered in the prefix cache (held or not) */
  int32_t num_evictable; /* cached blocks at count 0 (counted in num_free) */
  int64_t prefix_hits;   /* blocks handed out by pa_prefix_match so far */
} pa_pool_stats_t;

/* New pool of `num_blocks` blocks.  `free_order` (NULL = 0, 1, 2, ...) is a
 * permutation of [0, num_blocks): the first allocation returns free_order[0],
 * the next free_order[1], and so on.  A block whose count drops to 0 is pushed
 * back on top and is the next one handed out -- unless it is in the prefix
 * cache (below): then it stays cached and joins the end of an eviction list,
 * and an allocation takes it (dropping it from the cache) only when no
 * uncached block is free, oldest release first.  PA_ERR_INVALID_ARG if
 * num_blocks <= 0 or free_order is not a permutation. */
pa_status pa_pool_create(int32_t num_blocks, const int32_t* free_order, pa_pool** out);
void pa_pool_destroy(pa_pool* pool);

/* Take a block from the pool; its reference count becomes 1.
 * PA_ERR_OUT_OF_BLOCKS when none is free (nothing changes). */
pa_status pa_alloc(pa_pool* pool, int32_t* block_out);

/* One more reference on a held block.  PA_ERR_BAD_BLOCK if not held. */
pa_status pa_incref(pa_pool* pool, int32_t block);

/* Drop one reference; at 0 the block returns to the pool.  PA_ERR_BAD_BLOCK on
 * an id out of range or a block not held (double free). */
pa_status pa_free(pa_pool* pool, int32_t block);

/* One more reference on each of table[0..nblocks): a new sequence sharing
 * these blocks.  All-or-nothing: PA_ERR_BAD_BLOCK if any id is not held. */
pa_status pa_fork(pa_pool* pool, const int32_t* table, int32_t nblocks);

/* pa_free on table[0..nblocks) in order (a finished sequence). Stops at, and
 * returns, the first error. */
pa_status pa_free_table(pa_pool* pool, const int32_t* table, int32_t nblocks);

/* Slots for `n` new tokens at positions pos .. pos+n-1 of one sequence.
 * table_row (host, capacity max_blocks) holds *nblocks == ceil(pos/16) blocks.
 * If pos % 16 != 0 and the block holding pos has reference count > 1, it is
 * copied on write: a new block is taken, the table points at it, the source
 * loses one reference and (*cow_src, *cow_dst) name the pair to copy on the
 * device before the tokens are written; otherwise *cow_src = *cow_dst = -1.
 * New blocks are then taken in logical order as positions need them.
 * slots_out[i] = table_row[p / 16] * 16 + p % 16 for p = pos + i.
 * PA_ERR_INVALID_ARG if *nblocks != ceil(pos/16), n < 0 or the row would
 * exceed max_blocks; PA_ERR_OUT_OF_BLOCKS if the pool is short.  Either way
 * nothing changes. */
pa_status pa_append_slots(pa_pool* pool, int32_t* table_row, int32_t* nblocks,
                          int32_t max_blocks, int32_t pos, int32_t n, int64_t* slots_out,
                          int32_t* cow_src, int32_t* cow_dst);

/* Prefix cache ("PagedAttention for the professional", serve-command section:
 * requests that begin with the same tokens, such as one system prompt, reuse
 * the blocks holding them).  Only full blocks are cached.  A block's key is
 * (serial number of the cache entry of the block before it, 0 for the first
 * block of a sequence; its 16 token ids); serial numbers are never reused, so
 * a key stands for one exact token prefix and entries below an evicted block
 * can no longer be reached.  Calls that never register leave the pool
 * behaving exactly as without a cache.
 *
 * pa_prefix_match: the cached blocks holding the longest run of whole
 * leading blocks of tokens[0..num_tokens) (at most max_blocks), written to
 * table_out (host) in logical order; each gets one more reference (one for
 * the new sequence's table; an evictable block leaves the eviction list).
 * *num_matched = their number (0 when nothing is cached).  The new sequence
 * continues with pa_append_slots at pos = 16 * *num_matched.
 * PA_ERR_INVALID_ARG on a NULL pointer or negative size. */
pa_status pa_prefix_match(pa_pool* pool, const int32_t* tokens, int32_t num_tokens,
                          int32_t* table_out, int32_t max_blocks, int32_t* num_matched);

/* pa_prefix_register: enter the full blocks of a sequence whose blocks are
 * table_row[0..nblocks) and whose first num_tokens token ids are `tokens`:
 * block i holds tokens[16i .. 16i+16) for i < num_tokens / 16.  Call it once
 * those blocks' K/V are written (or enqueued on the stream that later
 * readers use).  A block already cached stays as it is; a block whose key is
 * already cached under another block is not entered (the chain continues
 * through that entry).  *num_added (may be NULL) = blocks entered.
 * All-or-nothing: PA_ERR_INVALID_ARG if num_tokens / 16 > nblocks or a
 * cached block holds other tokens, PA_ERR_BAD_BLOCK if a block is not held,
 * PA_ERR_HOST_MEMORY if the index cannot grow. */
pa_status pa_prefix_register(pa_pool* pool, const int32_t* table_row, int32_t nblocks,
                             const int32_t* tokens, int32_t num_tokens, int32_t* num_added);

/* Host tier ("KV Cache and PagedAttention: why your LLM server slows down":
 * when memory fills, small pages move to the CPU instead of whole
 * sequences).  A second pool whose ids index a cache in pinned host memory
 * of the same shape is the host tier.  pa_swap_blocks moves blocks[0..n)
 * (ids held in `src`) to `dst`: each gets a fresh dst block, taken in list
 * order before anything is released, pairs_out (host, [n][2]) receives
 * (src block, dst block) -- the copies pa_transfer_blocks must make, and the
 * caller's new table entries -- and each listed src block loses one
 * reference (a block still shared stays for its other holders).  A block may
 * be listed as often as it has references.  All-or-nothing:
 * PA_ERR_BAD_BLOCK if a block is not held (often enough),
 * PA_ERR_OUT_OF_BLOCKS if dst has fewer than n free blocks,
 * PA_ERR_INVALID_ARG on NULL pointers, n < 0 or src == dst. */
pa_status pa_swap_blocks(pa_pool* src, pa_pool* dst, const int32_t* blocks, int32_t n,
                         int64_t* pairs_out);

/* Reference count of a block (-1 if the id is out of range). */
int32_t pa_refcount(const pa_pool* pool, int32_t block);
/* Blocks an allocation can take: uncached free ones plus evictable cached ones. */
int32_t pa_num_free(const pa_pool* pool);
pa_status pa_pool_stats(const pa_pool* pool, pa_pool_stats_t* out);

/* Groups of sequences that share leading blocks, for
 * pa_paged_attention_decode_shared (host arrays).  Sequences whose tables
 * (host, [num_seqs][max_blocks], nblocks[s] entries in use) begin with the
 * same block form a candidate group, in the order of their first sequence;
 * its shared length is the longest run of leading entries equal in all its
 * rows.  Groups of two or more sequences sharing at least min_blocks (>= 1)
 * entries are written: group g is prefix_seqs[prefix_start[g] ..
 * prefix_start[g + 1]) in sequence order and shares prefix_blocks[g]
 * entries.  Capacities: prefix_seqs num_seqs, prefix_start num_seqs / 2 + 1,
 * prefix_blocks num_seqs / 2.  *num_groups / *num_members receive the
 * counts.  PA_ERR_INVALID_ARG on NULL pointers or bad sizes,
 * PA_ERR_HOST_MEMORY if scratch cannot be allocated. */
pa_status pa_shared_prefix_groups(const int32_t* tables, const int32_t* nblocks, int32_t num_seqs,
                                  int32_t max_blocks, int32_t min_blocks, int32_t* prefix_seqs,
                                  int32_t* prefix_start, int32_t* prefix_blocks,
                                  int32_t* num_groups, int32_t* num_members);

/* Whole blocks whose K and V for all layers fit in `bytes`:
 * bytes / (2 * layers * 16 * num_kv_heads * head_dim * elem_bytes), the KV_size
 * closed form of "KV Cache for the intermediate", section "Precise scientific
 * definition", taken per block.  -1 on a non-positive argument. */
int64_t pa_blocks_for_bytes(int64_t bytes, int32_t num_layers, int32_t num_kv_heads,
                            int32_t head_dim, int32_t elem_bytes);

/* ---------------------------------------------------------------------------
 * Device calls.
 * ------------------------------------------------------------------------- */

/* Write the K and V of `num_tokens` new tokens into their slots ("KV Cache and
 * PagedAttention: why your LLM server slows down", second article, section
 * "What is the KV cache?": only the new token's K/V are computed and stored).
 *   key, value   device [num_tokens][num_kv_heads][head_dim], contiguous
 *   k_cache, v_cache  device, layout above, num_blocks blocks
 *   slot_mapping device int64 [num_tokens]; a slot < 0 or >= num_blocks * 16 is
 *                skipped (no write)
 * Tokens must map to distinct slots.  head_dim: a multiple of 16 / elem bytes,
 * at most 512. */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               pa_dtype dtype, void* stream);

/* Copy whole blocks of both caches: for each pair, block dst of K and of V
 * becomes block src ("KV Cache and PagedAttention: why your LLM server slows
 * down", section "How PagedAttention fixes this": copy-on-write of shared
 * prefix blocks).
 *   block_pairs  device int64 [num_pairs][2] = (src, dst); a pair with an id
 *                out of [0, num_blocks) is skipped
 * The dsts must be distinct and none may also be a src (pairs run
 * concurrently).  Enqueue it before the pa_reshape_and_cache that writes into
 * the copies. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, pa_dtype dtype, void* stream);

/* Copy whole blocks between two caches of the same shape and dtype (PA_I8
 * for INT8 caches): for each pair, block dst of dst_k/dst_v becomes block src
 * of src_k/src_v.  Each cache pointer, and block_pairs (int64 [num_pairs][2]),
 * may be device memory or pinned host memory (hipHostMalloc; torch
 * pin_memory), reached through its device mapping; PA_ERR_INVALID_ARG for
 * memory the device cannot reach.  Pairs with an id out of range are
 * skipped.  The dsts must be distinct.  Like every call here it is only
 * enqueued on `stream`: host memory it reads (pairs, a host cache) must stay
 * allocated and unchanged until the stream has passed it. */
pa_status pa_transfer_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks,
                             void* dst_k, void* dst_v, int32_t dst_num_blocks,
                             const int64_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                             int32_t head_dim, pa_dtype dtype, void* stream);

/* Workspace bytes pa_paged_attention_decode needs for these sizes.
 * Fixed partitions (NONE or a positive size): the work list of the call (16
 * bytes per sequence and partition, rounded up to 32 entries, and 4 per
 * sequence) plus, when some sequence is split, the partial results
 * (4 * (2 + head_dim) bytes per sequence, query head and partition) and
 * 4 bytes per sequence and query head (arrival counts of the in-kernel merge).
 * PA_PARTITION_AUTO: as for the partition size it resolves to.  Each area is 256-byte aligned after a 256-byte header.  0 on invalid
 * sizes. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

/* The partition size PA_PARTITION_AUTO resolves to for these sizes
 * (PA_PARTITION_NONE or a positive multiple of 16); dtype PA_I8 gives the
 * choice of pa_paged_attention_decode_int8.  The decode may double it once
 * for a batch of evenly long sequences (see pa_paged_attention_decode). */
int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, pa_dtype dtype);

/* Decode attention over the paged cache:
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_s[t]) V_s[t],
 *   t = 0 .. context_lens[s]-1, K_s[t]/V_s[t] read through block_tables[s]
 *   from KV head h / (num_q_heads / num_kv_heads).
 * The textbook softmax and the argument `scale` are the reading taken; the
 * pages name the attention dot product without a formula.
 *   q, out        device [num_seqs][num_q_heads][head_dim], contiguous
 *   k_cache, v_cache  device, layout above
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries at or
 *                 after ceil(context_lens[s]/16) are never read, the others
 *                 must be valid block ids
 *   context_lens  device int32 [num_seqs]; counts the token being decoded
 *                 (its K/V must already be in the cache); 0 gives out = 0;
 *                 each must be <= max_context_len and <= 16 * max_blocks_per_seq
 *   partition_size  how the work is split:
 *                 a positive multiple of 16: sequences longer than it are
 *                 split into partitions of that many positions whose partial
 *                 results are merged by the running-max (log-sum-exp) rule
 *                 (on the matrix-core path, when that would make
 *                 more than max(2 * num_seqs, ceil(2048 / (num_kv_heads *
 *                 ceil(group / 16)))) partitions in all, the size is doubled
 *                 until it does not, at most 6 times, else one partition per
 *                 sequence);
 *                 PA_PARTITION_NONE: one pass over each whole sequence;
 *                 PA_PARTITION_AUTO: the partition size
 *                 pa_decode_auto_partition gives; on the matrix-core path
 *                 the device's work-list pass doubles it once for a batch of
 *                 evenly long sequences: when at twice the size the list
 *                 still holds >= 512 (item, head group) work-groups and its
 *                 longest item streams at most 1.5 x the blocks per wave of
 *                 the mean item (the workspace for the given size covers it)
 *   workspace     device, >= pa_decode_workspace_bytes(...) bytes, 256-byte
 *                 aligned; scratch that each call rewrites before reading.
 *                 Calls that share a workspace must not overlap (same stream,
 *                 or ordered by events).
 * Supported: dtype in {F32, F16, BF16}; num_q_heads % num_kv_heads == 0;
 * head_dim a multiple of 16 / elem bytes, at most 256 (the matrix-core path
 * serves bf16/fp16 at head_dim 64 and 128).  Otherwise PA_ERR_UNSUPPORTED or
 * PA_ERR_INVALID_ARG. */
pa_status pa_paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    float scale, void* out, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, pa_dtype dtype, void* stream);

/* pa_paged_attention_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace in a scratch
 * array of PA_DECODE_SCRATCH_BYTES that the library holds in device memory,
 * one per device, until the process ends.  The call allocates nothing.
 * Arguments as pa_paged_attention_decode without workspace and
 * workspace_bytes; PA_ERR_WORKSPACE when the call would need more than
 * PA_DECODE_SCRATCH_BYTES (pa_decode_workspace_bytes gives the need; a
 * larger partition size needs less), PA_ERR_DEVICE when no device is
 * current.  Every call on one device shares that device's array and
 * rewrites what it reads, so calls that overlap on one device (different
 * streams without ordering, or different host threads) race; calls ordered
 * on one stream do not. */
#define PA_DECODE_SCRATCH_BYTES ((size_t)128 << 20)
pa_status pa_paged_attention_decode_noalloc(const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* block_tables,
                                            const int32_t* context_lens, float scale, void* out,
                                            int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_blocks_per_seq, int32_t max_context_len,
                                            int32_t partition_size, pa_dtype dtype, void* stream);

/* pa_paged_attention_decode for a batch whose sequences share leading blocks
 * (the samples of one prompt hold its blocks by reference count: "KV Cache
 * and PagedAttention: why your LLM server slows down", section "How
 * PagedAttention fixes this"; "PagedAttention for the professional", results
 * list: n = 4 samples in about the memory of one).  The same outputs, with
 * each group's shared positions read from the cache once for all its
 * sequences (up to floor(16 / (num_q_heads / num_kv_heads)) sequences per
 * pass) instead of once per sequence.
 *   prefix_seqs    device int32 [num_members]: the sequences of every group,
 *                  group by group (pa_shared_prefix_groups computes them)
 *   prefix_start   device int32 [num_groups + 1]: group g is
 *                  prefix_seqs[prefix_start[g] .. prefix_start[g + 1])
 *   prefix_blocks  device int32 [num_groups]: leading table entries every
 *                  sequence of group g holds in common (the same block ids)
 *   num_groups, num_members  host counts (num_members <= 2^24)
 * A sequence belongs to at most one group, and a group lists at most
 * 32767 * floor(16 / (num_q_heads / num_kv_heads)) sequences.  Of a group,
 * only whole blocks below every member's length are read as shared; the rest
 * of each sequence is read through its own table.  Sequence ids out of range
 * are ignored; tables whose listed entries differ, or group ranges that
 * overlap, give other outputs than pa_paged_attention_decode, never an
 * out-of-range access.  The workspace
 * is sized by pa_decode_shared_workspace_bytes.  Groups are used on the
 * matrix-core path (bf16/fp16, head_dim 64/128) with at most 16 query heads
 * per KV head; otherwise the call decodes as pa_paged_attention_decode.
 * Other arguments and errors as pa_paged_attention_decode. */
pa_status pa_paged_attention_decode_shared(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* prefix_seqs, const int32_t* prefix_start,
    const int32_t* prefix_blocks, int32_t num_groups, int32_t num_members, float scale, void* out,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pa_dtype dtype, void* stream);

/* Workspace bytes of pa_paged_attention_decode_shared: as
 * pa_decode_workspace_bytes with one more partial slot per (sequence, query
 * head), (num_seqs + num_members) * (partitions) more work-list entries, and
 * 8 bytes per sequence and per group; equal to pa_decode_workspace_bytes when
 * num_groups is 0.  0 on invalid sizes. */
size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t partition_size,
                                        int32_t num_groups, int32_t num_members);

/* Chunked prefill: sequence s appends a chunk of n_s new tokens whose K/V are
 * already in the cache (pa_reshape_and_cache first, as for decode); query i
 * of the chunk sits at position p = len_s - n_s + i and attends to positions
 * 0..p (causal), as every token needs the K and V of all tokens before it
 * ("KV Cache and PagedAttention: why your LLM server slows down", second
 * article, section "What is the KV cache?").  One token per sequence is
 * decode.
 *   q, out        device [T][num_q_heads][head_dim], the chunks back to back:
 *                 sequence s owns rows query_start[s] .. query_start[s+1]-1
 *   query_start   device int32 [num_seqs + 1], non-decreasing, from 0
 *   context_lens  device int32 [num_seqs]: len_s including the chunk
 *                 (len_s >= n_s; larger n_s is read as len_s = n_s)
 *   max_chunk_len host bound of every n_s (a larger chunk is cut to it)
 * Other arguments as pa_paged_attention_decode.  dtype F16 or BF16, head_dim
 * 64 or 128, else PA_ERR_UNSUPPORTED. */
pa_status pa_paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* query_start,
                                     const int32_t* context_lens, float scale, void* out,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_blocks_per_seq,
                                     int32_t max_chunk_len, pa_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * INT8 KV cache ("KV Cache for the intermediate", section "KV Cache
 * Quantization": K and V kept as 8-bit integers instead of 16-bit floats
 * halve the cache, with per-channel scales).  Symmetric codes with one fp32
 * scale per (KV head, channel), k_scale and v_scale device [Hkv][D], all > 0,
 * chosen by the caller; the cache stands for the values code * scale.  Block
 * copies use pa_copy_blocks with dtype PA_I8.
 * ------------------------------------------------------------------------- */

/* Quantize and store the K and V of `num_tokens` new tokens:
 * code = clamp(rint(x / scale), -127, 127), with x the value of key / value
 * (dtype F32, F16 or BF16, [num_tokens][Hkv][D]) in fp32, one IEEE fp32
 * division and round-half-to-even; NaN gives 0.  Codes go to the INT8 layout
 * above.  Slots out of [0, num_blocks * 16) are skipped; tokens must map to
 * distinct slots.  head_dim: a multiple of 64, at most 512. */
pa_status pa_reshape_and_cache_int8(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping,
                                    const float* k_scale, const float* v_scale,
                                    int32_t num_tokens, int32_t num_blocks,
                                    int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                    void* stream);

/* pa_paged_attention_decode over an INT8 cache: out[s, h] = attention of
 * q[s, h] over the values code_K * k_scale, code_V * v_scale of the
 * sequence's positions.  q and out have dtype F16 or BF16; head_dim 64 or
 * 128; partition_size NONE, AUTO or a positive multiple of 16; the workspace is sized by
 * pa_decode_workspace_bytes as for a 16-bit cache.  Other arguments and
 * errors as pa_paged_attention_decode. */
pa_status pa_paged_attention_decode_int8(const void* q, const void* k_cache, const void* v_cache,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_tables,
                                         const int32_t* context_lens, float scale, void* out,
                                         int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         int32_t partition_size, void* workspace,
                                         size_t workspace_bytes, pa_dtype dtype, void* stream);

/* One decode step: pa_reshape_and_cache of the step's new tokens
 * (key/value/slot_mapping/num_new_tokens/num_blocks as there) followed by
 * pa_paged_attention_decode (the other arguments as there), with the same
 * results.  On the matrix-core path with fixed partitions the token writes
 * run in the same launch as the decode's work list, saving one kernel
 * launch per step; otherwise the two calls run one after the other.  The
 * write and decode arguments are all checked before anything is launched
 * (num_seqs = 0: only the write). */
pa_status pa_decode_step(const void* key, const void* value, const int64_t* slot_mapping,
                         int32_t num_new_tokens, int32_t num_blocks, const void* q, void* k_cache,
                         void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_blocks_per_seq, int32_t max_context_len,
                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                         pa_dtype dtype, void* stream);

/* pa_decode_step with shared prefixes: the step's token writes, then
 * pa_paged_attention_decode_shared (arguments as there and as
 * pa_decode_step), the writes riding in the launch that builds the work list
 * as in pa_decode_step. */
pa_status pa_decode_step_shared(
    const void* key, const void* value, const int64_t* slot_mapping, int32_t num_new_tokens,
    int32_t num_blocks, const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* prefix_seqs, const int32_t* prefix_start,
    const int32_t* prefix_blocks, int32_t num_groups, int32_t num_members, float scale, void* out,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size, void* workspace,
    size_t workspace_bytes, pa_dtype dtype, void* stream);

/* One decode step over an INT8 cache: pa_reshape_and_cache_int8 of the new
 * tokens followed by pa_paged_attention_decode_int8 (arguments as there),
 * the token writes running in the launch that builds the decode's work list.
 * Same results as the two calls; every argument is checked before anything
 * is launched (num_seqs = 0: only the write). */
pa_status pa_decode_step_int8(const void* key, const void* value, const int64_t* slot_mapping,
                              int32_t num_new_tokens, int32_t num_blocks, const void* q,
                              void* k_cache, void* v_cache, const float* k_scale,
                              const float* v_scale, const int32_t* block_tables,
                              const int32_t* context_lens, float scale, void* out,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_context_len, int32_t partition_size, void* workspace,
                              size_t workspace_bytes, pa_dtype dtype, void* stream);

/* pa_paged_attention_decode_int8 for a batch whose sequences share leading
 * blocks: each group's shared positions are read from the INT8 cache once for
 * all its sequences, as pa_paged_attention_decode_shared does for a 16-bit
 * cache ("KV Cache and PagedAttention: why your LLM server slows down",
 * section "How PagedAttention fixes this"; "KV Cache for the intermediate",
 * section "KV Cache Quantization").  The group arguments, their limits and
 * the treatment of malformed listings are those of
 * pa_paged_attention_decode_shared; the other arguments and errors those of
 * pa_paged_attention_decode_int8.  The workspace is sized by
 * pa_decode_shared_workspace_bytes with the same arguments (an INT8 cache
 * needs no more).  With more than 16 query heads per KV head the groups are
 * not used. */
pa_status pa_paged_attention_decode_int8_shared(
    const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* prefix_seqs, const int32_t* prefix_start, const int32_t* prefix_blocks,
    int32_t num_groups, int32_t num_members, float scale, void* out, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pa_dtype dtype, void* stream);

/* pa_decode_step_int8 with shared prefixes: the step's quantizing token
 * writes, then pa_paged_attention_decode_int8_shared (arguments as there and
 * as pa_decode_step_int8), the writes running in the launch that builds the
 * work list. */
pa_status pa_decode_step_int8_shared(
    const void* key, const void* value, const int64_t* slot_mapping, int32_t num_new_tokens,
    int32_t num_blocks, const void* q, void* k_cache, void* v_cache, const float* k_scale,
    const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* prefix_seqs, const int32_t* prefix_start, const int32_t* prefix_blocks,
    int32_t num_groups, int32_t num_members, float scale, void* out, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t partition_size, void* workspace, size_t workspace_bytes,
    pa_dtype dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Kernel timing.  Between pa_timing_begin and pa_timing_end every kernel the
 * library launches carries two HIP events attached to its dispatch on its own
 * stream, which record the start and the end of the kernel's execution (the
 * interval a kernel-trace profiler reports).  pa_timing_end waits for those
 * events and returns, per kernel kind, the summed milliseconds and the launch
 * count.  At most `capacity` launches are recorded; later ones run untimed.
 * ------------------------------------------------------------------------- */
#define PA_KERNEL_DECODE 0          /* main pass of pa_paged_attention_decode */
#define PA_KERNEL_DECODE_REDUCE 1   /* merge pass of split sequences */
#define PA_KERNEL_RESHAPE_AND_CACHE 2
#define PA_KERNEL_COPY_BLOCKS 3
#define PA_KERNEL_DECODE_PLAN 4     /* work list of pa_paged_attention_decode (in
                                       pa_decode_step: with the token writes) */
#define PA_KERNEL_TRANSFER_BLOCKS 5 /* pa_transfer_blocks */
#define PA_KERNEL_PREFILL 6         /* pa_paged_attention_prefill */
#define PA_NUM_KERNEL_KINDS 7

pa_status pa_timing_begin(int32_t capacity);
pa_status pa_timing_end(double* ms_out /* [PA_NUM_KERNEL_KINDS] */,
                        int32_t* launches_out /* [PA_NUM_KERNEL_KINDS] */);

/* The milliseconds of each launch of kernel kind `kind` that the last
 * pa_timing_end measured, in launch order (for medians and percentiles):
 * the first `capacity` of them into ms_out (host memory, which may be NULL
 * when capacity is 0), their count into *count_out (which may exceed
 * capacity).  Valid until the next pa_timing_end.  PA_ERR_INVALID_ARG for a
 * kind outside [0, PA_NUM_KERNEL_KINDS), a negative capacity or a NULL
 * pointer that is needed. */
pa_status pa_timing_launches(int32_t kind, double* ms_out, int32_t capacity,
                             int32_t* count_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
