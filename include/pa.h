/*
 * pa.h — PagedAttention decode for AMD Instinct MI355X (gfx950): the C ABI.
 *
 * One shared library, libpa.so, exports everything declared here.  All calls
 * are extern "C", take plain host or device pointers and sizes, never throw
 * across the boundary, and report failure through pa_status.
 *
 * Sources (the pages this library implements):
 *   [SRC-1] "PagedAttention 源码解析：KV Cache 怎么管理" (coreui.cn)
 *   [XDNF]  xdnf.cn article on PagedAttention block mapping, dynamic allocation
 *           and copy-on-write
 *   [ASC]   "Ascend C算子开发高阶实战：实现高性能KV Cache管理与PagedAttention融合算子"
 *           (cann.csdn.net)
 *   [IMPL]  "PagedAttention 实现细节" (pyllm.pages.dev)
 *   [ATB]   "Ascend平台下的PageAttention优化实践" (jsqmd.com)
 *
 * Data layout (device memory, all row-major, all owned by the caller):
 *   query, out      [num_seqs, num_heads, head_dim]               element type `dtype`
 *   key_cache       [num_blocks, num_kv_heads, block_size, head_dim]  element type `dtype`
 *                   (the separate key pool of [IMPL] §3.1/§3.4: one token's
 *                   key is head_dim contiguous elements)
 *   value_cache     [num_blocks, num_kv_heads, head_dim, block_size]  element type `dtype`
 *                   (block size innermost, the arrangement of [ASC] §3.1/§5.2:
 *                   one dim of a block's block_size tokens is contiguous)
 *                   In both pools one (block, kv head) tile is one contiguous
 *                   block_size * head_dim run.  The two orientations give the
 *                   decode kernel's matrix-core products 16-byte operand loads
 *                   along their contraction axes (head_dim for q.K, tokens for
 *                   P.V).
 *                   This value layout departs from [IMPL] §3.1/§3.4, where both
 *                   pools hold token rows [num_blocks, num_kv_heads, block_size,
 *                   head_dim]; it follows the Ascend kernel's value arrangement
 *                   instead.  Its cost falls on the write: one new token's value
 *                   is a column, head_dim elements each block_size elements
 *                   apart, so it touches every 128-byte line of its tile, and
 *                   the decode that follows pays 8-16 us for rereading those
 *                   lines at the LLaMA-7B-like shapes (64 sequences x 32 heads).
 *                   pa_upload_and_cache narrows that with a whole-tile write
 *                   where a value row is 64 bytes (or 32 bytes of 8-bit codes)
 *                   and non-temporal stores otherwise.
 *
 * Beyond the pages' problem interface (query, pools, block_tables,
 * context_lens, scale), the decode calls take two more arguments: seq_order
 * (an optional launch order of the sequences, longest first to balance the
 * last wave) and flags (PA_DECODE_CACHED_KV, the K/V cache policy).
 *   block_tables    [num_seqs, max_blocks_per_seq] int32; entry j of row s is
 *                   the physical block of logical block j (tokens j*bs ..
 *                   j*bs+bs-1) of sequence s; unused entries are -1 by
 *                   convention and never read
 *   context_lens    [num_seqs] int32, the number of cached tokens of each sequence
 *   slot_mapping    [num_tokens] int32, slot = block * block_size + offset
 *
 * Query head h reads KV head h / (num_heads / num_kv_heads) (contiguous
 * groups; num_heads must be a multiple of num_kv_heads).
 *
 * Supported shapes: dtype f32, f16, bf16 (8-bit pools: see the quantised KV
 * cache below); head_dim 64 or 128; block_size 16 or 32, and with head_dim
 * 128 also 8 or 64 (the block sizes 8-64 of [SRC-1] §五;
 * 8-bit pools: 16, 32 or 64).  Other values return PA_ERR_UNSUPPORTED.
 *
 * Streams: device calls enqueue work on `stream` (a hipStream_t; NULL is the
 * null stream) and return without synchronising.  The library allocates no
 * device memory; the split path's workspace is passed in by the caller, except
 * for pa_decode_split_static, whose partials live in a fixed array the library
 * holds on each device it runs on.
 *
 * Debug mode: with the environment variable PA_DEBUG=1 set when the library
 * is loaded, device calls first copy the index arrays back to the host
 * (synchronising `stream`) and validate them, returning PA_ERR_BAD_TABLE on
 * any violation, and synchronise after the launch to report kernel errors.
 *
 * Two more switches are read on every call: PA_SPLIT=never / always overrides
 * the automatic path choice of pa_decode_auto, pa_decode_quant,
 * pa_decode_masked and pa_decode_multi (always: whenever the workspace and
 * partition size allow a split); PA_LOG=1 makes pa_build_block_tables print
 * each table to stderr ("pa: seq <id>: [blocks] len <n>").
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 5

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,        /* null pointer, negative size, bad combination */
  PA_ERR_NO_FREE_BLOCKS = 2,     /* the pool cannot satisfy the request; state unchanged */
  PA_ERR_UNKNOWN_SEQ = 3,        /* no sequence with this id */
  PA_ERR_SEQ_EXISTS = 4,         /* a sequence with this id already exists */
  PA_ERR_UNSUPPORTED = 5,        /* dtype / head_dim / block_size not built */
  PA_ERR_BAD_TABLE = 6,          /* PA_DEBUG validation: index outside its range, or a write race */
  PA_ERR_WORKSPACE_TOO_SMALL = 7,
  PA_ERR_HIP = 8,                /* a HIP runtime call or kernel launch failed */
  PA_ERR_UNKNOWN_PREFIX = 9      /* no prefix-cache entry with this id */
} pa_status;

/* Element types.  PA_F32, PA_F16 and PA_BF16 are model types (query, out,
 * new K/V rows, 16-bit and 32-bit pools).  PA_FP8_E4M3, PA_INT8 and
 * PA_INT8_TOKEN are the 8-bit KV code types of the quantised cache (see
 * pa_reshape_and_cache_quant): they are valid only as kv_dtype of the calls
 * that take one and as the dtype of pa_copy_blocks / pa_swap_blocks on 8-bit
 * pools. */
typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3, /* OCP FP8 E4M3 ("fn"): bias 7, 3 mantissa bits, max 448, NaN 0x7F/0xFF */
  PA_INT8 = 4,     /* two's-complement int8, one scale per pool */
  PA_INT8_TOKEN = 5 /* int8 with one fp32 scale per (token, KV head), kept in the block's tiles */
} pa_dtype;

/* Decode flags (bit mask).  By default K/V rows are read with a streaming
 * (non-temporal) cache hint: each KV element is read once per step, so it
 * should not displace anything.  PA_DECODE_CACHED_KV reads them with the
 * default policy instead, for pools where several sequences in the batch
 * share blocks (forked branches, shared prefixes), so that the sharers' reads
 * can hit the caches; order such sharers next to each other in seq_order.
 * Results do not depend on the flag. */
#define PA_DECODE_CACHED_KV 1u
/* pa_decode_quant only: take the split path (partials + merge) regardless of
 * the launch shape; the workspace must then be large enough. */
#define PA_DECODE_SPLIT 2u

/* ======================================================================== *
 * Host block allocator                                                      *
 * ======================================================================== *
 * The pool's bookkeeping on the host ([SRC-1] §二/§三 PagedKVCache,
 * [XDNF] §3.3/§3.4/§4.2, [IMPL] §3.3 and §3.4 BlockSpaceManager,
 * [ASC] §7.1 BlockManager, [ATB] §4.2 BlockManager):
 *   - free blocks form a first-in-first-out queue: allocation takes the head,
 *     a block whose refcount reaches 0 goes to the tail ([SRC-1] §二 worked
 *     example: 32, 16, 48 tokens -> [0,1], [2], [3,4,5], free [6,7,8,...]);
 *   - a sequence of n tokens holds ceil(n / block_size) blocks;
 *   - each block has a refcount: 1 when allocated, +1 per extra sharer;
 *   - copy-on-write is decided before a write ([XDNF] §3.4, [IMPL] §3.3).
 * Every call is all-or-nothing: on error the state is unchanged.  Calls on
 * one handle are serialised by an internal mutex.  Sequence ids are arbitrary
 * int64 values chosen by the caller.  The allocator touches no device memory.
 */
typedef struct pa_allocator pa_allocator;

typedef struct pa_allocator_stats {
  int64_t blocks_allocated;  /* blocks taken from the free queue */
  int64_t blocks_freed;      /* blocks returned to the free queue */
  int64_t cow_copies;        /* copy-on-write pairs emitted */
} pa_allocator_stats;

/* Create a pool of num_blocks blocks of block_size tokens.  initial_free_order:
 * NULL for 0..num_blocks-1, else a host array of num_blocks ids that must be
 * a permutation of 0..num_blocks-1 (PA_ERR_INVALID_ARG otherwise).  *out
 * receives the handle; the caller destroys it with pa_allocator_destroy. */
pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* initial_free_order, pa_allocator** out);
void pa_allocator_destroy(pa_allocator* a);
/* Deep copy of the whole state (free queue order, refcounts, sequences, stats). */
pa_status pa_allocator_clone(const pa_allocator* a, pa_allocator** out);

/* New sequence holding num_tokens >= 0 tokens: ceil(num_tokens / bs) blocks
 * from the head of the free queue, each with refcount 1 ([SRC-1] §三). */
pa_status pa_seq_create(pa_allocator* a, int64_t seq_id, int32_t num_tokens);

/* Fork for parallel sampling / beam search ([XDNF] §3.4): the child gets the
 * parent's first ceil(n / bs) blocks, each gaining one reference, and length
 * n = num_tokens (0 <= n <= parent length; -1 means the parent's length). */
pa_status pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child, int32_t num_tokens);

/* Reserve the slot of the sequence's next token (position L = current length)
 * ([XDNF] §4.2 append_token_kv, §3.1 addressing; [IMPL] §3.3):
 *   L % bs == 0            -> a fresh block is appended to the table;
 *   last block refcount >1 -> copy-on-write: a fresh block replaces it in the
 *                             table, *cow_src / *cow_dst receive (old, new),
 *                             the old refcount drops by one, the new is 1;
 *   otherwise              -> the token is written in place.
 * *slot = table[L / bs] * bs + L % bs; the length becomes L + 1.  *cow_src and
 * *cow_dst are -1 when no copy is needed.  The caller must copy the whole
 * block (pa_copy_blocks) before writing the token (pa_reshape_and_cache). */
pa_status pa_seq_append_slot(pa_allocator* a, int64_t seq_id, int32_t* slot,
                             int32_t* cow_src, int32_t* cow_dst);

/* One decode step's bookkeeping: pa_seq_append_slot for seq_ids[0..n-1] in
 * that order (so earlier sharers copy and the last remaining sharer writes in
 * place).  slots: host [n]; cow_pairs: host [n, 2] (src, dst) capacity;
 * *num_pairs receives the number of pairs written.  All-or-nothing. */
pa_status pa_seq_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n,
                              int32_t* slots, int32_t* cow_pairs, int32_t* num_pairs);

/* Release a sequence ([XDNF] §4.2 free_sequence): each block in table order
 * loses one reference and goes to the tail of the free queue at 0. */
pa_status pa_seq_free(pa_allocator* a, int64_t seq_id);

pa_status pa_can_allocate(const pa_allocator* a, int32_t num_blocks, int32_t* ok);
int32_t pa_num_free_blocks(const pa_allocator* a);
/* Refcount of a block, or -1 when `block` is outside [0, num_blocks). */
int32_t pa_ref_count(const pa_allocator* a, int32_t block);
pa_status pa_seq_len(const pa_allocator* a, int64_t seq_id, int32_t* len);
/* Copy a sequence's table into host out[0..capacity); *num_blocks receives its
 * length (PA_ERR_INVALID_ARG if it exceeds capacity). */
pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out,
                             int32_t capacity, int32_t* num_blocks);
/* Copy the free queue, head first, into host out[0..capacity). */
pa_status pa_free_list(const pa_allocator* a, int32_t* out, int32_t capacity, int32_t* n);
/* Fill host tables [n, max_blocks] (rows padded with -1) and context_lens [n]
 * for the listed sequences ([ATB] §4.2 get_block_table / get_context_lens).
 * PA_ERR_INVALID_ARG if a table is longer than max_blocks. */
pa_status pa_build_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t n,
                                int32_t max_blocks, int32_t* tables, int32_t* context_lens);
pa_status pa_allocator_get_stats(const pa_allocator* a, pa_allocator_stats* out);

/* Launch order for the decode calls: order[0..n) receives the indices of the
 * sequences sorted by context_lens (host [n]) from longest to shortest, ties
 * in index order.  Passing it as `seq_order` starts the longest sequences
 * first, so short ones fill the gaps they leave (longest-processing-time-first
 * scheduling); this changes no result.  Host arrays; PA_ERR_INVALID_ARG on a
 * null pointer or negative n. */
pa_status pa_order_longest_first(const int32_t* context_lens, int32_t n, int32_t* order);

/* Groups for pa_decode_shared, from host block tables (host int32
 * [n, max_blocks]) and context lengths (host [n]).  Consecutive sequences whose
 * first table entry is the same block form a group when there are at least two
 * (the branches of a fork sit next to each other in a batch built in fork
 * order); a sequence alone is a group of one with prefix 0.  A group's row is
 * its longest member (the first of them); each member's prefix P_i is the
 * number of leading table entries it shares with the row, times block_size,
 * capped at its context, and the row's own prefix is its whole context.
 * Forked branches that each copied their last block on a write share every
 * other block, so P_i covers all but that block.  Writes group_start (host
 * [n + 1], from 0 to n), prefix_len (host [n]), *num_groups and
 * *max_group_size (1 when no group has two members; 0 for n = 0).
 * PA_ERR_INVALID_ARG on a null pointer or a negative size. */
pa_status pa_shared_prefix_groups(const int32_t* tables, const int32_t* context_lens, int32_t n, int32_t max_blocks,
                                  int32_t block_size, int32_t* group_start, int32_t* prefix_len,
                                  int32_t* num_groups, int32_t* max_group_size);

/* ------------------------------------------------------------------------ *
 * Prefix caching ([IMPL] §3.2 CachedPrefix / PrefixCacheManager): requests
 * that share a prompt prefix (a system prompt) share the blocks holding its
 * KV.  An entry maps the prefix's tokens to ceil(n / bs) blocks, counts the
 * requests using it (users) and holds one reference on each block.  The key
 * is the token sequence itself, compared in full (the page hashes it to 12
 * hex digits; exact keys keep different prompts from sharing blocks).
 * ------------------------------------------------------------------------ */

/* Look up tokens[0..num_tokens).  Known: one more user, *hit = 1.  New: the
 * entry takes ceil(num_tokens / bs) blocks from the head of the free queue,
 * has one user and *hit = 0; the caller computes the prefix's KV and writes
 * it into those blocks (pa_prefix_info lists them).  *prefix_id receives the
 * entry's id (ids count up from 1 and are not reused).  PA_ERR_NO_FREE_BLOCKS
 * leaves the state unchanged. */
pa_status pa_prefix_get_or_create(pa_allocator* a, const int32_t* tokens, int32_t num_tokens,
                                  int64_t* prefix_id, int32_t* hit);

/* One user fewer; at zero the entry releases its block references (table
 * order; blocks still used by sequences stay allocated) and is removed.
 * PA_ERR_UNKNOWN_PREFIX for an unknown id. */
pa_status pa_prefix_release(pa_allocator* a, int64_t prefix_id);

/* An entry's blocks (host out[0..capacity), *num_blocks receives the count),
 * its token count and its number of users.  Any output pointer but
 * num_blocks may be NULL. */
pa_status pa_prefix_info(const pa_allocator* a, int64_t prefix_id, int32_t* blocks, int32_t capacity,
                         int32_t* num_blocks, int32_t* num_tokens, int32_t* users);

/* New sequence on a cached prefix of n_p tokens in P blocks: its table starts
 * with the entry's blocks (one more reference each, never written through
 * this sequence) followed by ceil(own_tokens / bs) fresh blocks for its own
 * tokens, which start at position P * bs ([IMPL] §3.2's demo counts them in
 * blocks of their own).  Its length counts positions: P * bs + own_tokens.
 * When n_p < P * bs, positions [n_p, P * bs) hold no token: a hole that the
 * decode must skip (pa_build_masks gives it, pa_decode_masked skips it).
 * Appends continue after the own tokens.  A fork keeps the hole and may not
 * end inside it (PA_ERR_INVALID_ARG). */
pa_status pa_seq_create_with_prefix(pa_allocator* a, int64_t seq_id, int64_t prefix_id, int32_t own_tokens);

/* Per sequence the positions [mask_lo, mask_hi) that hold no token, for
 * pa_decode_masked (both 0 when there is none).  mask_lo, mask_hi: host [n]. */
pa_status pa_build_masks(const pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* mask_lo,
                         int32_t* mask_hi);

/* ------------------------------------------------------------------------ *
 * Swap to a host pool ([IMPL] §3.4: the cache engine has a device-side pool
 * and a host-side one used for swapping) and sliding-window release.
 * ------------------------------------------------------------------------ */

/* (Re)create the host pool: num_host_blocks block ids 0.. with their own FIFO
 * free queue and counts (the memory is the caller's: pinned host pools of the
 * device pools' shapes, see pa_swap_blocks).  PA_ERR_INVALID_ARG while any
 * sequence is swapped out. */
pa_status pa_allocator_set_host_pool(pa_allocator* a, int32_t num_host_blocks);

/* Move a group of sequences to the host pool.  Every distinct device block of
 * their tables (table order, first appearance; -1 entries skipped) takes the
 * head of the host queue; pairs[2i], pairs[2i+1] = (device id, host id) for
 * the copy (pa_swap_blocks from the device pools into the host pools); each
 * reference the group held moves to the host block, and a device block goes
 * back to the free queue when nothing else holds it.  Blocks shared inside
 * the group stay shared; blocks shared with sequences outside it are copied
 * and keep their other references.  pairs: host int32 [capacity, 2].
 * Duplicated ids count once.  A swapped sequence can only be swapped in or
 * freed (other verbs: PA_ERR_INVALID_ARG).  All-or-nothing
 * (PA_ERR_NO_FREE_BLOCKS when the host pool is short). */
pa_status pa_seq_swap_out(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* pairs, int32_t capacity,
                          int32_t* num_pairs);

/* The mirror image: every distinct host block of a swapped group takes the
 * head of the device queue; pairs = (host id, device id); host blocks go back
 * to the host queue when free. */
pa_status pa_seq_swap_in(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* pairs, int32_t capacity,
                         int32_t* num_pairs);

/* Host queue, head first, and a host block's count (-1 outside the pool). */
pa_status pa_host_free_list(const pa_allocator* a, int32_t* out, int32_t capacity, int32_t* n);
int32_t pa_host_ref_count(const pa_allocator* a, int32_t block);

/* Sliding window ([SRC-1] §六 lists it): only the last `window` positions of
 * the sequence stay live.  Every block whose positions all lie before
 * len - window is released and its table entry becomes -1, now and after
 * every append; pa_build_masks then gives [0, len - window) for
 * pa_decode_masked, which never reads those blocks.  A fork keeps the window
 * and fails (PA_ERR_INVALID_ARG) when its own window needs a released block.
 * PA_ERR_INVALID_ARG for window < 1, a swapped sequence or one with a prefix
 * hole. */
pa_status pa_seq_set_window(pa_allocator* a, int64_t seq_id, int32_t window);

/* ======================================================================== *
 * Device operations                                                         *
 * ======================================================================== */

/* Write new K/V rows into the pools through the slot mapping ([ASC] §3.1
 * slot_mapping; [IMPL] §3.4 _add_kv_cache):
 *   for i < num_tokens with 0 <= s = slot_mapping[i] < num_blocks*block_size:
 *     key_cache[s / bs, h, s % bs, :]   = key[i, h, :]    for every KV head h,
 *     value_cache[s / bs, h, :, s % bs] = value[i, h, :].
 * key, value: device [num_tokens, num_kv_heads, head_dim].  Negative slots are
 * skipped (padding); slots past the pool are skipped too (and rejected under
 * PA_DEBUG).  Two tokens with the same slot race: invalid input.  A pure copy,
 * bit-exact. */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, pa_dtype dtype, void* stream);

/* Copy-on-write block copies ([IMPL] §3.3: the whole block is copied):
 * for each pair p < num_pairs, block pairs[2p] (src) -> pairs[2p+1] (dst) in
 * both pools, all KV heads, all tokens (the whole tile of each pool).  pairs: device int32 [num_pairs, 2].
 * Pairs run concurrently: a block that is the destination of one pair must
 * not be the source or destination of another (rejected under PA_DEBUG).
 * Pairs with an id outside [0, num_blocks) are skipped.  Bit-exact. */
pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, pa_dtype dtype, void* stream);

/* Swap copies ([IMPL] §3.4, the GPU and CPU pools of the cache engine):
 * block pairs[2p] of the source pools -> block pairs[2p+1] of the destination
 * pools, for p < num_pairs, K and V, whole blocks (the pairs pa_seq_swap_out
 * and pa_seq_swap_in return).  Each side is either device memory or
 * page-locked host memory (hipHostMalloc, or torch's pin_memory()) of the
 * pools' shapes with num_src_blocks / num_dst_blocks blocks; K and V of one
 * side live in the same kind of memory.  pairs: device memory or page-locked
 * host memory, int32 [num_pairs, 2], read on the device when the copy runs.
 * Host memory is read with system-scope loads; host-side results are visible
 * once the stream has finished.  Pairs with an id outside its pool are
 * skipped.  dtype: the pools' element type (8-bit code types included).
 * PA_ERR_INVALID_ARG when a pointer is neither kind.  Bit-exact. */
pa_status pa_swap_blocks(void* dst_key_cache, void* dst_value_cache, const void* src_key_cache,
                         const void* src_value_cache, const int32_t* pairs, int32_t num_pairs,
                         int32_t num_src_blocks, int32_t num_dst_blocks, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pa_dtype dtype, void* stream);

/* Move one step's index data (block tables, context lengths, slot mapping,
 * copy pairs, launch order) from page-locked host memory to the device with a
 * kernel on `stream`, instead of a copy-engine transfer.  This is the upload
 * half of materialising the host bookkeeping on the device (block tables from
 * the allocator, [ATB] §4.2 get_block_table / get_context_lens; slot_mapping,
 * [ASC] §3.1).  On the compute stream a copy-engine transfer is bracketed by
 * cross-engine synchronisations that idle the GPU for tens of microseconds
 * per step; the kernel needs only the ordinary dispatch gap.
 *   dst: device memory, nbytes bytes, 4-byte aligned.
 *   src: page-locked host memory mapped for the device (hipHostMalloc, or a
 *        torch tensor from pin_memory()), nbytes bytes, 4-byte aligned.  The
 *        caller must not modify it until the work on `stream` has completed.
 *   nbytes: a multiple of 4 (0 is a no-op).
 * Returns PA_ERR_INVALID_ARG, without launching anything, when src is not
 * such host memory or dst is not device memory.  Bit-exact. */
pa_status pa_upload(void* dst, const void* src, size_t nbytes, void* stream);

/* pa_upload and the slot-mapping write of the step's new K/V rows in one
 * launch (two launches would cost a dependent-dispatch gap between them):
 * copies nbytes from src (page-locked host memory) to dst (device) as
 * pa_upload, and writes key/value [num_tokens, num_kv_heads, head_dim] of
 * `dtype` at the slots slot_mapping[0..num_tokens), which it reads straight
 * from page-locked host memory (typically inside src).  kv_dtype == dtype:
 * the write of pa_reshape_and_cache; PA_FP8_E4M3 / PA_INT8: the quantising
 * write of pa_reshape_and_cache_quant with k_scale, v_scale (PA_INT8_TOKEN is
 * not taken here: PA_ERR_UNSUPPORTED; use pa_upload, then
 * pa_reshape_and_cache_quant).  The two parts
 * are independent: nothing in dst may be needed by the write, and a write
 * into a block that a copy-on-write pair of the same step copies must wait
 * for that copy (use pa_upload, pa_copy_blocks, then the write).  The call
 * also reads slot_mapping on the host, so it must hold its final values when
 * the call is made.  When no two tokens' slots fall in one block (a decode
 * step appending one token per sequence) and a value tile's dim row is 64
 * bytes (block_size x element bytes; or 32 bytes of 8-bit codes), the write
 * stores each written value tile whole (every cache line of the tile, the
 * other columns unchanged) rather than one element per dim row; otherwise,
 * for model-type pools, it stores the elements with non-temporal stores.
 * The result is the same.  PA_TILE_WRITE=always / never overrides the
 * row-size rule
 * (never the one-token-per-block condition).  Errors as in pa_upload and the
 * write it stands for.  Bit-exact. */
pa_status pa_upload_and_cache(void* dst, const void* src, size_t nbytes, const void* key, const void* value,
                              void* key_cache, void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                              int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              float k_scale, float v_scale, pa_dtype dtype, pa_dtype kv_dtype, void* stream);

/* Measurement hook.  The next call of this library made on the calling
 * thread attaches start_event to the start of its first kernel and
 * stop_event to the end of its last (hipExtLaunchKernel).  Such events bound
 * the call's kernels more tightly than events recorded on the stream before
 * and after the call, whose own processing falls inside the window; like
 * them, they still leave a few microseconds of idle GPU around the call.
 * Every device call of the library honours the setting.  A call that reaches
 * its launch clears it; a call that launches nothing (rejected, or with
 * nothing to do, such as zero sequences) leaves it set.  The events are
 * hipEvent_t the caller created with timing enabled; either may be NULL.
 * Read them with hipEventElapsedTime once the stream has passed the call.
 * Always PA_OK. */
pa_status pa_set_launch_events(void* start_event, void* stop_event);

/* Single-pass paged decode attention ([IMPL] §3.1 index-based kernel and
 * §3.4 PagedAttention.forward; [ATB] §3.2 PagedAttentionOperation.apply;
 * [ASC] §三/§四 fused gather + QK^T + softmax + OV):
 *   for each sequence s and query head h, with n = context_lens[s],
 *   g = h / (num_heads / num_kv_heads), token t in block
 *   b = block_tables[s, t / bs] at offset o = t % bs,
 *   K_t = key_cache[b, g, o, :], V_t = value_cache[b, g, :, o]:
 *     z_t = scale * <query[s,h,:], K_t>,  out[s,h,:] = sum_t softmax(z)_t V_t
 * accumulated in fp32 with an online softmax (running max and sum, both
 * rescaled when the max grows), written in `dtype` (round to nearest even).
 * n == 0 gives a zero row.  max_context_len bounds every n and is used to
 * size the launch.  seq_order: NULL, or device int32 [num_seqs], a
 * permutation of 0..num_seqs-1 giving the order in which sequences are
 * started (see pa_order_longest_first); it does not change any result.
 * Entries outside [0, num_seqs) are ignored (rejected under PA_DEBUG); a
 * sequence missing from the permutation gets no output.  flags: PA_DECODE_*
 * bits (unknown bits are PA_ERR_INVALID_ARG).
 * Invalid device data never causes an out-of-bounds access: a context length
 * outside [0, min(max_context_len, max_blocks_per_seq*bs)] or a block id
 * outside [0, num_blocks) among the first ceil(n / bs) entries makes that
 * sequence's output rows NaN (PA_ERR_BAD_TABLE under PA_DEBUG). */
pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                    int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                    float scale, pa_dtype dtype, uint32_t flags, void* stream);

/* Split-context workspace.  For P = ceil(max_context_len / partition_size)
 * partitions, the workspace holds three fp32 arrays, each starting at a
 * 256-byte aligned offset:
 *   m [num_seqs, num_heads, P]         m_p = max logit of partition p (natural units)
 *   l [num_seqs, num_heads, P]         l_p = sum_t exp(z_t - m_p)
 *   o [num_seqs, num_heads, P, head_dim] o_p = sum_t exp(z_t - m_p) V_t / l_p
 * Partition p of sequence s covers tokens [p*PS, min((p+1)*PS, n)); only the
 * first ceil(n / PS) partitions of a sequence are written.  Returns 0 on an
 * invalid argument. */
size_t pa_decode_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size);

/* Split-context decode for few, very long sequences ([ATB] §2.3 describes a
 * second kernel for that case): one pass writes the per-partition partials
 * (m_p, l_p, o_p) above into `workspace`, then pa_lse_reduce merges them into
 * `out`.  Same arguments and error behaviour as pa_decode, plus
 * partition_size (a multiple of block_size, at most 4096) and the
 * caller-owned device workspace of workspace_bytes bytes. */
pa_status pa_decode_split(void* out, const void* query, const void* key_cache,
                          const void* value_cache, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* seq_order, int32_t num_seqs,
                          int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                          float scale, pa_dtype dtype, uint32_t flags, int32_t partition_size,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the library's static split workspace (pa_decode_split_static):
 * 32 MiB per device, enough for the partials of 4 sequences x 32 heads of
 * dimension 128 over 131072-token contexts in 512-token partitions. */
#define PA_STATIC_SCRATCH_BYTES (32u * 1024u * 1024u)

/* pa_decode_split without a workspace argument, for callers that cannot
 * allocate device memory (work recorded under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the partials go to a
 * file-scope device array of PA_STATIC_SCRATCH_BYTES owned by the library,
 * one per device, held from the first call on that device until the process
 * ends.  The call makes no allocation (no hipMalloc / hipFree, none by a
 * library routine).  Arguments, results and error behaviour are those of
 * pa_decode_split; a shape whose partials need more than
 * PA_STATIC_SCRATCH_BYTES (pa_decode_split_workspace_bytes) returns
 * PA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  Every call on a
 * device shares that device's array and nothing in it needs clearing (each
 * partial is written before it is read), so calls on one device that may
 * overlap in time (different streams, different host threads) race on it:
 * serialise them, e.g. on one stream. */
pa_status pa_decode_split_static(void* out, const void* query, const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                 int32_t max_context_len, float scale, pa_dtype dtype, uint32_t flags,
                                 int32_t partition_size, void* stream);

/* Decode with the path chosen for the launch.  The vLLM notes of [ATB] §2.3
 * keep a second kernel for few, very long requests; here the choice comes
 * from the launch shape instead of the page's length thresholds:
 *   split (pa_decode_split with partition_size and workspace) when the single
 *   pass would start fewer workgroups than the device holds at once
 *   (num_seqs x KV-head groups below the resident capacity, so compute units
 *   would idle while a few workgroups walk long contexts) and max_context_len
 *   spans at least 4 partitions;
 *   otherwise the single pass (pa_decode).
 * Arguments as pa_decode_split; the errors are those of the path that runs.
 * The split runs only when it can: with workspace NULL or smaller than
 * pa_decode_split_workspace_bytes for this shape, or a partition_size that
 * pa_decode_split refuses, the single pass runs.  *path (may be NULL)
 * receives 0 for the single pass and 1 for split.  Both paths agree within
 * the stated tolerances. */
pa_status pa_decode_auto(void* out, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                         int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                         int32_t max_context_len, float scale, pa_dtype dtype, uint32_t flags,
                         int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* path,
                         void* stream);

/* One decode step with the slot-mapping write fused in: equivalent to
 * pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
 * num_seqs, ...) followed by pa_decode_auto, in one launch.  The pages write
 * each step's new K/V into its block ([IMPL] §3.4 _add_kv_cache; [ASC] §3.1
 * slot_mapping) and attend over the context that includes it (the step
 * writes, then decodes).
 *   key, value: device [num_seqs, num_kv_heads, head_dim], one new token per
 *     sequence (row s belongs to sequence s).
 *   slot_mapping: device int32 [num_seqs]; slot_mapping[s] must be the slot of
 *     token context_lens[s] - 1 of sequence s (the slot pa_seq_append_slot
 *     returned), or negative for no write.  A slot elsewhere is still written,
 *     but the decode may read that block's old or new contents (a race).
 *   key_cache, value_cache: written (one key row and one value column per
 *     sequence and KV head) and read.
 * The decode does not wait for the write: the wave whose step holds token
 * context_lens[s] - 1 takes its key row and value column from key / value
 * directly (when slot_mapping[s] is inside the pool; otherwise it reads the
 * pool there, as the write-then-decode order would), and workgroups after the
 * decode's own in the same launch store the new rows.  Output and pools are
 * bit-identical to the two calls.  Other arguments, the path choice, *path and
 * the errors are those of pa_decode_auto; under PA_DEBUG the slots are
 * validated as in pa_reshape_and_cache. */
pa_status pa_decode_append(void* out, const void* query, const void* key, const void* value,
                           const int32_t* slot_mapping, void* key_cache, void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                           int32_t max_context_len, float scale, pa_dtype dtype, uint32_t flags,
                           int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* path,
                           void* stream);

/* Log-sum-exp merge of split partials (the standard rule; the pages do not
 * spell it out): with M = max_p m_p and w_p = l_p * exp(m_p - M),
 *   out[s,h,:] = sum_p w_p o_p / sum_p w_p   over p < ceil(n / partition_size),
 * written in `dtype`; n == 0 gives zeros; an invalid n gives NaN rows.
 * `workspace` is laid out as described for pa_decode_split_workspace_bytes
 * with the same num_seqs, num_heads, head_dim, max_context_len and
 * partition_size. */
pa_status pa_lse_reduce(void* out, const void* workspace, size_t workspace_bytes,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                        int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                        pa_dtype dtype, void* stream);

/* Decode with masked positions: pa_decode's definition over the tokens
 * t < n = context_lens[s] that lie outside [mask_lo[s], mask_hi[s]).  This is
 * the decode of a sequence built on a cached prefix ([IMPL] §3.2; the hole
 * [n_p, P * bs) from pa_build_masks) and of a sliding window over the last W
 * tokens ([SRC-1] §六 lists the window among the features: mask [0, n - W)).
 *   mask_lo, mask_hi: device int32 [num_seqs], or both NULL (no mask); an
 *     interval with mask_hi <= mask_lo masks nothing.
 * Blocks whose positions below n are all masked are never read: their table
 * entries may hold anything (a window's dropped blocks), and steps wholly
 * inside the interval cost nothing when it covers the start of the context.
 * A sequence with every token masked gets a zero row.  Pools are `dtype`
 * (kv_dtype == dtype, the scales ignored) or 8-bit codes (kv_dtype
 * PA_FP8_E4M3 / PA_INT8 with k_scale, v_scale, or PA_INT8_TOKEN, as
 * pa_decode_quant).  Path,
 * flags (PA_DECODE_CACHED_KV, PA_DECODE_SPLIT), workspace, *path and errors
 * as in pa_decode_quant; under PA_DEBUG only blocks with an unmasked token
 * are validated. */
pa_status pa_decode_masked(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* mask_lo,
                           const int32_t* mask_hi, const int32_t* seq_order, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t num_blocks, int32_t max_context_len, float scale, float k_scale, float v_scale,
                           pa_dtype dtype, pa_dtype kv_dtype, uint32_t flags, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, int32_t* path, void* stream);

/* Workspace of pa_decode_multi's split path: the three arrays of
 * pa_decode_split_workspace_bytes with one row per query row (num_query_tokens
 * in place of num_seqs), then one int32 per query row at the next 256-byte
 * boundary (each row's causal context length, written by the partials pass for
 * the merge).  Returns 0 on an invalid argument. */
size_t pa_decode_multi_workspace_bytes(int32_t num_query_tokens, int32_t num_heads, int32_t head_dim,
                                       int32_t max_context_len, int32_t partition_size);

/* Decode with several query tokens per sequence, causal among themselves: the
 * verification pass of speculative decoding, which [XDNF] §6.3 combines with
 * paging.  The query rows of sequence s are query_start[s] ..
 * query_start[s+1] - 1: the last L of its n = context_lens[s] tokens, whose
 * K/V are already in the pools.  Row query_start[s] + i (i < L) sits at
 * position n - L + i and attends to positions 0 .. n - L + i:
 *   out[r, h, :] = sum_{t <= n-L+i} softmax_t(scale <query[r,h], K_t>) V_t.
 *   query, out: device [num_query_tokens, num_heads, head_dim], dtype.
 *   query_start: device int32 [num_seqs + 1], from 0 to num_query_tokens,
 *     non-decreasing; every span at most max_query_len and at most n (a longer
 *     span, or L > n, gives NaN rows or no output; rejected under PA_DEBUG).
 * One launch covers every span: the q.K tile's 16 columns hold (query token,
 * head) pairs of one KV head, so each workgroup reads its KV once for up to 16
 * such pairs.  Pools, scales, kv_dtype, flags, partition_size, path choice
 * (PA_DECODE_SPLIT / auto / single without a workspace) and errors as in
 * pa_decode_masked, with pa_decode_multi_workspace_bytes for the workspace. */
pa_status pa_decode_multi(void* out, const void* query, const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                          const int32_t* seq_order, int32_t num_seqs, int32_t num_query_tokens,
                          int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                          int32_t max_context_len, float scale, float k_scale, float v_scale, pa_dtype dtype,
                          pa_dtype kv_dtype, uint32_t flags, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, int32_t* path, void* stream);

/* Workspace of pa_decode_shared: room for the three arrays of
 * pa_decode_split_workspace_bytes for num_seqs rows with partitions of an
 * eighth of max_context_len rounded up to 64 tokens (eight partitions, the
 * most a call uses); at the next 256-byte boundaries each sequence's own-token
 * partial, m and l (fp32 [num_seqs, num_heads] each) and o (fp32 [num_seqs,
 * num_heads, head_dim]); then, in the last 4 * num_seqs bytes, one int32 per
 * sequence (the prefix length its partitions covered).  A call lays the
 * three partition arrays out from the start for the partition count it picks
 * (see pa_decode_shared), at most eight.  Returns 0 on an invalid argument. */
size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t max_context_len);

/* Decode for batches whose sequences share their leading blocks: the branches
 * of parallel sampling or beam search, forked from one parent ([XDNF] §3.4
 * fork; [IMPL] §3.3: forked sequences point at the same physical blocks until
 * one of them writes).  The result is pa_decode's definition for every
 * sequence; only the reading differs.
 *   group_start: device int32 [num_groups + 1], from 0 to num_seqs, increasing:
 *     sequences group_start[g] .. group_start[g+1] - 1 form group g (at most
 *     max_group_size of them; a sequence sharing nothing is a group of one).
 *   prefix_len: device int32 [num_seqs], each member's prefix P_i,
 *     0 <= P_i <= its context length; the first ceil(P_i / bs) table entries
 *     of every member equal those of its group's row, the member with the
 *     largest P_i (the first of them), e.g. from pa_shared_prefix_groups.
 * One launch, then the merge.  The launch's first wave items read each
 * group's prefixes once: a tile of members reads up to its longest P_i
 * through the table row of the member that has it, with the members'
 * queries as the columns of the q.K tile and each member's column seeing
 * only its own first P_i tokens, into per-member partials; its remaining
 * items read each sequence's own tokens P_i .. n-1 (one wave per sequence and
 * head tile; the prefix's blocks are not read) into one more partial.  The
 * merge combines them by the log-sum-exp rule.  Each prefix is cut into P
 * partitions of max_context_len / P (rounded up to 64 tokens), one wave
 * each, P in 1..8 chosen so that the prefix items fill whole rounds of the
 * workgroups the device holds at once; PA_SHARED_PARTS=1..8 (read on every
 * call) forces P.  Every member of a group larger than max_group_size gets
 * NaN rows; sequences outside every group, or members that do not share the
 * blocks they claim, give undefined values (all of this is rejected under
 * PA_DEBUG).  Pools, scales, kv_dtype
 * and errors as in pa_decode_masked; flags: PA_DECODE_CACHED_KV only;
 * workspace: at least pa_decode_shared_workspace_bytes, 256-byte aligned. */
pa_status pa_decode_shared(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_start,
                           const int32_t* prefix_len, int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
                           float k_scale, float v_scale, pa_dtype dtype, pa_dtype kv_dtype, uint32_t flags,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ======================================================================== *
 * Quantised (8-bit) KV cache                                                *
 * ======================================================================== *
 * [XDNF] §2.3 and §6.3 store the KV cache in 8-bit integers alongside paging:
 * quantisation changes the values the pools hold, paging only how the memory
 * is organised; [IMPL] §3.4 lists int8 among the paged backend's dtypes.  The
 * pages fix neither the code format nor the scales; here:
 *   - the pools have the layouts above with 1-byte elements of kv_dtype
 *     (PA_FP8_E4M3 or PA_INT8): key codes [num_blocks, num_kv_heads,
 *     block_size, head_dim], value codes [num_blocks, num_kv_heads, head_dim,
 *     block_size];
 *   - one fp32 scale per pool: the key pool stands for decode(code) * k_scale,
 *     the value pool for decode(code) * v_scale;
 *   - a stored code is Q(x / scale), the quotient in fp32 (correctly rounded),
 *     Q rounding to nearest with ties to even.  E4M3: finite values beyond
 *     +-448 and +-inf saturate to +-448, NaN is stored as 0x7F, zeros keep
 *     their sign.  INT8: saturate to [-127, 127], NaN is stored as 0.
 * PA_INT8_TOKEN keeps a scale per (token, KV head) instead ([XDNF] §2.3/§6.3
 * name per-token int8 among the choices): each new key row and each new value
 * row of head_dim elements gets s = max |x| / 127 (fp32 division) and codes
 * Q(x / s) with Q as for PA_INT8, so its largest element is stored as +-127;
 * a row of zeros has s = 0.  Rows must be finite (a NaN row's codes and scale
 * are not specified).  The scales live in the pools themselves: each
 * (block, KV head) tile is its block_size * head_dim codes (laid out as
 * above) followed by a scale area of whole 128-byte lines
 * (PA_TOKEN_TILE_BYTES; every tile's code rows stay line-aligned), and a pool
 * is [num_blocks, num_kv_heads, PA_TOKEN_TILE_BYTES] bytes.  With
 * block_size 16 the key and value scales of a (block, KV head) share the key
 * tile's area, which is one line: the key scale of token row o at byte
 * 16 * head_dim + 4 o, its value scale at byte 16 * head_dim + 64 + 4 o, and
 * the value tile's area is unused (the decode then fetches one scale line per
 * block, not two half-used ones).  With larger blocks each tile's area holds
 * the scales of its own rows, row o's at byte block_size * head_dim + 4 o.
 * Block copies and swaps move whole tiles, scales included.  With
 * PA_INT8_TOKEN the k_scale and v_scale arguments are not used.
 * pa_copy_blocks and pa_swap_blocks copy 8-bit pools with dtype = kv_dtype. */

/* Bytes of one (block, KV head) tile of a PA_INT8_TOKEN pool. */
#define PA_TOKEN_TILE_BYTES(block_size, head_dim) \
  ((block_size) * (head_dim) + ((block_size) * 4 + 127) / 128 * 128)

/* The slot-mapping write of pa_reshape_and_cache into 8-bit pools: every
 * element of key[i, h, :] (of type dtype: PA_F32, PA_F16 or PA_BF16) is
 * quantised with k_scale and stored at key_cache[s / bs, h, s % bs, :]; value
 * rows likewise with v_scale at value_cache[s / bs, h, :, s % bs].  kv_dtype
 * selects the code format; PA_INT8_TOKEN quantises each (token, KV head) row
 * with its own scale and stores the scale in its tile (see above).  Slots,
 * skipping, races and errors as in pa_reshape_and_cache; k_scale and v_scale
 * must be finite and > 0 (PA_ERR_INVALID_ARG) unless kv_dtype is
 * PA_INT8_TOKEN.  Bit-exact (integer codes and their scales). */
pa_status pa_reshape_and_cache_quant(const void* key, const void* value, void* key_cache, void* value_cache,
                                     const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                     pa_dtype kv_dtype, float k_scale, float v_scale, void* stream);

/* Paged decode attention over 8-bit pools: pa_decode's definition with
 * K_t = decode(key code) * k_scale and V_t = decode(value code) * v_scale
 * (PA_INT8_TOKEN: times the scale of K_t's and V_t's own rows).
 * query and out are PA_F16 or PA_BF16 (dtype); the codes are widened exactly
 * to dtype on the fly, the scales folded into the logit scale and the output.
 * Path: the single pass when workspace is NULL; the split path (partials +
 * merge, as pa_decode_split) when flags has PA_DECODE_SPLIT; otherwise the
 * pa_decode_auto rule.  *path (may be NULL) receives 0 for the single pass,
 * 1 for split.  Other arguments, sizes, flags and the handling of invalid
 * device data as in pa_decode_split; k_scale and v_scale must be finite and
 * > 0 (PA_ERR_INVALID_ARG). */
pa_status pa_decode_quant(void* out, const void* query, const void* key_cache, const void* value_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* seq_order,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                          int32_t max_context_len, float scale, float k_scale, float v_scale, pa_dtype dtype,
                          pa_dtype kv_dtype, uint32_t flags, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, int32_t* path, void* stream);

/* ======================================================================== *
 * Errors and version                                                        *
 * ======================================================================== */
const char* pa_status_string(pa_status s);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* pa_last_error(void);
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
