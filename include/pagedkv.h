/*
 * pagedkv.h — batched attention over a paged KV cache, C ABI (gfx950).
 *
 * What the library does (TensorSharp "高级功能" page):
 *  - section "连续批处理与分页 KV 缓存": the KV cache is split into fixed-size
 *    blocks taken from one shared pool, so memory is allocated per block; every
 *    full block is content-hashed and identical prefixes are shared between
 *    concurrent and later requests instead of being recomputed;
 *  - section "原生分页注意力": one native call gathers K/V out of the paged
 *    buffers for many sequences and runs attention over them, with a variant
 *    that takes per-head sink logits; the "批量前向" paragraph of that section
 *    pairs every batched forward with a paged K/V scatter-write;
 *  - section "内存优化", paged KV pool item: LRU eviction and cross-session
 *    content-hash reuse of cached blocks.
 * One call serves single-token decode rows, chunked-prefill rows (section
 * "性能优化", chunked prefill item) and speculative-verify windows (section
 * "MTP / NextN 推测解码": all drafted rows are verified in one batched forward).
 *
 * Conventions for every entry point:
 *  - Return value: KV_OK (0) or a negative KV_E* code. The message of the last
 *    failure on the calling thread is available from kv_last_error() until the
 *    next failing call on that thread. No C++ exception crosses this boundary.
 *  - On any error, out-parameters and pool state are left unchanged.
 *  - Device entry points take device pointers that the caller owns (allocated
 *    with hipMalloc or by PyTorch); they enqueue work on `hip_stream`
 *    (a hipStream_t, NULL = default stream) and return without synchronising.
 *    Buffers must stay valid until that work has completed. The library keeps
 *    no device pointer after a call returns.
 *  - Host arguments are validated before anything is enqueued. Contents of
 *    device arrays (block ids, lengths, offsets) are the caller's contract:
 *    kernels never read or write outside the buffers whose sizes the host
 *    arguments describe (out-of-range block ids are treated as empty blocks),
 *    but results for a row whose metadata breaks the contract are unspecified.
 *
 * Pool layout (the pages fix none; this is the library's interface).
 * X = 16 / sizeof(element): 8 for bf16, 4 for fp32. block_size = 16.
 *   K_pool [num_blocks][num_kv_heads][head_dim / X][block_size][X]
 *   V_pool [num_blocks][num_kv_heads][head_dim][block_size]
 * Token t of a sequence lives in physical block block_table[t / 16] at offset
 * t % 16; its slot id is block * 16 + offset. K keeps each token's 16-byte
 * pieces of the head dimension side by side across the 16 tokens of a block;
 * V is stored transposed within a block (one row of 16 tokens per channel).
 * Both make every (block, KV head) tile a contiguous 16 * head_dim element run.
 *
 * 8-bit pools (KV_FP8; "内存优化" names quantized KV blocks but fixes no codec):
 * each (token, KV head) row x of head_dim values is stored as OCP FP8 E4M3FN
 * codes c with one float32 scale s = max|x| / 448 (float32 division), the codes
 * being x / s (float32 division) clamped to [-448, 448] and rounded to the
 * nearest code, ties to the even code; a row of zeros stores s = 0 and zero
 * codes. The value the attention uses is c * s. A (block, KV head) tile is
 * 16 * head_dim code bytes followed by the 16 tokens' float32 scales
 * (16 * head_dim + 64 bytes); the pools are
 *   K_pool, V_pool [num_blocks][num_kv_heads][16 * head_dim + 64] bytes,
 * codes placed, for token t and channel c,
 *   K: c = 64 p + 32 jj + 8 g + e  at byte ((p * 4 + g) * 16 + t) * 16 + jj * 8 + e
 *   V: t = 8 h + e, c = 16 (2 d + dd) + n  at byte (((d * 16 + n) * 2 + h) * 2 + dd) * 8 + e
 * (head_dim a multiple of 64). Queries and the new K/V rows handed to
 * kv_append_scatter are bf16.
 *
 * 4-bit pools (KV_FP4; the same section's KV block codec has a 4-bit setting,
 * again with no format): each (token, KV head) row is stored as OCP FP4 E2M1
 * codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) with one
 * float32 scale s = max|x| / 6, the codes being x / s clamped to [-6, 6] and
 * rounded to the nearest code, ties to the even code (both divisions float32);
 * a row of zeros stores s = 0 and zero codes. The value used is c * s. A
 * (block, KV head) tile is 8 * head_dim code bytes, two codes a byte (the
 * even code index in the low nibble), then the 16 tokens' float32 scales;
 *   K_pool, V_pool [num_blocks][num_kv_heads][8 * head_dim + 64] bytes,
 * code index (nibble) of token t, channel c:
 *   K: c = 32 j + 8 g + e  at  ((g * 16 + t) * (head_dim / 32) + j) * 8 + e
 *   V: t = 8 h + e, c = 16 dt + n  at  ((n * 2 + h) * (head_dim / 16) + dt) * 8 + e
 * Two tokens share each V byte: writes of single tokens into a block update
 * their V nibbles atomically, so tokens of one block may be written by one
 * call or by calls on different streams.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kv_status {
    KV_OK = 0,
    KV_EINVAL = -1,        /* invalid host argument (null pointer, size, shape) */
    KV_ENOMEM = -2,        /* pool has too few free blocks */
    KV_EUNSUPPORTED = -3,  /* no kernel for this (dtype, head_dim, block_size) */
    KV_EDEVICE = -4,       /* HIP runtime reported an error at launch */
    KV_EINTERNAL = -5      /* unexpected internal failure */
};

enum kv_dtype { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2, KV_FP4 = 3 };

#define PAGEDKV_ABI_VERSION 1

/* ABI version of the loaded library (PAGEDKV_ABI_VERSION). Library plumbing:
 * no passage of the pages describes it. */
int kv_abi_version(void);

/* Message of the last failed call on this thread ("" if none). The pointer is
 * owned by the library and stays valid until the next failing call on the
 * thread. The pages describe no such call; it carries the style of failure
 * they ask for (TensorSharp "高级功能" page, "内存优化": a request the pool
 * cannot serve fails at once with an explicit message that gives the
 * numbers, instead of degrading silently), so every KV_E* code comes with
 * the sizes that caused it. */
const char *kv_last_error(void);

/* ------------------------------------------------------------------------ */
/* Host block manager (touches no device memory)                             */
/* ------------------------------------------------------------------------ */

typedef struct kv_pool kv_pool;

/*
 * Create a block manager for a caller-owned device pool of `num_blocks` blocks
 * of `block_size` tokens ("连续批处理与分页 KV 缓存": fixed-size blocks from a
 * shared pool). The free list is FIFO; it starts in `initial_free_order`
 * (a permutation of 0..num_blocks-1, copied) or in ascending order if NULL.
 * *out receives the new pool, owned by the caller and freed by
 * kv_pool_destroy. A pool is not thread-safe: callers serialise access.
 * Errors: KV_EINVAL (non-positive sizes, not a permutation, out == NULL).
 */
int kv_pool_create(int32_t num_blocks, int32_t block_size,
                   const int32_t *initial_free_order, kv_pool **out);

/* Free a pool created by kv_pool_create (NULL is ignored). */
void kv_pool_destroy(kv_pool *pool);

/*
 * Append `n_new` tokens (host array `new_token_ids`) to sequence `seq_id`
 * (created on first use) and place them in blocks ("块哈希前缀共享": every full
 * block is content-hashed and identical prefixes share physical blocks).
 *
 * Policy, in order:
 *  1. a partially filled last block of the sequence is filled in place;
 *  2. each new full block whose first token is new gets the chained hash
 *     h_j = FNV-1a-64(h_{j-1} as 8 little-endian bytes || its block_size token
 *     ids as int32 little-endian), h_{-1} = 0; if a registered block has that
 *     hash, the same token ids and the same parent block (same physical block,
 *     same reuse generation) it is shared: its refcount goes up and, if it sat
 *     unreferenced in the free list, it is taken out; its tokens get slot -1
 *     (already resident, nothing to write);
 *  3. every other block is popped from the front of the free list (a cached
 *     block that is popped loses its hash entry); a new full block is then
 *     registered under its hash unless another block already holds that hash.
 *     Partial blocks are private and unhashed until they fill up.
 * Because sharing needs an unbroken chain of shared parents, hits only happen
 * for a run of blocks that starts at a block boundary.
 *
 * Outputs (host arrays, caller-owned):
 *   block_table_row [max_blocks]: the sequence's physical block ids, -1 past
 *                                 its last block;
 *   *num_blocks: blocks used; *context_len: tokens after the append;
 *   slot_mapping [n_new]: slot id of each new token, or -1 if it is already
 *                         resident in a shared block.
 * Errors: KV_EINVAL (null pool/pointers with n_new > 0, n_new < 0, sequence
 * would need more than max_blocks blocks), KV_ENOMEM (free list too short;
 * nothing is changed).
 */
int kv_pool_alloc(kv_pool *pool, int64_t seq_id, const int32_t *new_token_ids, int32_t n_new,
                  int32_t *block_table_row, int32_t max_blocks, int32_t *num_blocks,
                  int32_t *context_len, int32_t *slot_mapping);

/*
 * Drop sequence `seq_id`. Its blocks lose one reference each, last block
 * first; blocks that reach zero go to the back of the free list and keep their
 * hash entry, so a later request with the same prefix can still share them
 * until they are popped again ("内存优化": LRU eviction, cross-session reuse).
 * Errors: KV_EINVAL (null pool, unknown sequence).
 */
int kv_pool_release(kv_pool *pool, int64_t seq_id);

/* Counts: blocks in the free list, of which still hash-addressable (cached),
 * and blocks with a nonzero refcount ("内存优化": the paged pool's LRU list
 * of cached blocks beside the blocks in use; the counts are this library's
 * observability of it, not a call the pages name). Any output pointer may be
 * NULL. */
int kv_pool_stats(const kv_pool *pool, int32_t *free_blocks, int32_t *cached_blocks,
                  int32_t *live_blocks);

/* Test hook: every block hash computed from now on is ANDed with `mask`
 * (default all ones). A narrow mask forces hash collisions, which must never
 * make two different token runs share a block, because a hit also compares
 * the token ids and the parent block. Errors: KV_EINVAL (null pool). */
int kv_pool_set_hash_mask(kv_pool *pool, uint64_t mask);

/*
 * Roll sequence `seq_id` back to its first new_len tokens, the KV side of a
 * speculative round's rollback (TensorFold page, section on the GPU accept
 * kernel: the state after the accepted path is restored, the KV cache
 * included). Blocks wholly past new_len are returned as kv_pool_release
 * returns them (last first, hash entries kept). When new_len ends inside a
 * block that was full, its later slots will be written again:
 *   - a block only this sequence holds loses its hash entry and starts a new
 *     reuse generation (no chain through its old contents can be followed);
 *   - a block other sequences hold too is replaced, in this sequence only, by
 *     a block popped from the free list: *copy_src and *copy_dst name the old
 *     and the new block, and the caller copies the old block's K/V into the
 *     new one (kv_copy_blocks) before writing to it. Otherwise both are -1.
 * The sequence's table row is then kv_pool_alloc(pool, seq_id, NULL, 0, ...)'s.
 * new_len = 0 keeps an empty sequence. Nothing changes on error.
 * Errors: KV_EINVAL (null pool or outputs, unknown sequence, new_len outside
 * 0 .. context length, new_len ending inside a dropped block), KV_ENOMEM (a
 * copy is needed and no block would be free).
 */
int kv_pool_truncate(kv_pool *pool, int64_t seq_id, int32_t new_len, int32_t *copy_src,
                     int32_t *copy_dst);

/*
 * Free the blocks of sequence `seq_id` that lie wholly below position
 * first_kept (blocks j with (j + 1) * block_size <= first_kept), for
 * sliding-window attention, whose rows never see them again (TensorSharp
 * "高级功能" page, "性能优化": sliding-window layers, prefix reuse bounded by
 * the window). Freed blocks lose one reference each, go to the back of the free
 * list when unreferenced (hash entries kept) and read -1 in the sequence's
 * table row from now on; positions keep their meaning. Blocks that later
 * become full after a freed block are not registered for sharing, and no
 * sharing is looked up for the sequence after a freed block.
 * Errors: KV_EINVAL (null pool, unknown sequence, first_kept < 0).
 */
int kv_pool_drop_prefix(kv_pool *pool, int64_t seq_id, int32_t first_kept);

/*
 * Copy whole blocks of both pools, every KV head and slot: block src[i] to
 * block dst[i], i < n (the copy kv_pool_truncate asks for). src and dst are
 * device int32 [n]; no dst may appear twice or among the src. Pools, sizes
 * and dtype as for kv_append_scatter; entries outside 0 .. num_blocks - 1
 * copy nothing. Stream-ordered, asynchronous.
 * Errors: KV_EINVAL, KV_EUNSUPPORTED, KV_EDEVICE.
 */
int kv_copy_blocks(void *k_pool, void *v_pool, const int32_t *src, const int32_t *dst, int32_t n,
                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, void *hip_stream);

/*
 * Ancestor masks of one tree window (host): bit j of masks[r] is set when
 * window row j is row r or one of its ancestors, parents[r] being -1 (the
 * token before the window) or an earlier row. These are the tree_mask words
 * paged_attention_masked_forward takes. n <= 32.
 * Errors: KV_EINVAL (null pointer, n outside 0 .. 32, a parent not in
 * -1 .. r - 1); masks is unchanged on error.
 */
int kv_tree_masks(const int32_t *parents, int32_t n, uint32_t *masks);

/*
 * The accept walk of a verify round on the device (TensorFold page, section
 * on the GPU accept kernel: each draft is compared with the target's choice
 * and the accepted path follows, from the root, the first child whose draft
 * token equals that choice). Sequence s owns window rows
 * query_start_loc[s] .. query_start_loc[s + 1]; for window row r
 * (index within the sequence) parents[qsl[s] + r] is the parent row index, or
 * -1 for the token before the window; draft_tokens[qsl[s] + r] is the row's
 * draft token and choices[qsl[s] + r] the target's token after the row;
 * root_choices[s] is the target's token after the token before the window.
 * The walk starts at the root with want = root_choices[s], moves to the first
 * row (lowest index) whose parent is the current node and whose draft token
 * is want, then takes want = that row's choice, until no such row exists.
 * Out: path[qsl[s] + k] = k-th accepted window row index (the rest of the
 * sequence's entries -1), path_len[s], bonus[s] = the final want (the target's
 * token after the accepted path). All arrays are device int32. Parents outside
 * -1 .. r - 1 give an unspecified path; the walk ends after at most q_len
 * moves whatever the input. Stream-ordered, asynchronous.
 * Errors: KV_EINVAL (null pointer, negative size), KV_EDEVICE.
 */
int kv_accept_paths(const int32_t *parents, const int32_t *draft_tokens, const int32_t *choices,
                    const int32_t *root_choices, const int32_t *query_start_loc, int32_t num_seqs,
                    int32_t *path, int32_t *path_len, int32_t *bonus, void *hip_stream);

/* ------------------------------------------------------------------------ */
/* Device entry points                                                        */
/* ------------------------------------------------------------------------ */

/*
 * Paged K/V scatter-write ("批量前向" paragraph: paged K/V scatter-write).
 * For each i < n with slot = slot_mapping[i] >= 0:
 *   K_pool[slot / 16][h][d / X][slot % 16][d % X] = k_new[i][h][d]
 *   V_pool[slot / 16][h][d][slot % 16]            = v_new[i][h][d]
 * for all h < num_kv_heads, d < head_dim: a bit copy. Slots of -1 are skipped;
 * slots outside the pool are skipped. Slots must be distinct within a call.
 * With dtype KV_FP8 or KV_FP4, k_new and v_new are bf16 and each (token,
 * head) row is quantized as described under "8-bit pools" or "4-bit pools"
 * and written with its scale.
 *   k_new, v_new  device [n][num_kv_heads][head_dim], element type `dtype`
 *                 (bf16 for KV_FP8 and KV_FP4)
 *   slot_mapping  device int32 [n]
 *   k_pool, v_pool device pools in the layout above, num_blocks blocks
 * Supported: dtype KV_BF16 or KV_F32 with head_dim a multiple of 16 up to 256;
 * KV_FP8 and KV_FP4 with head_dim 64 or 128; block_size 16.
 * Errors: KV_EINVAL, KV_EUNSUPPORTED, KV_EDEVICE.
 */
int kv_append_scatter(const void *k_new, const void *v_new, const int32_t *slot_mapping,
                      int32_t n, void *k_pool, void *v_pool, int32_t num_blocks,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t dtype, void *hip_stream);

/*
 * The producer step before attention in one pass (TensorSharp "高级功能"
 * page: a fused QK-Norm + NeoX RoPE kernel for Qwen 3.5/3.6, and the batched
 * forward's paged K/V scatter-write). For token i (position positions[i]) and
 * every head row x of q ([n][num_q_heads][head_dim]) and k
 * ([n][num_kv_heads][head_dim]), all bf16:
 *   y = x / sqrt(mean(x^2) + eps) * (weight_offset + w)   (w: q_norm_weight or
 *       k_norm_weight, bf16 [head_dim]; NULL: no weight factor)
 *   the first rotary_dim dimensions of y turn in NeoX pairs (j, j + rotary_dim/2)
 *       by the angle positions[i] * rope_theta^(-2j / rotary_dim):
 *       (a, b) -> (a cos - b sin, b cos + a sin); the rest pass through
 *   the result is rounded once to bf16 (computed in float32, the angle in float64).
 * Q rows go to q_out ([n][num_q_heads][head_dim] bf16); K rows and the v rows
 * (unchanged) go into the bf16 pools at slot_mapping[i] as kv_append_scatter
 * writes them (-1: not written). weight_offset 1 serves zero-centred norm
 * weights. Supported: dtype KV_BF16, head_dim 64, 128 or 256, block_size 16,
 * rotary_dim even, at most head_dim, rotary_dim / 2 a multiple of head_dim / 16
 * (0: no rotation). Rows, q_out and pools are 16-byte aligned.
 * Stream-ordered, asynchronous.
 * Errors: KV_EINVAL, KV_EUNSUPPORTED, KV_EDEVICE.
 */
int kv_qknorm_rope_scatter(const void *q, const void *k, const void *v, const int32_t *positions,
                           const void *q_norm_weight, const void *k_norm_weight, float eps, float weight_offset,
                           float rope_theta, int32_t rotary_dim, const int32_t *slot_mapping, int32_t n,
                           void *q_out, void *k_pool, void *v_pool, int32_t num_blocks, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                           void *hip_stream);

/*
 * Bytes of device workspace paged_attention_forward needs for these sizes
 * (0 on invalid sizes). Library plumbing, no passage: the split-K partial
 * states it sizes are this library's way of spreading long contexts over the
 * GPU, not part of what the pages describe. The workspace holds per-split partial results; its
 * contents need no initialisation and are meaningless after a call. Calls that
 * may run at the same time (different streams) need different workspaces.
 */
size_t paged_attention_workspace_size(int32_t num_seqs, int32_t total_q_rows,
                                      int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_context_len);

/*
 * Batched attention over the paged cache ("原生分页注意力"; sinks: its WithSinks
 * variant). Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]
 * (q_len rows) and context_lens[s] keys, which include its q_len new tokens
 * (scatter them first, on the same stream). Row r of s sits at position
 * p = context_lens[s] - q_len + r and attends to keys 0..p (causal, bottom-right
 * aligned: decode rows see the whole context, verify and prefill rows see the
 * keys up to themselves). Query head h reads KV head h / (num_q_heads /
 * num_kv_heads). For every row i and query head h:
 *   x_t = scale * <q[i][h], k_t>,  M = max(max_t x_t, sinks[h] if sinks),
 *   out[i][h] = sum_t e^{x_t - M} v_t / (sum_t e^{x_t - M} + e^{sinks[h] - M}),
 * the sink term present only when `sinks` is non-NULL; the sink logit is not
 * multiplied by `scale` and carries no value vector.
 *
 *   q               device [total_q_rows][num_q_heads][head_dim], type `dtype`
 *   k_pool, v_pool  device pools (layout above), type `dtype`
 *   block_tables    device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens    device int32 [num_seqs], 1 <= q_len <= context_lens[s]
 *                   <= max_context_len
 *   query_start_loc device int32 [num_seqs + 1], ascending, [0] = 0,
 *                   [num_seqs] = total_q_rows, q_len <= max_q_len
 *   num_blocks      blocks each pool holds; a block id outside
 *                   0 .. num_blocks - 1 reads as an empty block, so no
 *                   table entry can make a kernel read outside the pools
 *   sinks           device float [num_q_heads] or NULL
 *   out             device float [total_q_rows][num_q_heads][head_dim]
 *   workspace       device, >= paged_attention_workspace_size(...) bytes
 * max_q_len and max_context_len only size the launch and the workspace; they
 * never change a result. Every row's arithmetic depends only on its own query,
 * its visible keys and values, scale and sink: the same row gives the same bits
 * alone, in any batch, and inside any window (a verify window row equals the
 * same query run as a single decode row over the keys up to it).
 * Supported: head_dim 64 or 128, block_size 16, dtype KV_BF16, KV_F32,
 * KV_FP8 or KV_FP4 (q in bf16, pools of 8- or 4-bit tiles: the keys and
 * values are the stored codes times their scales).
 * Streams: every launch is ordered on hip_stream. A batch with both prefill
 * chunks (more than 32 rows per sequence and KV head) and shorter rows,
 * captured into a graph on hip_stream, runs the prefill launch on a side
 * stream the library keeps for the device (created, at default priority, by
 * the first such call made outside capture; without one the capture stays
 * on hip_stream), forked from hip_stream and joined back into it by events,
 * so the two launches run side by side in the graph. Calls made at the same
 * time from several host threads on one device must not mix a capture with
 * calls outside it: the side stream belongs to the capture until it ends.
 * Errors: KV_EINVAL, KV_EUNSUPPORTED, KV_EDEVICE.
 */
int paged_attention_forward(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *query_start_loc,
                            int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                            int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                            const float *sinks, float *out, void *workspace,
                            size_t workspace_bytes, void *hip_stream);

/*
 * paged_attention_forward for a batch whose first sequences share a prompt
 * prefix ("连续批处理与分页 KV 缓存": identical prefix blocks are shared
 * between concurrent requests through the block hash, so many sequences hold
 * one system prompt in the same physical blocks). Sequences 0 .. prefix_seqs
 * - 1 are expected to be decode rows (one query row each) whose first
 * prefix_tokens positions lie in the same physical blocks; the caller knows
 * this from the block manager (kv_pool_alloc reports those slots as
 * resident). The splits that lie wholly inside the prefix are then computed
 * once for each group of up to four such sequences, as one 16-row tile that
 * reads the shared blocks once, instead of once per sequence.
 * The result is paged_attention_forward's, bit for bit, whatever the hint:
 * every group checks the block ids of each split it takes and the rows of its
 * sequences; where they differ, or a sequence has more than one row, it
 * computes its sequences one after another over their own blocks. Other
 * arguments, ownership and errors are paged_attention_forward's;
 * prefix_seqs < 2, a prefix shorter than the first split (256 tokens), more
 * than 8 query heads per KV head, or a batch with 17 to 32 rows per sequence
 * and KV head and no longer sequence take paged_attention_forward's launch.
 * Errors also: KV_EINVAL for prefix_seqs or prefix_tokens < 0.
 */
int paged_attention_prefix_forward(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                   int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                   const float *sinks, int32_t prefix_seqs, int32_t prefix_tokens, float *out,
                                   void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * paged_attention_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, kernels and results, bit for bit, without
 * `workspace` and `workspace_bytes`. The split states live in a scratch array
 * the library holds in device memory, one per device, 64 MiB
 * (67108864 bytes), kept until the process ends; its device address is
 * looked up once per device on the first call there. The call allocates
 * nothing. Every call on one device shares that device's array, and the
 * array needs no clearing (each call writes every split state it reads), so
 * calls that may overlap on one device (different streams, or several host
 * threads) race and must be serialized by the caller. Every launch stays
 * on hip_stream (no side stream, under capture or not).
 * Errors: those of paged_attention_forward; KV_EINVAL also when the batch
 * needs more than 64 MiB of split states (paged_attention_workspace_size of
 * its sizes), with the number in the message; KV_EDEVICE when the scratch
 * array's address cannot be found.
 */
int paged_attention_forward_noalloc(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, const int32_t *query_start_loc,
                                    int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                    int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                    const float *sinks, float *out, void *hip_stream);

/*
 * One decode step's append and attention in one call ("原生分页注意力", its
 * batched-forward paragraph: the batched forward paired with a paged K/V
 * scatter-write). Row i's own token is the new token of its sequence: it sits
 * at position context_lens[s] - q_len + r (so context_lens already counts it),
 * its K/V are k_new[i], v_new[i] ([total_q_rows][num_kv_heads][head_dim],
 * type `dtype`) and its pool slot is slot_mapping[i] (-1: the token is already
 * resident, write nothing). The call equals kv_append_scatter(k_new, v_new,
 * slot_mapping, total_q_rows, ...) followed by paged_attention_forward(...) on
 * the same stream, bit for bit in `out` and in the pools. Other arguments,
 * ownership and errors are those of paged_attention_forward; k_pool and v_pool
 * are written. A bf16 batch of single-row sequences (decode) with at most 16
 * query heads per KV head writes and uses the new tokens inside the attention
 * launch; any other batch, and every
 * KV_FP8 or KV_FP4 batch (k_new, v_new in bf16), is scattered first.
 */
int paged_attention_append_forward(const void *q, const void *k_new, const void *v_new,
                                   const int32_t *slot_mapping, void *k_pool, void *v_pool, int32_t dtype,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                   int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                   const float *sinks, float *out, void *workspace, size_t workspace_bytes,
                                   void *hip_stream);

/*
 * paged_attention_forward with fewer visible keys per row.
 * Tree windows (TensorFold page, section on the GPU accept kernel: a verify
 * round lays its drafts out as a chain or a tree of at most 16 rows, the tree
 * carrying alternative paths): tree_mask is device uint32 [total_q_rows] or
 * NULL. With base = context_lens[s] - q_len, row r of sequence s sees every
 * key below base, its own key base + r, and the key base + j (j < r) when bit
 * j of tree_mask[query_start_loc[s] + r] is set; bits at or above r are
 * ignored. All bits below r set is the causal window. With a tree_mask every
 * q_len must be at most 32 (max_q_len > 32: KV_EINVAL).
 * Sliding window (TensorSharp "高级功能" page: SWA-1024 drafters in
 * "MTP / NextN 推测解码", sliding-window layers in "性能优化"):
 * sliding_window = 0 for none, else the row at position p
 * sees only keys t > p - sliding_window. Table entries of blocks that no row
 * of the call can see may be -1 (kv_pool_drop_prefix).
 * Both only remove keys; the row's own key always stays visible. With
 * tree_mask NULL and sliding_window 0 the call is paged_attention_forward.
 * Each row's result depends only on its query, its position, its visible keys,
 * scale and sink: the same row gives the same bits in any batch, and a tree
 * row equals itself in the window cut after it.
 * Other arguments, ownership and errors are those of paged_attention_forward;
 * tree_mask is 4-byte aligned; sliding_window < 0 is KV_EINVAL.
 */
int paged_attention_masked_forward(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                   int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                   const float *sinks, const uint32_t *tree_mask, int32_t sliding_window,
                                   float *out, void *workspace, size_t workspace_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
