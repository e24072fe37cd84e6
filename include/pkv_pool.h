/*
 * pkv_pool.h -- the physical block pool of libpkv.so (host side) and the
 * block copy that copy-on-write needs (device side).
 *
 * The pool is the control plane that produces the kernels' block tables and
 * slot mappings.  The pages describe it in prose only:
 *   - the cache is cut into uniform blocks of a fixed number of tokens, and one
 *     global pool of physical blocks serves every request: a request takes free
 *     blocks when it needs room and returns them when it ends, so there is no
 *     external fragmentation ([NVE] §2.2);
 *   - a request's block table maps its logical blocks to physical ones, which
 *     need not be contiguous ([NVE] §2.2; [LLM4] §17.7);
 *   - requests with a common prefix (a shared system prompt) point at the same
 *     physical blocks, so the prefix is held once, and writes to shared blocks
 *     go through copy-on-write; paging makes prefix caching easy ([NVE] §2.2;
 *     [LLM4] §17.6, §17.7);
 *   - one block id addresses the block in every layer's K and V pools ([NV2]
 *     §05.2).
 * Page tags as in pkv.h.
 *
 * Where the pages stop, the pool takes these rules:
 *   - sharing is by reference count: a block is free when no live sequence's
 *     table holds it;
 *   - the free list is first-in first-out (a fresh pool hands out 0, 1, 2, ...);
 *     a finished sequence returns its blocks last block first;
 *   - prefix caching (when enabled) covers full blocks: a full block is known by
 *     its tokens and the block before it (that block's id and how many times
 *     the id has been handed out), so a hit means the same whole prefix.  A
 *     freed block stays known until it is handed out again;
 *   - an n-token prompt takes at most (n - 1) / block_size blocks from the
 *     cache, so at least its last token is computed;
 *   - appending into a partly filled block that another sequence also holds
 *     (after pkv_pool_fork) moves the appender to a fresh block and reports the
 *     pair (old, new), which the caller copies with pkv_copy_blocks before the
 *     store.
 *
 * Sequence ids are caller-chosen 64-bit integers.  Token ids are opaque int32
 * values used only to recognise shared prefixes.  A pool is not thread-safe:
 * one thread (the scheduler's) owns it.  Every call returns a pkv_status;
 * PKV_ERR_CAPACITY and PKV_ERR_SEQUENCE leave the pool unchanged, and
 * pkv_last_error() describes the failure.
 */
#ifndef PKV_POOL_H
#define PKV_POOL_H

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_pool pkv_pool;

/* A pool of num_blocks blocks of block_size tokens (every block free).
 * prefix_caching != 0 enables the prefix cache.  *out receives the handle,
 * owned by the caller until pkv_pool_destroy. */
int pkv_pool_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                    pkv_pool **out);
void pkv_pool_destroy(pkv_pool *pool);

/* Admit a prompt of num_tokens (>= 1) tokens (host arrays).  slots_out
 * [num_tokens] receives each token's cache slot (block * block_size +
 * offset), or -1 for a token whose block came from the prefix cache (so
 * pkv_store skips it); *num_cached_out the number of leading tokens already
 * cached (a multiple of block_size; those tokens are the context a chunked
 * prefill starts from).  PKV_ERR_CAPACITY when the blocks it needs are not
 * free; PKV_ERR_SEQUENCE when seq_id is live. */
int pkv_pool_add_seq(pkv_pool *pool, int64_t seq_id, const int32_t *tokens, int32_t num_tokens,
                     int32_t *slots_out, int32_t *num_cached_out);

/* One decode token for each of n live sequences, in order (host arrays).
 * slots_out [n] receives each new token's slot; copies_out [n][2] receives
 * the (src, dst) pairs of the copy-on-writes, *num_copies_out their count.
 * The copies must run before the store of these tokens.  On an error at
 * sequence i the appends before it have taken effect: *num_done_out = i
 * (n on success). */
int pkv_pool_append(pkv_pool *pool, const int64_t *seq_ids, const int32_t *tokens, int32_t n,
                    int32_t *slots_out, int32_t *copies_out, int32_t *num_copies_out,
                    int32_t *num_done_out);

/* child_id shares every block of parent_id (parallel sampling). */
int pkv_pool_fork(pkv_pool *pool, int64_t parent_id, int64_t child_id);

/* The sequence ends: each of its blocks loses a reference and returns to the
 * free list when none is left. */
int pkv_pool_free_seq(pkv_pool *pool, int64_t seq_id);

/* Block tables and context lengths of n live sequences (host arrays):
 * block_tables_out [n][max_blocks_per_seq], rows padded with -1;
 * context_lens_out [n].  PKV_ERR_SHAPE when a sequence holds more than
 * max_blocks_per_seq blocks. */
int pkv_pool_block_tables(const pkv_pool *pool, const int64_t *seq_ids, int32_t n,
                          int32_t max_blocks_per_seq, int32_t *block_tables_out,
                          int32_t *context_lens_out);

/* Queries: free blocks; references to a block (-1 when out of range); tokens
 * of a sequence (-1 when unknown). */
int32_t pkv_pool_num_free(const pkv_pool *pool);
int32_t pkv_pool_refcount(const pkv_pool *pool, int32_t block);
int32_t pkv_pool_seq_len(const pkv_pool *pool, int64_t seq_id);

/*
 * pkv_copy_blocks -- copy whole physical blocks on the device: for each pair
 * (src, dst) of copies [num_copies][2] (int32, device) and each of the
 * num_pools pools, block dst becomes a byte copy of block src (copy-on-write,
 * [NVE] §2.2; [LLM4] §17.7).
 *   pools        host array of num_pools device pointers, each a pool of
 *                num_blocks blocks of block_bytes bytes, 16-byte aligned.  For
 *                a bf16 cache pass every layer's K and V pools with
 *                block_bytes = num_kv_heads * 16 * head_dim * 2; for an FP8
 *                cache call once for the code pools (... * head_dim) and once
 *                for the scale pools (num_kv_heads * 16 * 4).
 *   block_bytes  a positive multiple of 16
 * A pair with an id outside [0, num_blocks) or with src == dst copies
 * nothing.  The pairs must not depend on order (no dst twice, no dst that is
 * also a src): the pool's pairs never do.  Enqueued on `stream`.
 */
int pkv_copy_blocks(void *const *pools, int32_t num_pools, size_t block_bytes, int32_t num_blocks,
                    const int32_t *copies, int32_t num_copies, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_POOL_H */
