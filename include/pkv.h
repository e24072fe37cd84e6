/*
 * pkv.h -- C ABI of libpkv.so: paged-KV-cache store and attention on MI355X
 * (gfx950).
 *
 * Pages this interface follows (titles as printed on the pages):
 *   [NV2]  "Nano-vLLM Part 2: model internals, KV cache and tensor
 *          parallelism" (seekfood.cn/news/749872)
 *   [NVE]  the Nano-vLLM engine deep-dive that opens with "from 'it runs' to
 *          'it runs well'" (mhpq.cn/news/130328)
 *   [LLM4] "LLM basics primer: from text to token, embedding, QKV and
 *          Transformer, part 4" (CSDN; qwbw.cn/news/156881)
 *
 * ---------------------------------------------------------------- layouts --
 * The pages name the cache's dimensions (block, layer, K/V, token: [NV2]
 * §05.2) but not their order.  This library takes, per layer:
 *   k_cache, v_cache  bf16 [num_blocks][num_kv_heads][block_size][head_dim]
 *                     contiguous; one (block, kv head) tile is one run of
 *                     block_size * head_dim elements.  block_size is 16,
 *                     the block size [NVE] §2.2 gives as its example.
 *   k, v (new tokens) bf16 [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping      int32 [num_tokens]; slot = physical_block * 16 + offset
 *                     ([NVE] §2.2: the cache is managed by block or by slot).
 *   q, out (decode)   bf16 [num_seqs][num_q_heads][head_dim]
 *   q, out (prefill)  bf16 [total_new][num_q_heads][head_dim], prompts packed
 *                     in order; prompt p owns rows cu_new_lens[p] ..
 *                     cu_new_lens[p+1]-1.
 *   block_tables      int32 [num_seqs][max_blocks_per_seq]: logical block i of
 *                     sequence s lives in physical block block_tables[s][i]
 *                     ([NVE] §2.2 block table; [LLM4] §17.7 logical -> physical
 *                     mapping).  Entries past a sequence's last block are never
 *                     read.  Sequences may share physical blocks (prefix
 *                     sharing, [LLM4] §17.6-17.7).
 *   context_lens      int32 [num_seqs]: cached tokens per sequence AFTER this
 *                     step's store -- decode appends the new token, then
 *                     attends over the whole cache including it ([NVE] §2.1).
 * Query head h reads KV head h / (num_q_heads / num_kv_heads): grouped-query
 * attention with contiguous groups ([LLM4] §21.1, GQA shares KV heads).
 *
 * ------------------------------------------------------------ conventions --
 * Ownership: the caller owns every buffer.  The library never allocates,
 *   frees or synchronises; every call enqueues kernels on `stream` and
 *   returns.  All pointers except `stream` are device pointers.
 * Alignment: every device pointer must be 16-byte aligned.
 * Supported: head_dim 64 or 128; block_size 16; num_q_heads a multiple of
 *   num_kv_heads with a group size of 1, 2, 4 or 8.
 * Errors: every call returns a pkv_status.  Argument errors are found on the
 *   host before anything is launched; a launch failure returns PKV_ERR_HIP.
 *   pkv_last_error() gives a one-line, thread-local description of the most
 *   recent failure on the calling thread.
 * Device-resident indices (slots, block ids, context lengths) are a caller
 *   precondition: slots unique within a call and below num_blocks * 16, block
 *   ids below num_blocks, context_lens at most max_blocks_per_seq * 16.  The
 *   kernels never touch memory outside the pools when they are violated (an
 *   out-of-range slot is not written, an out-of-range block is not read), but
 *   the output for an offending sequence is then unspecified.
 * Numerics: bf16 inputs, fp32 accumulation and softmax, bf16 output rounded
 *   to nearest even.  Slots outside a sequence's live context never
 *   influence its output, whatever bits they hold (NaN included).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,        /* a required pointer is null */
    PKV_ERR_SHAPE = 2,       /* a size is negative or inconsistent */
    PKV_ERR_UNSUPPORTED = 3, /* head_dim, block_size or group size not supported */
    PKV_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
    PKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
    PKV_ERR_HIP = 6,         /* the HIP runtime reported an error */
    PKV_ERR_CAPACITY = 7,    /* the block pool has too few free blocks */
    PKV_ERR_SEQUENCE = 8,    /* a sequence id is unknown, or already taken */
    PKV_ERR_INDEX = 9        /* a block id, context length or slot is out of range, or a
                                slot repeats (pkv_check_tables, debug-bounds builds) */
} pkv_status;

/* One layer's K and V pools.  k and v are device pointers to bf16 arrays of
 * [num_blocks][num_kv_heads][block_size][head_dim].  Placement is the
 * caller's; it matters for decode speed through the HBM channels the two
 * pools' blocks map to: on MI355X a layer's V pool right after its K pool in
 * one allocation measured up to 3% faster than V a further 2 MiB on, or than
 * all layers' K pools allocated before all their V pools. */
typedef struct {
    void *k;
    void *v;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
} pkv_cache;

/*
 * pkv_store -- append new tokens' K and V to the paged cache.
 * For every i < num_tokens with slot_mapping[i] >= 0:
 *   cache.k[slot / 16][h][slot % 16][:] = k[i][h][:]   (and the same for v)
 * for every KV head h.  A pure bit copy: stored bits equal the input bits.
 * slot_mapping[i] < 0 skips token i (padding).  Follows [NVE] §2.1 (decode
 * appends each new token's K and V to the cache) and [NV2] §05.3 (a kernel
 * writes the new K/V into the cache).
 * k, v: bf16 [num_tokens][cache.num_kv_heads][cache.head_dim], device.
 * num_tokens == 0 is a no-op.
 */
int pkv_store(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
              pkv_cache cache, hipStream_t stream);

/*
 * pkv_decode_partition_tokens -- the work split pkv_decode_attn uses when
 * passed partition_tokens = 0:
 *   -W (W in 1..8): the single-pass kernel, one workgroup of W wavefronts per
 *      (sequence, KV head); the waves split the sequence's blocks evenly and
 *      merge through LDS.  Chosen when there are at least 128 such units,
 *      max_context_len <= 8192 and no wave walks more than 1024 tokens.
 *   P > 0 (a multiple of 16): two-pass split-KV, one wavefront per (sequence,
 *      KV head, P-token partition), partials merged by a second kernel; P is
 *      chosen so that the partitions fill the GPU.
 * Returns 0 on invalid arguments.
 */
int32_t pkv_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t max_context_len);

/*
 * pkv_decode_workspace_bytes -- device scratch pkv_decode_attn needs for the
 * split-KV partials of num_seqs x num_q_heads rows with the given
 * partition_tokens.  0 for the single-pass kernel (partition_tokens < 0) and
 * when every context fits one partition.  partition_tokens = 0 sizes for the
 * two-pass split with num_kv_heads = 1, an upper bound for every head count
 * and for whichever kernel the automatic choice picks.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_tokens);

/*
 * pkv_decode_attn -- single-query attention of each sequence's new token over
 * its cached tokens, read through its block table:
 *   out[s][h][:] = softmax(scale * q[s][h] . K_s^T) V_s
 * over keys 0 .. context_lens[s]-1 of KV head h / G ([NVE] §3 formula and
 * decode shapes; [LLM4] §21.1 GQA).  The softmax subtracts the running
 * maximum before exponentiating ([NVE] §3.2).  Every wavefront serves the
 * whole query group of its KV head, so each cached K/V byte is read once.
 * partition_tokens selects the work split (see pkv_decode_partition_tokens):
 *   0 = automatic, P > 0 = two-pass split-KV with P-token partitions,
 *   -W = single-pass with W waves per (sequence, KV head).
 * A sequence with context_lens[s] == 0 gets out = 0.
 * max_context_len: host-side upper bound of context_lens (sizes the grid).
 * workspace: device scratch of at least pkv_decode_workspace_bytes(num_seqs,
 *   num_q_heads, head_dim, max_context_len, partition_tokens) bytes; may be
 *   null when that is 0.  Its contents on entry do not matter.
 */
int pkv_decode_attn(const void *q, pkv_cache cache, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                    int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                    void *workspace, size_t workspace_bytes, int32_t partition_tokens,
                    hipStream_t stream);

/*
 * pkv_decode_attn_noalloc -- pkv_decode_attn for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments minus the workspace, same kernels and
 * arithmetic (the output is bit-identical to pkv_decode_attn with the same
 * partition_tokens).  The split-KV partials go to a scratch array the library
 * owns on each GPU (a static device array of pkv_decode_noalloc_max_bytes()
 * bytes, held until the process ends); nothing is allocated or freed, and the
 * scratch needs no clearing (every partial is written before it is read).
 * Returns PKV_ERR_WORKSPACE, before any launch, when the split would need
 * more partials than the scratch holds (pkv_decode_workspace_bytes() >
 * pkv_decode_noalloc_max_bytes()); the single-pass split (partition_tokens <
 * 0) needs none.  All calls on one GPU share its scratch: calls that overlap
 * in time on one GPU (other streams, other threads) race on it.
 */
int pkv_decode_attn_noalloc(const void *q, pkv_cache cache, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                            float scale, void *out, int32_t partition_tokens,
                            hipStream_t stream);
/* Bytes of the per-GPU scratch behind pkv_decode_attn_noalloc (64 MiB). */
size_t pkv_decode_noalloc_max_bytes(void);

/*
 * pkv_store_decode_attn -- one decode step of a layer in one launch: the
 * store of each sequence's new token followed by decode attention over the
 * cache including it.  Equivalent to
 *   pkv_store(k, v, slot_mapping, num_seqs, cache, stream);
 *   pkv_decode_attn(q, cache, ..., stream);
 * ([NVE] §2.1: decode appends the new token's K and V, then attends over the
 * whole cache including it), with one new token per sequence:
 *   k, v          bf16 [num_seqs][cache.num_kv_heads][cache.head_dim], device
 *   slot_mapping  int32 [num_seqs]: sequence s's token goes to slot
 *                 slot_mapping[s] (< 0 skips the store)
 * and every other argument as for pkv_decode_attn.  Within the launch the
 * attention of sequence s takes its last position's K/V from k[s], v[s] when
 * slot_mapping[s] is the slot the block table gives that position (the usual
 * case), and from the cache otherwise.  Precondition, beyond pkv_decode_attn's:
 * a stored slot is read in this call by no position other than its own
 * sequence's last one (true whenever the slot lies in a block only its
 * sequence references, as an appended token's slot does).
 */
int pkv_store_decode_attn(const void *k, const void *v, const int32_t *slot_mapping,
                          const void *q, pkv_cache cache, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *context_lens,
                          int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                          float scale, void *out, void *workspace, size_t workspace_bytes,
                          int32_t partition_tokens, hipStream_t stream);

/*
 * pkv_store_decode_attn_rope -- pkv_store_decode_attn with the rotary
 * position embedding fused in: each sequence's q and new-token k are rotated
 * at the sequence's last position p = context_lens[s] - 1 before they are used
 * (k also before it is stored), as a model does before attention ([NVE] §3.2:
 * RoPE embeds position into Q and K, and efficient engines fuse it into the
 * attention kernel; [LLM4] §21.2: RoPE rotates Q/K inside attention).  For
 * every head row x and i < d/2, with c_i = cos_sin[p][i], s_i =
 * cos_sin[p][d/2 + i]:
 *   y[i]       = x[i] c_i - x[i + d/2] s_i
 *   y[i + d/2] = x[i + d/2] c_i + x[i] s_i
 * each product and sum rounded in fp32 (no fused multiply-add), y rounded to
 * bf16 (nearest even).  The cached K before this step must already be
 * rotated (at each token's own position).
 *   cos_sin        fp32 [max_positions][head_dim], device, 16-byte aligned
 *   max_positions  rows of the table; must be >= max_context_len (positions
 *                  are clamped into the table; an empty context rotates its
 *                  stored token at position 0)
 * Every other argument as for pkv_store_decode_attn.
 */
int pkv_store_decode_attn_rope(const void *k, const void *v, const int32_t *slot_mapping,
                               const void *q, const float *cos_sin, int32_t max_positions,
                               pkv_cache cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                               float scale, void *out, void *workspace, size_t workspace_bytes,
                               int32_t partition_tokens, hipStream_t stream);

/*
 * pkv_mixed_attn -- one continuous-batching iteration in one launch: decode
 * sequences and prefill chunks together ([NVE] §5.1-5.2: iteration-level
 * scheduling runs the running sequences' next tokens and newly admitted
 * requests as one batch; [LLM4] §17.5).  Every sequence is computed as in
 * pkv_prefill_attn -- new token i of sequence s sits at position c_s + i and
 * attends to keys 0 .. c_s + i -- and arguments have the same layout and
 * meaning, with:
 *   num_decode_seqs  sequences 0 .. num_decode_seqs-1 are decode sequences,
 *                    one new token each; they are computed as decode (the
 *                    sequence's K/V split across the waves of a workgroup).  A
 *                    sequence there with more new tokens is still computed in
 *                    full, more slowly; one with none writes nothing.
 *   num_seqs         all sequences; num_decode_seqs .. num_seqs-1 are prefill
 *                    chunks, computed as MFMA query tiles.
 *   max_new_len      bounds the prefill chunks' new tokens (decode sequences
 *                    need not count).
 *   workspace        optional (null: none).  With pkv_mixed_workspace_bytes
 *                    bytes or more, prefill chunks with long cached contexts
 *                    are split over several workgroups by key range, and a
 *                    second small launch merges their partial results; this
 *                    shortens the step when chunks are few.  No initial
 *                    contents are needed.  Calls that share a workspace must
 *                    not overlap.
 * The K/V of every new token must be stored before the call (one pkv_store
 * over the whole batch).  The result does not depend on the split beyond
 * fp32 rounding.  With num_decode_seqs = 0 this is chunked prefill that can
 * split few long-context chunks (the last chunk of a long prompt), which
 * pkv_prefill_attn runs as one workgroup per query block and KV head.
 */
int pkv_mixed_attn(const void *q, pkv_cache cache, const int32_t *block_tables,
                   int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                   const int32_t *context_lens, int32_t num_decode_seqs, int32_t num_seqs,
                   int32_t max_new_len, int32_t max_context_len, int32_t num_q_heads, float scale,
                   void *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes pkv_mixed_attn can use for these sizes (0: no split). */
size_t pkv_mixed_workspace_bytes(int32_t num_seqs, int32_t num_decode_seqs, int32_t max_new_len,
                                 int32_t max_context_len, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim);

/*
 * pkv_decode_attn_prefix -- pkv_decode_attn for a batch in which groups of
 * consecutive sequences share their first tokens through the same physical
 * blocks (prefix sharing: [LLM4] §17.6-17.7; [NVE] §2.2 prefix cache).  The
 * result is pkv_decode_attn's, up to the order of fp32 rounding; the shared
 * blocks are read once per group instead of once per sequence.  The group's
 * queries attend to the prefix together on the matrix cores (one query tile
 * per group, KV head and key range; P is rounded to bf16 in two parts, as in
 * pkv_prefill_attn), the sequences' remaining tokens are split evenly among
 * the tail waves, and a second launch merges the partial results exactly.
 *   group_starts     int32 [num_groups + 1], device: group g is sequences
 *                    group_starts[g] .. group_starts[g+1]-1 (nondecreasing,
 *                    within 0 .. num_seqs).  A sequence outside every group
 *                    shares nothing.
 *   prefix_lens      int32 [num_groups], device: tokens at the front of every
 *                    sequence of group g that lie in the same physical blocks
 *                    (rounded down to whole blocks; 0: the group shares nothing).
 *   num_groups       >= 0 (0: every sequence is computed as split-KV decode).
 *   max_group_size   host-side bound of the sizes of groups with a prefix;
 *                    sizes the grid.
 *   partition_tokens the shortest run of tail tokens one wave takes: a
 *                    positive multiple of 16, or 0 for automatic.  The tails
 *                    of all (sequence, KV head) pairs form one list that the
 *                    tail waves split evenly (runs of at least this length).
 *   num_seqs         at most 8192 (the tail list is kept in LDS).
 *   workspace        device scratch of at least
 *                    pkv_decode_prefix_workspace_bytes(num_seqs, num_q_heads,
 *                    cache.num_kv_heads, cache.head_dim, max_context_len,
 *                    partition_tokens) bytes; no initial contents needed.
 *                    Calls that share a workspace must not overlap.
 * Every other argument as for pkv_decode_attn.  Preconditions on device data
 * (not checked on the host): the first prefix_lens[g] / 16 entries of every
 * member's block-table row equal those of the group's first row (the prefix
 * is read through that row).  A sequence whose group's prefix exceeds its
 * context, or that lies beyond the first max_group_size sequences of its
 * group, gets NaN output.  pkv_prefix_groups finds valid groups from host
 * copies of the block tables.
 */
int pkv_decode_attn_prefix(const void *q, pkv_cache cache, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, const int32_t *context_lens,
                           int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                           float scale, const int32_t *group_starts, const int32_t *prefix_lens,
                           int32_t num_groups, int32_t max_group_size, void *out, void *workspace,
                           size_t workspace_bytes, int32_t partition_tokens, hipStream_t stream);

/*
 * pkv_check_tables -- host-side check of the device-resident indices of one
 * call, on host copies, before they are handed to a kernel.  The kernels
 * treat these as caller preconditions: they clamp what breaks them (an
 * out-of-range block id reads block 0, an out-of-pool slot is skipped, a
 * context past the table is cut), which keeps every access inside the pools
 * but gives plausible, wrong attention.  The block table maps each sequence's
 * logical blocks to physical ones ([NVE] §2.2; [LLM4] §17.7); this checks
 * that the mapping a batch uses is one the pools can honour:
 *   - 0 <= context_lens[s] <= max_blocks_per_seq * 16 (and <= max_context_len
 *     when max_context_len >= 0);
 *   - every block id a context reaches, block_tables[s][0 .. ceil(ctx/16)-1],
 *     lies in [0, num_blocks);
 *   - every slot_mapping[i] (num_tokens of them; slot_mapping may be null when
 *     num_tokens is 0) is negative (skip) or below num_blocks * 16, and no two
 *     non-negative slots are equal.
 * Returns PKV_OK, PKV_ERR_NULL / PKV_ERR_SHAPE for unusable arguments, or
 * PKV_ERR_INDEX for the first violation found (sequences in order, then
 * slots), described in pkv_last_error(); *bad_seq and *bad_index (either may
 * be null) then name it: (s, -1) for a context length, (s, i) for entry i of
 * row s, (-1, i) for slot i.  All pointers are host memory; nothing is
 * launched.  Cost: O(sum of blocks reached + num_tokens) plus a sort of the
 * slots.
 */
int pkv_check_tables(const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                     const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                     int32_t *bad_seq, int32_t *bad_index);

/* Workspace bytes pkv_decode_attn_prefix needs for these sizes (0 on invalid
 * arguments). */
size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_tokens);

/*
 * pkv_prefix_groups -- groups for pkv_decode_attn_prefix, from HOST copies of
 * the block tables and context lengths.  Scans the sequences in order: a run
 * starts at sequence s, takes as its prefix the whole blocks s and s + 1
 * share at the front of their rows (blocks wholly inside both contexts), and
 * extends over each next sequence that shares at least those blocks with s.
 * A run of two or more sequences whose prefix holds at least
 * min_prefix_tokens tokens (at least one block) is a group; consecutive
 * sequences in no such run form groups of prefix 0.  A batch that lists
 * requests with a common prompt next to each other ([NVE] §2.2: the prefix
 * cache hands them the same blocks) is grouped fully.
 *   group_starts    host, room for num_seqs + 1 entries
 *   prefix_lens     host, room for num_seqs entries
 *   num_groups      out: groups written
 *   max_group_size  out: the largest group with a prefix (0 if none)
 */
int pkv_prefix_groups(const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t num_seqs, int32_t min_prefix_tokens,
                      int32_t *group_starts, int32_t *prefix_lens, int32_t *num_groups,
                      int32_t *max_group_size);

/*
 * pkv_prefill_attn -- chunked causal prefill over the paged cache.  Prompt p
 * has n_p = cu_new_lens[p+1] - cu_new_lens[p] new tokens whose K/V are
 * already stored after c_p = context_lens[p] - n_p cached ones.  New token i
 * sits at position c_p + i and attends to keys 0 .. c_p + i inclusive: itself
 * and everything before it, never a later token ([NVE] §3.2 causal mask;
 * [LLM4] §22 steps 6-8).  Q K^T and P V run on the matrix cores (bf16 in, fp32
 * accumulate); the softmax runs in fp32 and P is rounded to bf16 before P V.
 * cu_new_lens: int32 [num_seqs + 1], device: cu_new_lens[0] == 0, non-decreasing,
 *   cu_new_lens[num_seqs] == rows of q and out, and n_p <= context_lens[p]
 *   (device-resident, so a caller precondition like the block ids).
 * max_new_len, max_context_len: host-side upper bounds of n_p and
 * context_lens (they size the grid).
 */
int pkv_prefill_attn(const void *q, pkv_cache cache, const int32_t *block_tables,
                     int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                     const int32_t *context_lens, int32_t num_seqs, int32_t max_new_len,
                     int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                     hipStream_t stream);

/*
 * ---------------------------------------------------------------- FP8 ----
 * An FP8 KV cache: [LLM4] §17.6 counts it at one byte per element (half of
 * BF16) among the levers on KV memory, without fixing the format or the
 * scaling.  This library uses OCP FP8 E4M3 codes (bias 7, largest finite
 * magnitude 448, subnormals, 0x7f / 0xff = NaN) with one fp32 scale per
 * (token, KV head):
 *   scale = amax / 448 over the head's head_dim values (1 if all are zero)
 *   code  = E4M3(x / scale), x / scale clamped to [-448, 448], rounded to
 *           nearest, ties to even;  both divisions correctly rounded fp32
 *   cached value = code_value * scale
 * so a cached token costs 2 x head_dim + 8 bytes per KV head (K and V).
 * Layout, per layer:
 *   k, v              uint8 codes [num_blocks][num_kv_heads][block_size][head_dim]
 *   k_scale, v_scale  fp32 [num_blocks][num_kv_heads][block_size]
 * All four pointers 16-byte aligned.
 */
typedef struct {
    void *k;
    void *v;
    float *k_scale;
    float *v_scale;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
} pkv_cache_fp8;

/*
 * pkv_store_fp8 -- pkv_store into an FP8 cache: each stored (token, KV head)
 * row of k and v (bf16, as for pkv_store) is quantized as above; its codes and
 * scale go to the slot's row.  slot_mapping[i] < 0 skips token i.
 */
int pkv_store_fp8(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                  pkv_cache_fp8 cache, hipStream_t stream);

/*
 * pkv_decode_partition_tokens_fp8 -- the automatic work split of
 * pkv_decode_attn_fp8 (same encoding as pkv_decode_partition_tokens, and at
 * present the same choice).  pkv_decode_workspace_bytes(..., 0) bounds its
 * workspace too.
 */
int32_t pkv_decode_partition_tokens_fp8(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t max_context_len);

/*
 * pkv_decode_attn_fp8 -- pkv_decode_attn over an FP8 cache: the same
 * attention on the cached values code_value * scale (bf16 q and out, fp32
 * arithmetic).  Arguments and work split as for pkv_decode_attn.
 */
int pkv_decode_attn_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                        int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                        void *workspace, size_t workspace_bytes, int32_t partition_tokens,
                        hipStream_t stream);

/*
 * pkv_prefill_attn_fp8 -- pkv_prefill_attn over an FP8 cache: the same
 * chunked causal attention ([NVE] §3.2; [LLM4] §22) on the cached values
 * code_value * scale ([LLM4] §17.6), bf16 q and out.  Q K^T and P V run on the
 * matrix cores on the codes (every E4M3 value is exactly a bf16 value); each
 * key's K scale multiplies its scores, and its V scale its weights before
 * their rounding to bf16, the weight sum adding each rounded weight over the
 * V scale.  The new tokens' codes and scales must be stored (pkv_store_fp8)
 * before the call.  Arguments, preconditions and errors as for
 * pkv_prefill_attn, with the cache as for pkv_decode_attn_fp8.
 */
int pkv_prefill_attn_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                         const int32_t *context_lens, int32_t num_seqs, int32_t max_new_len,
                         int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                         hipStream_t stream);

/*
 * pkv_mixed_attn_fp8 -- pkv_mixed_attn over an FP8 cache ([NVE] §5.1-5.2;
 * [LLM4] §17.5-17.6): the decode sequences run as pkv_decode_attn_fp8's
 * single pass with 4 waves, the prefill chunks as pkv_prefill_attn_fp8's
 * query tiles (split by key range when a workspace is given, as for
 * pkv_mixed_attn; pkv_mixed_workspace_bytes sizes it).  The new tokens'
 * codes and scales must be stored (pkv_store_fp8) before the call.
 * Arguments, preconditions and errors as for pkv_mixed_attn, with the cache
 * as for pkv_decode_attn_fp8.
 */
int pkv_mixed_attn_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                       int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                       const int32_t *context_lens, int32_t num_decode_seqs, int32_t num_seqs,
                       int32_t max_new_len, int32_t max_context_len, int32_t num_q_heads,
                       float scale, void *out, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * pkv_decode_attn_prefix_fp8 -- pkv_decode_attn_prefix over an FP8 cache
 * ([LLM4] §17.6-17.7; [NVE] §2.2): each group's shared prefix read once by the
 * FP8 query tile (MFMA on the codes, scales on the scores and weights), each
 * sequence's tail as pkv_decode_attn_fp8 reads it: on the matrix cores when the
 * sequence holds more than 128 keys and the batch has at most 379 sequences
 * (123 at head_dim 64; beyond that every tail takes the fp32 VALU path, same
 * result up to rounding).  Arguments, groups,
 * workspace (pkv_decode_prefix_workspace_bytes), preconditions and errors as
 * for pkv_decode_attn_prefix, with the cache as for pkv_decode_attn_fp8.
 */
int pkv_decode_attn_prefix_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                               float scale, const int32_t *group_starts,
                               const int32_t *prefix_lens, int32_t num_groups,
                               int32_t max_group_size, void *out, void *workspace,
                               size_t workspace_bytes, int32_t partition_tokens,
                               hipStream_t stream);

/*
 * pkv_store_decode_attn_fp8 -- pkv_store_decode_attn over an FP8 cache: the
 * store of each sequence's new token, quantized exactly as pkv_store_fp8 does
 * (codes and scale to slot_mapping[s]'s row), followed by pkv_decode_attn_fp8
 * over the cache including it, in one launch.  Equivalent to
 *   pkv_store_fp8(k, v, slot_mapping, num_seqs, cache, stream);
 *   pkv_decode_attn_fp8(q, cache, ..., stream);
 * bit for bit: where the attention takes the last position's K/V from k[s],
 * v[s] instead of the cache, it uses the quantized codes and scale it stores.
 * Arguments, work split, workspace and precondition as for
 * pkv_store_decode_attn.
 */
int pkv_store_decode_attn_fp8(const void *k, const void *v, const int32_t *slot_mapping,
                              const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                              float scale, void *out, void *workspace, size_t workspace_bytes,
                              int32_t partition_tokens, hipStream_t stream);

/*
 * pkv_kv_bytes -- KV-cache bytes for `tokens` cached tokens:
 *   2 (K and V) x layers x kv_heads x head_dim x tokens x bytes_per_elem
 * ([LLM4] §17.3 and §17.6: KV heads, not query heads; tokens summed over
 * requests).  Returns 0 for negative arguments.
 */
uint64_t pkv_kv_bytes(int32_t layers, int32_t kv_heads, int32_t head_dim, int64_t tokens,
                      int32_t bytes_per_elem);

/*
 * pkv_read_probe -- a measurement aid, not part of the attention path: one
 * kernel that streams `bytes` of device memory at `buf` with 16-byte
 * nontemporal loads, so that a benchmark can time the HBM read rate this GPU
 * reaches in the same run as the kernels it rates.
 *   buf    device pointer, 16-byte aligned; bytes a multiple of 16 (0: nothing)
 *   sink   device pointer to one uint32; written only in the unlikely case
 *          that the folded contents equal a fixed pattern (the value is of no
 *          use; it keeps the loads from being optimised away)
 * Errors: PKV_ERR_NULL, PKV_ERR_ALIGN, PKV_ERR_SHAPE (bytes not a multiple
 * of 16), PKV_ERR_HIP.  Enqueued on `stream`.
 */
int pkv_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/*
 * Debug-bounds builds.  libpkv_debug.so is the same library built with
 * PKV_DEBUG_BOUNDS: its kernels still clamp a broken device-resident index
 * (see pkv_check_tables) so that no access leaves the pools, and they also
 * record the first one they meet.  pkv_debug_status waits for the device
 * (hipDeviceSynchronize), then fills out[4] with the first violation
 * recorded since the last clear: out[0] what broke (0 none; 1 a block id
 * outside [0, num_blocks); 2 a slot past the pool; 3 a context length < 0 or
 * past the block table or max_context_len; 4 a block-copy pair outside the
 * pool), out[1] the offending value, out[2] where it was met (the sequence
 * for 2 and 3 from decode, the token for 2 from the store, the position in
 * the block-table row for 1, the pair for 4), out[3] the number of reports
 * (several threads may report one violation).  clear != 0 then resets the
 * record.  In the normal build it returns PKV_ERR_UNSUPPORTED with out
 * zeroed.  pkv_debug_bounds_enabled() is 1 in the debug build, else 0.
 */
int pkv_debug_bounds_enabled(void);
int pkv_debug_status(uint32_t out[4], int clear);

/* Static, human-readable name of a pkv_status value. */
const char *pkv_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
