// pkv_internal.h -- kernel launchers behind the C ABI (host side, not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Error reporting shared by every exported entry: record a one-line,
// thread-local description for pkv_last_error() and return the status.
extern thread_local char g_last_error[512];
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();

struct StoreArgs {
    const void *k, *v;
    const int32_t *slots;
    int32_t num_tokens;
    void *k_cache, *v_cache;
    int32_t num_blocks, num_kv_heads, head_dim;
};
hipError_t launch_store(const StoreArgs &a, hipStream_t stream);

struct StoreFp8Args {
    const void *k, *v;  // bf16 [num_tokens][num_kv_heads][head_dim]
    const int32_t *slots;
    int32_t num_tokens;
    void *k_cache, *v_cache;    // fp8 codes [num_blocks][num_kv_heads][16][head_dim]
    float *k_scale, *v_scale;   // fp32 [num_blocks][num_kv_heads][16]
    int32_t num_blocks, num_kv_heads, head_dim;
};
hipError_t launch_store_fp8(const StoreFp8Args &a, hipStream_t stream);

struct DecodeArgs {
    const void *q;
    const void *k_cache, *v_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    int32_t max_blocks_per_seq, num_seqs, max_context_len;
    int32_t num_blocks, num_q_heads, num_kv_heads, head_dim;
    int32_t partition_tokens, max_parts;
    int32_t fused_waves;  // > 0: single-pass kernel with this many waves per (seq, kv head)
    float scale;
    void *out;
    float *ws_out;  // [num_seqs][num_q_heads][max_parts][head_dim]
    float *ws_ml;   // [num_seqs][num_q_heads][max_parts][2]
    // fused store (all null for plain decode): one new token per sequence,
    // k_new / v_new [num_seqs][num_kv_heads][head_dim] written at slots[s]
    // into k_store / v_store (the same pools as k_cache / v_cache)
    const void *k_new = nullptr, *v_new = nullptr;
    const int32_t *slots = nullptr;
    void *k_store = nullptr, *v_store = nullptr;
    // FP8 cache: k_cache / v_cache hold E4M3 codes, these their fp32 scales
    // [num_blocks][num_kv_heads][16]
    bool fp8 = false;
    const float *k_scale = nullptr, *v_scale = nullptr;
    // fused store into an FP8 cache: the scale arrays written (the same
    // arrays as k_scale / v_scale); k_store / v_store are the code pools
    float *k_scale_store = nullptr, *v_scale_store = nullptr;
    // rotary embedding of q and the stored token at each sequence's last
    // position: fp32 table [rope_positions][head_dim] (cos, then sin), or null
    const float *rope_table = nullptr;
    int32_t rope_positions = 0;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// Size of the file-scope device scratch of decode.hip, and its address on the
// current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void **ptr);

struct PrefillArgs {
    const void *q;
    const void *k_cache, *v_cache;
    const float *k_scale = nullptr, *v_scale = nullptr;  // FP8 cache (prefill only)
    bool fp8 = false;
    const int32_t *block_tables;
    const int32_t *cu_new_lens;
    const int32_t *context_lens;
    int32_t max_blocks_per_seq, num_seqs, max_new_len, max_context_len;
    int32_t num_blocks, num_q_heads, num_kv_heads, head_dim;
    float scale;
    void *out;
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// Most workgroups a prefill unit of a mixed step splits into (prefill_tile.h).
constexpr int kMaxSegments = 8;

// Mixed decode + prefill step (mixed.hip): sequences 0 .. num_decode-1 are
// decode sequences; max_new_len bounds the others' new tokens.
constexpr int kMixedWaves = 4;  // waves of a mixed-step workgroup (either kind)
// Workgroups of 4 waves MI355X holds at once: 256 compute units, two each at
// the mixed kernel's register and LDS use.
constexpr int kResidentWorkgroups = 512;
struct MixedArgs : PrefillArgs {
    int32_t num_decode;
    int32_t seg_slots = 1;       // workgroups a prefill unit may split into
    float *partials = nullptr;   // [prefill units][seg_slots] partial results
};
hipError_t launch_mixed(const MixedArgs &a, hipStream_t stream);
// Prefill query blocks of a mixed launch, and the bytes of one segment's
// partial result.
// The prefill query tile of the mixed and shared-prefix launches: 4 waves of
// 32 columns (32 / group tokens x the group's heads each); one segment's
// partial result of a split unit holds head_dim + 4 floats per column
// (prefill_tile.h checks both against its geometry).
constexpr int kTileWaves = 4;
constexpr int kTileCols = 32;
inline int mixed_query_blocks(int32_t max_new_len, int32_t group) {
    const int twg = kTileWaves * (kTileCols / group);
    return (max_new_len + twg - 1) / twg;
}
constexpr size_t mixed_partial_bytes(int32_t head_dim) {
    return (size_t)kTileWaves * kTileCols * (size_t)(head_dim + 4) * sizeof(float);
}

// Decode with shared prefixes (cascade.hip): group g = sequences
// group_starts[g] .. group_starts[g + 1] - 1 sharing their first
// prefix_lens[g] tokens; the tails run as partitions of partition_tokens.
struct CascadeArgs {
    const void *q;
    const void *k_cache, *v_cache;
    const float *k_scale = nullptr, *v_scale = nullptr;  // FP8 cache
    bool fp8 = false;
    const int32_t *block_tables;
    const int32_t *context_lens;
    int32_t max_blocks_per_seq, num_seqs, max_context_len;
    int32_t num_blocks, num_q_heads, num_kv_heads, head_dim;
    const int32_t *group_starts;  // device [num_groups + 1]
    const int32_t *prefix_lens;   // device [num_groups]
    int32_t num_groups, max_group_size;
    int32_t partition_tokens, max_parts;  // max_parts: tail slots per row
    int32_t tail_workgroups;              // 2 (FP8) or 6 (bf16) per compute unit
    float scale;
    void *out;
    float *ws_out;     // [num_seqs][num_q_heads][max_parts + kMaxSegments][head_dim]
    float *ws_ml;      // [num_seqs][num_q_heads][max_parts + kMaxSegments][2]
    int32_t *ws_list;  // [1 + num_seqs + 1]: the tail list's wave count and offsets
};
// Sequences of one shared-prefix decode call (the tail list's offsets live in
// the LDS of a tail workgroup).
constexpr int32_t kMaxPrefixSeqs = 8192;
// Compute units of the current device (cascade.hip; they size the tail
// workgroups of a shared-prefix decode), asked once per device; 256 when the
// runtime cannot tell.
int32_t compute_units();
hipError_t launch_cascade(const CascadeArgs &a, hipStream_t stream);
inline int cascade_prefix_qblocks(int32_t max_group_size, int32_t group) {
    const int twg = kTileWaves * (kTileCols / group);
    return max_group_size <= 0 ? 0 : (max_group_size + twg - 1) / twg;
}

// Whole-block copies (copy.hip).
constexpr int kMaxCopyPools = 64;  // pool pointers per launch (kernel arguments)
struct CopyArgs {
    void *const *pools;  // host array of num_pools device pointers
    int32_t num_pools;
    size_t block_bytes;
    int32_t num_blocks;
    const int32_t *copies;  // device [num_copies][2]
    int32_t num_copies;
    hipStream_t stream;
};
hipError_t launch_copy_blocks(const CopyArgs &a);

// The debug-bounds status words of the kernel translation units (all zero in
// a build without PKV_DEBUG_BOUNDS): copy out [4] words, optionally clear.
hipError_t debug_word_store(uint32_t *out, bool clear);
hipError_t debug_word_decode(uint32_t *out, bool clear);
hipError_t debug_word_prefill(uint32_t *out, bool clear);
hipError_t debug_word_mixed(uint32_t *out, bool clear);
hipError_t debug_word_cascade(uint32_t *out, bool clear);
hipError_t debug_word_copy(uint32_t *out, bool clear);

// Streaming read of `bytes` (a multiple of 16) at `buf`; writes at most one
// word to `sink`.
hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

}  // namespace pkv
