// pkv_api.cpp -- the exported C ABI of libpkv.so (declared in include/pkv.h).
//
// Host side only: argument validation (before anything is launched), launch
// geometry, workspace sizing and error strings.  The arithmetic lives in the
// kernels (store.hip, decode.hip, prefill.hip).
#include "pkv.h"
#include "pkv_pool.h"

#include <stdarg.h>

#include <algorithm>
#include <utility>
#include <vector>
#include <stdio.h>
#include <string.h>

#include "pkv_internal.h"

namespace pkv {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return PKV_OK;
}

}  // namespace pkv

namespace {

using pkv::fail;
using pkv::g_last_error;
using pkv::ok;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int32_t kBlock = 16;

int check_cache(const pkv_cache &c) {
    if (c.num_blocks < 0 || c.num_kv_heads <= 0 || c.head_dim <= 0 || c.block_size <= 0)
        return fail(PKV_ERR_SHAPE, "cache: num_blocks %d, num_kv_heads %d, head_dim %d, block_size %d",
                    c.num_blocks, c.num_kv_heads, c.head_dim, c.block_size);
    if (c.head_dim != 64 && c.head_dim != 128)
        return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are supported", c.head_dim);
    if (c.block_size != kBlock)
        return fail(PKV_ERR_UNSUPPORTED, "block_size %d: only 16 is supported", c.block_size);
    if (c.num_blocks > 0 && (!c.k || !c.v)) return fail(PKV_ERR_NULL, "cache.k or cache.v is null");
    if (!aligned16(c.k) || !aligned16(c.v))
        return fail(PKV_ERR_ALIGN, "cache.k / cache.v must be 16-byte aligned");
    return PKV_OK;
}

// One layer's pools as the launchers see them (bf16, or FP8 codes + scales).
struct CacheDesc {
    void *k, *v;
    float *k_scale, *v_scale;
    int32_t num_blocks, num_kv_heads, head_dim, block_size;
    bool fp8;
};

CacheDesc desc_of(const pkv_cache &c) {
    return CacheDesc{c.k, c.v, nullptr, nullptr, c.num_blocks, c.num_kv_heads, c.head_dim,
                     c.block_size, false};
}

CacheDesc desc_of(const pkv_cache_fp8 &c) {
    return CacheDesc{c.k, c.v, c.k_scale, c.v_scale, c.num_blocks, c.num_kv_heads, c.head_dim,
                     c.block_size, true};
}

int check_cache(const CacheDesc &c) {
    pkv_cache plain{c.k, c.v, c.num_blocks, c.num_kv_heads, c.head_dim, c.block_size};
    int rc = check_cache(plain);
    if (rc || !c.fp8) return rc;
    if (c.num_blocks > 0 && (!c.k_scale || !c.v_scale))
        return fail(PKV_ERR_NULL, "cache.k_scale or cache.v_scale is null");
    if (!aligned16(c.k_scale) || !aligned16(c.v_scale))
        return fail(PKV_ERR_ALIGN, "cache.k_scale / cache.v_scale must be 16-byte aligned");
    return PKV_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
    if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
        return fail(PKV_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                    num_q_heads, num_kv_heads);
    const int32_t g = num_q_heads / num_kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(PKV_ERR_UNSUPPORTED, "group size %d: only 1, 2, 4 and 8 are supported", g);
    return PKV_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Partition length for split-KV decode: aim for about 16 wavefronts per CU
// (256 CUs) if every sequence had the longest context; never shorter than 4
// blocks (the fixed cost of a unit is a q load and a cross-row merge) and
// never longer than 32 blocks (so a long-context straggler is split enough:
// measured on 256 sequences of lognormal length, 512 tokens ran 10-12%
// faster than 1024).
int32_t partition_for(int64_t units, int32_t max_context_len) {
    constexpr int64_t kTargetWaves = 4096;
    constexpr int32_t kMin = 64, kMax = 512;
    if (max_context_len <= 0) return kMin;
    int64_t want = ((int64_t)max_context_len * units + kTargetWaves - 1) / kTargetWaves;
    int32_t p = kMin;
    while (p < kMax && p < want) p <<= 1;
    return p;
}

// Waves per workgroup for the single-pass kernel, or 0 when the two-pass
// split is the better choice.  Single-pass needs enough (sequence, KV head)
// units to fill the GPU by itself and contexts short enough that one
// workgroup per unit is not a straggler; it then gives each unit enough waves
// for kTargetWaves in all (1024 = four per CU; the FP8 kernels too, since
// their products moved to the matrix cores: 32 x 4096 GQA FP8 ran 49.0 us at
// 4 waves against 50.1 at 8, 53.0-56.4 at 5-7), at least
// four (one per SIMD of the compute unit a workgroup lands on) and at least
// one block per wave.  A wave of the longest context must not walk more than
// kMaxWaveTokens: with many units of mixed lengths the choice would be one
// wave per unit, and the longest sequence's lone wave the whole launch
// (measured: 256 lognormal contexts up to 6565 tokens, 361 us single-pass
// against 175 us split).  With more units than compute units, several
// workgroups share each one and the longest unit's waves set the launch
// time, so they get up to 8 waves and must walk at most kShortWaveTokens
// (measured, store + decode, us: 16 MHA sequences of U{128..2048} tokens 54.4
// at 2 waves against 49.8 at 4; 64 x 2048 GQA 100 against 88.5; 64 GQA
// sequences of U{128..4096} tokens 115 split against 110.7 at 8 waves; the
// 32 x 4096 GQA batch, 256 units, stays at 4 waves: 85.5 against 86.5 at 8).
int32_t fused_waves_for(int64_t units, int32_t max_context_len, int64_t kTargetWaves) {
    constexpr int64_t kMinUnits = 128, kComputeUnits = 256;
    constexpr int32_t kMaxContext = 8192, kMinWaves = 4, kMaxWaves = 8, kMaxWaveTokens = 1024,
                      kShortWaveTokens = 512;
    if (units < kMinUnits || max_context_len <= 0 || max_context_len > kMaxContext) return 0;
    int32_t w = (int32_t)((kTargetWaves + units - 1) / units);
    w = w < kMinWaves ? kMinWaves : (w > kMaxWaves ? kMaxWaves : w);
    int32_t limit = kMaxWaveTokens;
    if (units > kComputeUnits) {
        limit = kShortWaveTokens;
        if (ceil_div(max_context_len, w) > limit) w = kMaxWaves;
    }
    const int32_t blocks = (max_context_len + kBlock - 1) / kBlock;
    w = w > blocks ? blocks : w;
    return ceil_div(max_context_len, w) > limit ? 0 : w;
}

// pkv_prefill_attn over either cache: argument checks, then the launch.
int prefill_call(const void *q, const CacheDesc &cache, const int32_t *block_tables,
                 int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                 const int32_t *context_lens, int32_t num_seqs, int32_t max_new_len,
                 int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                 hipStream_t stream, const char *what) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_heads(num_q_heads, cache.num_kv_heads))) return rc;
    if (num_seqs < 0 || max_new_len < 0 || max_context_len < 0 || max_blocks_per_seq < 0)
        return fail(PKV_ERR_SHAPE, "num_seqs %d, max_new_len %d, max_context_len %d", num_seqs,
                    max_new_len, max_context_len);
    if (num_seqs == 0 || max_new_len == 0) return ok();
    if (max_new_len > max_context_len)
        return fail(PKV_ERR_SHAPE, "max_new_len %d exceeds max_context_len %d", max_new_len,
                    max_context_len);
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
        return fail(PKV_ERR_SHAPE, "max_context_len %d exceeds max_blocks_per_seq %d x 16",
                    max_context_len, max_blocks_per_seq);
    if (cache.num_blocks == 0)
        return fail(PKV_ERR_SHAPE, "an empty pool cannot hold a context of %d tokens",
                    max_context_len);
    if (!q || !out || !context_lens || !cu_new_lens || !block_tables)
        return fail(PKV_ERR_NULL, "q, out, cu_new_lens, context_lens or block_tables is null");
    if (!aligned16(q) || !aligned16(out))
        return fail(PKV_ERR_ALIGN, "q / out must be 16-byte aligned");
    if (num_seqs > 65535 || cache.num_kv_heads > 65535)
        return fail(PKV_ERR_SHAPE, "num_seqs %d / num_kv_heads %d exceed one launch's grid",
                    num_seqs, cache.num_kv_heads);
    pkv::PrefillArgs a{};
    a.q = q;
    a.k_cache = cache.k;
    a.v_cache = cache.v;
    a.k_scale = cache.k_scale;
    a.v_scale = cache.v_scale;
    a.fp8 = cache.fp8;
    a.block_tables = block_tables;
    a.cu_new_lens = cu_new_lens;
    a.context_lens = context_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.max_new_len = max_new_len;
    a.max_context_len = max_context_len;
    a.num_blocks = cache.num_blocks;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache.num_kv_heads;
    a.head_dim = cache.head_dim;
    a.scale = scale;
    a.out = out;
    return hip_status(pkv::launch_prefill(a, stream), what);
}

}  // namespace

namespace {

// Split geometry of a mixed launch: how many workgroups a prefill unit may
// use, and the workspace that needs (0 when units are not split).  Units are
// split only when there are fewer of them than compute units (256) and their
// contexts are long: up to one segment per 512 keys of max_context_len (the
// smallest segment the kernel makes), at most 8.  With more units the GPU is already full and a split only adds the
// partial results' traffic and the merge launch (measured: 4 chunks x 8 KV
// heads x 16 query blocks ran 219 us split against 229 us whole, merge
// included, while one 64-token chunk after 4032 cached keys is one
// workgroup's walk over 64 key chunks per KV head).
struct MixedSplit {
    int64_t units = 0;
    int32_t slots = 1;
    size_t bytes = 0;
};

MixedSplit mixed_split(int32_t num_seqs, int32_t num_decode_seqs, int32_t max_new_len,
                       int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim) {
    MixedSplit m;
    if (num_seqs <= num_decode_seqs || max_new_len <= 0 || num_kv_heads <= 0 ||
        num_q_heads < num_kv_heads)
        return m;
    m.units = (int64_t)(num_seqs - num_decode_seqs) * num_kv_heads *
              pkv::mixed_query_blocks(max_new_len, num_q_heads / num_kv_heads);
    const int64_t by_ctx = ((int64_t)max_context_len + 511) / 512;
    const int64_t by_fill = (256 + m.units - 1) / m.units;
    m.slots = (int32_t)std::max<int64_t>(1, std::min<int64_t>(pkv::kMaxSegments, std::min(by_ctx, by_fill)));
    if (m.slots > 1) m.bytes = (size_t)m.units * m.slots * pkv::mixed_partial_bytes(head_dim);
    return m;
}

// pkv_mixed_attn over either cache: argument checks, the split, the launch.
int mixed_call(const void *q, const CacheDesc &cache, const int32_t *block_tables,
               int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
               const int32_t *context_lens, int32_t num_decode_seqs, int32_t num_seqs,
               int32_t max_new_len, int32_t max_context_len, int32_t num_q_heads, float scale,
               void *out, void *workspace, size_t workspace_bytes, hipStream_t stream,
               const char *what) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_heads(num_q_heads, cache.num_kv_heads))) return rc;
    if (num_seqs < 0 || num_decode_seqs < 0 || num_decode_seqs > num_seqs || max_new_len < 0 ||
        max_context_len < 0 || max_blocks_per_seq < 0)
        return fail(PKV_ERR_SHAPE, "num_decode_seqs %d, num_seqs %d, max_new_len %d, max_context_len %d",
                    num_decode_seqs, num_seqs, max_new_len, max_context_len);
    if (num_seqs == 0) return ok();
    if (max_new_len > max_context_len)
        return fail(PKV_ERR_SHAPE, "max_new_len %d exceeds max_context_len %d", max_new_len,
                    max_context_len);
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
        return fail(PKV_ERR_SHAPE, "max_context_len %d exceeds max_blocks_per_seq %d x 16",
                    max_context_len, max_blocks_per_seq);
    if (cache.num_blocks == 0)
        return fail(PKV_ERR_SHAPE, "an empty pool cannot hold a context of %d tokens",
                    max_context_len);
    if (!q || !out || !context_lens || !cu_new_lens || !block_tables)
        return fail(PKV_ERR_NULL, "q, out, cu_new_lens, context_lens or block_tables is null");
    if (!aligned16(q) || !aligned16(out))
        return fail(PKV_ERR_ALIGN, "q / out must be 16-byte aligned");
    // the largest grid any group size and split can make: query blocks hold at
    // least 16 tokens (group 8), a unit splits into at most kMaxSegments
    // workgroups, and the merge launch uses at most that many per unit
    const int64_t nqb = (max_new_len + 15) / 16;
    if ((int64_t)num_decode_seqs * cache.num_kv_heads +
            (int64_t)(num_seqs - num_decode_seqs) * cache.num_kv_heads * nqb * pkv::kMaxSegments >
        INT32_MAX)
        return fail(PKV_ERR_SHAPE, "%d sequences of up to %d new tokens exceed one launch's grid",
                    num_seqs, max_new_len);
    pkv::MixedArgs a{};
    a.q = q;
    a.k_cache = cache.k;
    a.v_cache = cache.v;
    a.k_scale = cache.k_scale;
    a.v_scale = cache.v_scale;
    a.fp8 = cache.fp8;
    a.block_tables = block_tables;
    a.cu_new_lens = cu_new_lens;
    a.context_lens = context_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.max_new_len = max_new_len;
    a.max_context_len = max_context_len;
    a.num_blocks = cache.num_blocks;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache.num_kv_heads;
    a.head_dim = cache.head_dim;
    a.scale = scale;
    a.out = out;
    a.num_decode = num_decode_seqs;
    if (workspace) {  // without one, prefill units run whole
        const MixedSplit m = mixed_split(num_seqs, num_decode_seqs, max_new_len, max_context_len,
                                         num_q_heads, cache.num_kv_heads, cache.head_dim);
        if (m.slots > 1) {
            if (workspace_bytes < m.bytes)
                return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                            m.bytes);
            if (!aligned16(workspace))
                return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
            a.seg_slots = m.slots;
            a.partials = static_cast<float *>(workspace);
        }
    }
    return hip_status(pkv::launch_mixed(a, stream), what);
}


}  // namespace

extern "C" {

size_t pkv_mixed_workspace_bytes(int32_t num_seqs, int32_t num_decode_seqs, int32_t max_new_len,
                                 int32_t max_context_len, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim) {
    if (num_seqs < 0 || num_decode_seqs < 0 || num_decode_seqs > num_seqs || max_new_len < 0 ||
        max_context_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0 || (head_dim != 64 && head_dim != 128))
        return 0;
    return mixed_split(num_seqs, num_decode_seqs, max_new_len, max_context_len, num_q_heads,
                       num_kv_heads, head_dim).bytes;
}

int pkv_mixed_attn(const void *q, pkv_cache cache, const int32_t *block_tables,
                   int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                   const int32_t *context_lens, int32_t num_decode_seqs, int32_t num_seqs,
                   int32_t max_new_len, int32_t max_context_len, int32_t num_q_heads, float scale,
                   void *out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return mixed_call(q, desc_of(cache), block_tables, max_blocks_per_seq, cu_new_lens,
                      context_lens, num_decode_seqs, num_seqs, max_new_len, max_context_len,
                      num_q_heads, scale, out, workspace, workspace_bytes, stream,
                      "pkv_mixed_attn launch");
}

int pkv_mixed_attn_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                       int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                       const int32_t *context_lens, int32_t num_decode_seqs, int32_t num_seqs,
                       int32_t max_new_len, int32_t max_context_len, int32_t num_q_heads,
                       float scale, void *out, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    return mixed_call(q, desc_of(cache), block_tables, max_blocks_per_seq, cu_new_lens,
                      context_lens, num_decode_seqs, num_seqs, max_new_len, max_context_len,
                      num_q_heads, scale, out, workspace, workspace_bytes, stream,
                      "pkv_mixed_attn_fp8 launch");
}

int pkv_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    if (bytes == 0) return ok();
    if (!buf || !sink) return fail(PKV_ERR_NULL, "buf or sink is null");
    if (!aligned16(buf)) return fail(PKV_ERR_ALIGN, "buf must be 16-byte aligned");
    if (bytes % 16 != 0) return fail(PKV_ERR_SHAPE, "bytes %zu is not a multiple of 16", bytes);
    return hip_status(pkv::launch_read_probe(buf, bytes, sink, stream), "pkv_read_probe launch");
}

int pkv_copy_blocks(void *const *pools, int32_t num_pools, size_t block_bytes, int32_t num_blocks,
                    const int32_t *copies, int32_t num_copies, hipStream_t stream) {
    if (num_pools < 0 || num_blocks < 0 || num_copies < 0)
        return fail(PKV_ERR_SHAPE, "num_pools %d, num_blocks %d, num_copies %d", num_pools,
                    num_blocks, num_copies);
    if (num_pools == 0 || num_copies == 0) return ok();
    if (!pools || !copies) return fail(PKV_ERR_NULL, "pools or copies is null");
    if (block_bytes == 0 || block_bytes % 16 != 0)
        return fail(PKV_ERR_SHAPE, "block_bytes %zu: a positive multiple of 16", block_bytes);
    if (!aligned16(copies)) return fail(PKV_ERR_ALIGN, "copies must be 16-byte aligned");
    for (int32_t i = 0; i < num_pools; ++i) {
        if (!pools[i]) return fail(PKV_ERR_NULL, "pools[%d] is null", i);
        if (!aligned16(pools[i])) return fail(PKV_ERR_ALIGN, "pools[%d] is not 16-byte aligned", i);
    }
    const size_t chunks = (block_bytes + 4095) / 4096;  // the finest chunking a launch uses
    if (chunks * (size_t)num_copies > (size_t)INT32_MAX)
        return fail(PKV_ERR_SHAPE, "%d copies of %zu-byte blocks: too many workgroups", num_copies,
                    block_bytes);
    pkv::CopyArgs a{pools, num_pools, block_bytes, num_blocks, copies, num_copies, stream};
    const hipError_t e = pkv::launch_copy_blocks(a);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_copy_blocks launch: %s", hipGetErrorString(e));
    return ok();
}

const char *pkv_status_string(int status) {
    switch (status) {
        case PKV_OK: return "PKV_OK";
        case PKV_ERR_NULL: return "PKV_ERR_NULL: a required pointer is null";
        case PKV_ERR_SHAPE: return "PKV_ERR_SHAPE: a size is negative or inconsistent";
        case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: head_dim, block_size or group size not supported";
        case PKV_ERR_ALIGN: return "PKV_ERR_ALIGN: a device pointer is not 16-byte aligned";
        case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: workspace missing or too small";
        case PKV_ERR_HIP: return "PKV_ERR_HIP: the HIP runtime reported an error";
        case PKV_ERR_CAPACITY: return "PKV_ERR_CAPACITY: not enough free blocks in the pool";
        case PKV_ERR_SEQUENCE: return "PKV_ERR_SEQUENCE: unknown or duplicate sequence id";
        case PKV_ERR_INDEX:
            return "PKV_ERR_INDEX: a block id, context length or slot is out of range, or a slot repeats";
        default: return "unknown pkv status";
    }
}

const char *pkv_last_error(void) { return g_last_error; }

uint64_t pkv_kv_bytes(int32_t layers, int32_t kv_heads, int32_t head_dim, int64_t tokens,
                      int32_t bytes_per_elem) {
    if (layers < 0 || kv_heads < 0 || head_dim < 0 || tokens < 0 || bytes_per_elem < 0) return 0;
    return 2ull * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim * (uint64_t)tokens *
           (uint64_t)bytes_per_elem;
}

int pkv_store(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
              pkv_cache cache, hipStream_t stream) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if (num_tokens < 0) return fail(PKV_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
    if (num_tokens == 0) return ok();
    if (!k || !v || !slot_mapping) return fail(PKV_ERR_NULL, "k, v or slot_mapping is null");
    if (!aligned16(k) || !aligned16(v))
        return fail(PKV_ERR_ALIGN, "k / v must be 16-byte aligned");
    const int64_t total = (int64_t)num_tokens * cache.num_kv_heads * (cache.head_dim / 8);
    if (total > (int64_t)0x7f000000)
        return fail(PKV_ERR_SHAPE, "store of %d tokens is too large for one call", num_tokens);
    pkv::StoreArgs a{k, v, slot_mapping, num_tokens, cache.k, cache.v, cache.num_blocks,
                     cache.num_kv_heads, cache.head_dim};
    return hip_status(pkv::launch_store(a, stream), "pkv_store launch");
}

}  // extern "C"

namespace {

int32_t auto_split(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len, bool fp8) {
    if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0) return 0;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    (void)fp8;  // the same split for both caches
    const int32_t w = fused_waves_for(units, max_context_len, 1024);
    if (w > 0) return -w;
    return partition_for(units, max_context_len);
}

}  // namespace

extern "C" {

int32_t pkv_decode_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t max_context_len) {
    return auto_split(num_seqs, num_kv_heads, max_context_len, false);
}

int32_t pkv_decode_partition_tokens_fp8(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t max_context_len) {
    return auto_split(num_seqs, num_kv_heads, max_context_len, true);
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_tokens) {
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
    if (partition_tokens < 0) return 0;  // single-pass: no partials
    if (partition_tokens % kBlock != 0) return 0;
    const int32_t p = partition_tokens ? partition_tokens : partition_for(num_seqs, max_context_len);
    const int32_t parts = ceil_div(max_context_len, p);
    if (parts <= 1) return 0;
    return (size_t)num_seqs * num_q_heads * parts * (size_t)(head_dim + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// Shared by pkv_decode_attn and pkv_store_decode_attn: validation, the work
// split and the launch.  `fused` carries the store's k, v and slots (all null
// for plain decode).
int decode_call(const void *q, const CacheDesc &cache, const int32_t *block_tables,
                int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                void *workspace, size_t workspace_bytes, int32_t partition_tokens,
                hipStream_t stream, const void *k_new, const void *v_new, const int32_t *slots,
                const char *what, const float *rope_table = nullptr,
                int32_t rope_positions = 0, bool library_scratch = false) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_heads(num_q_heads, cache.num_kv_heads))) return rc;
    if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0)
        return fail(PKV_ERR_SHAPE, "num_seqs %d, max_context_len %d, max_blocks_per_seq %d",
                    num_seqs, max_context_len, max_blocks_per_seq);
    if (num_seqs == 0) return ok();
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
        return fail(PKV_ERR_SHAPE, "max_context_len %d exceeds max_blocks_per_seq %d x 16",
                    max_context_len, max_blocks_per_seq);
    if (max_context_len > 0 && cache.num_blocks == 0)
        return fail(PKV_ERR_SHAPE, "an empty pool cannot hold a context of %d tokens",
                    max_context_len);
    if (!q || !out || !context_lens || (max_blocks_per_seq > 0 && !block_tables))
        return fail(PKV_ERR_NULL, "q, out, context_lens or block_tables is null");
    if (!aligned16(q) || !aligned16(out))
        return fail(PKV_ERR_ALIGN, "q / out must be 16-byte aligned");
    if (partition_tokens < -8 || (partition_tokens > 0 && partition_tokens % kBlock != 0))
        return fail(PKV_ERR_SHAPE,
                    "partition_tokens %d is neither a positive multiple of 16, 0, nor -1..-8",
                    partition_tokens);
    const int32_t choice =
        partition_tokens ? partition_tokens
                         : auto_split(num_seqs, cache.num_kv_heads, max_context_len, cache.fp8);
    const int32_t fused = choice < 0 ? -choice : 0;
    const int32_t p = choice > 0 ? choice : kBlock;
    const int32_t parts = fused ? 1 : (max_context_len > 0 ? ceil_div(max_context_len, p) : 1);
    const size_t need =
        fused ? 0 : pkv_decode_workspace_bytes(num_seqs, num_q_heads, cache.head_dim, max_context_len, p);
    if (library_scratch && need > 0) {  // the partials go to the library's own array
        if (need > pkv::kNoAllocScratchBytes)
            return fail(PKV_ERR_WORKSPACE,
                        "the split needs %zu bytes of partials, more than the library's %zu-byte "
                        "scratch: use pkv_decode_attn with a workspace, or longer partitions",
                        need, pkv::kNoAllocScratchBytes);
        hipError_t e = pkv::noalloc_scratch(&workspace);
        if (e != hipSuccess)
            return fail(PKV_ERR_HIP, "%s: scratch address: %s", what, hipGetErrorString(e));
        workspace_bytes = pkv::kNoAllocScratchBytes;
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (need > 0 && !aligned16(workspace))
        return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
    if ((int64_t)num_seqs * num_q_heads * parts > (int64_t)0x7fffffff / 256)
        return fail(PKV_ERR_SHAPE, "too many partitions for one call");
    if (num_seqs > 65535 || cache.num_kv_heads > 65535)
        return fail(PKV_ERR_SHAPE, "num_seqs %d / num_kv_heads %d exceed one launch's grid",
                    num_seqs, cache.num_kv_heads);

    pkv::DecodeArgs a{};
    a.q = q;
    a.k_cache = cache.k;
    a.v_cache = cache.v;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.max_context_len = max_context_len;
    a.num_blocks = cache.num_blocks;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache.num_kv_heads;
    a.head_dim = cache.head_dim;
    a.partition_tokens = p;
    a.max_parts = parts;
    a.fused_waves = fused;
    a.scale = scale;
    a.out = out;
    float *ws = static_cast<float *>(workspace);
    a.ws_out = need ? ws : nullptr;
    a.ws_ml = need ? ws + (size_t)num_seqs * num_q_heads * parts * cache.head_dim : nullptr;
    a.rope_table = rope_table;
    a.rope_positions = rope_positions;
    a.fp8 = cache.fp8;
    a.k_scale = cache.k_scale;
    a.v_scale = cache.v_scale;
    if (slots != nullptr) {
        a.k_new = k_new;
        a.v_new = v_new;
        a.slots = slots;
        a.k_store = cache.k;
        a.v_store = cache.v;
        a.k_scale_store = cache.k_scale;
        a.v_scale_store = cache.v_scale;
    }
    return hip_status(pkv::launch_decode(a, stream), what);
}

}  // namespace

extern "C" {

int pkv_decode_attn(const void *q, pkv_cache cache, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                    int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                    void *workspace, size_t workspace_bytes, int32_t partition_tokens,
                    hipStream_t stream) {
    return decode_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                       workspace_bytes, partition_tokens, stream, nullptr, nullptr, nullptr,
                       "pkv_decode_attn launch");
}

int pkv_decode_attn_noalloc(const void *q, pkv_cache cache, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                            float scale, void *out, int32_t partition_tokens,
                            hipStream_t stream) {
    return decode_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, out, nullptr, 0,
                       partition_tokens, stream, nullptr, nullptr, nullptr,
                       "pkv_decode_attn_noalloc launch", nullptr, 0, true);
}

size_t pkv_decode_noalloc_max_bytes(void) { return pkv::kNoAllocScratchBytes; }

int pkv_store_decode_attn(const void *k, const void *v, const int32_t *slot_mapping,
                          const void *q, pkv_cache cache, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *context_lens,
                          int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                          float scale, void *out, void *workspace, size_t workspace_bytes,
                          int32_t partition_tokens, hipStream_t stream) {
    if (num_seqs > 0 && (!k || !v || !slot_mapping))
        return fail(PKV_ERR_NULL, "k, v or slot_mapping is null");
    if (!aligned16(k) || !aligned16(v))
        return fail(PKV_ERR_ALIGN, "k / v must be 16-byte aligned");
    return decode_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                       workspace_bytes, partition_tokens, stream, k, v, slot_mapping,
                       "pkv_store_decode_attn launch");
}

int pkv_store_decode_attn_rope(const void *k, const void *v, const int32_t *slot_mapping,
                               const void *q, const float *cos_sin, int32_t max_positions,
                               pkv_cache cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                               float scale, void *out, void *workspace, size_t workspace_bytes,
                               int32_t partition_tokens, hipStream_t stream) {
    if (num_seqs > 0 && (!k || !v || !slot_mapping || !cos_sin))
        return fail(PKV_ERR_NULL, "k, v, slot_mapping or cos_sin is null");
    if (!aligned16(k) || !aligned16(v) || !aligned16(cos_sin))
        return fail(PKV_ERR_ALIGN, "k / v / cos_sin must be 16-byte aligned");
    if (num_seqs > 0 && (max_positions <= 0 || max_context_len > max_positions))
        return fail(PKV_ERR_SHAPE, "max_positions %d must cover max_context_len %d",
                    max_positions, max_context_len);
    return decode_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                       workspace_bytes, partition_tokens, stream, k, v, slot_mapping,
                       "pkv_store_decode_attn_rope launch", cos_sin, max_positions);
}

int pkv_decode_attn_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                        int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                        void *workspace, size_t workspace_bytes, int32_t partition_tokens,
                        hipStream_t stream) {
    return decode_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                       workspace_bytes, partition_tokens, stream, nullptr, nullptr, nullptr,
                       "pkv_decode_attn_fp8 launch");
}

int pkv_store_decode_attn_fp8(const void *k, const void *v, const int32_t *slot_mapping,
                              const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                              float scale, void *out, void *workspace, size_t workspace_bytes,
                              int32_t partition_tokens, hipStream_t stream) {
    if (num_seqs > 0 && (!k || !v || !slot_mapping))
        return fail(PKV_ERR_NULL, "k, v or slot_mapping is null");
    if (!aligned16(k) || !aligned16(v))
        return fail(PKV_ERR_ALIGN, "k / v must be 16-byte aligned");
    return decode_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, out, workspace,
                       workspace_bytes, partition_tokens, stream, k, v, slot_mapping,
                       "pkv_store_decode_attn_fp8 launch");
}

int pkv_store_fp8(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                  pkv_cache_fp8 cache, hipStream_t stream) {
    int rc = check_cache(desc_of(cache));
    if (rc) return rc;
    if (num_tokens < 0) return fail(PKV_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
    if (num_tokens == 0) return ok();
    if (!k || !v || !slot_mapping) return fail(PKV_ERR_NULL, "k, v or slot_mapping is null");
    if (!aligned16(k) || !aligned16(v))
        return fail(PKV_ERR_ALIGN, "k / v must be 16-byte aligned");
    const int64_t threads = (int64_t)num_tokens * cache.num_kv_heads * (cache.head_dim / 8);
    if (threads > (int64_t)0x7f000000)
        return fail(PKV_ERR_SHAPE, "store of %d tokens is too large for one call", num_tokens);
    pkv::StoreFp8Args a{k, v, slot_mapping, num_tokens, cache.k, cache.v, cache.k_scale,
                        cache.v_scale, cache.num_blocks, cache.num_kv_heads, cache.head_dim};
    return hip_status(pkv::launch_store_fp8(a, stream), "pkv_store_fp8 launch");
}

int pkv_prefill_attn(const void *q, pkv_cache cache, const int32_t *block_tables,
                     int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                     const int32_t *context_lens, int32_t num_seqs, int32_t max_new_len,
                     int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                     hipStream_t stream) {
    return prefill_call(q, desc_of(cache), block_tables, max_blocks_per_seq, cu_new_lens,
                        context_lens, num_seqs, max_new_len, max_context_len, num_q_heads, scale,
                        out, stream, "pkv_prefill_attn launch");
}

int pkv_prefill_attn_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *cu_new_lens,
                         const int32_t *context_lens, int32_t num_seqs, int32_t max_new_len,
                         int32_t max_context_len, int32_t num_q_heads, float scale, void *out,
                         hipStream_t stream) {
    return prefill_call(q, desc_of(cache), block_tables, max_blocks_per_seq, cu_new_lens,
                        context_lens, num_seqs, max_new_len, max_context_len, num_q_heads, scale,
                        out, stream, "pkv_prefill_attn_fp8 launch");
}

}  // extern "C"

namespace {

// Tail partition length of pkv_decode_attn_prefix (one wave's work for one
// KV head): the split-KV choice for the longest context, at most 256 tokens
// (a tail is usually much shorter than its context; measured on 256
// sequences in 8 groups sharing 2048-token prefixes with lognormal tails,
// store + prefix decode per step: 211.9-213.1 us at 256 against 222.2-222.7
// us at 512 and 227.4 us at 128).
int32_t prefix_partition_for(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
    return std::min<int32_t>(256, partition_for((int64_t)num_seqs * num_kv_heads, max_context_len));
}

// Tail slots of a workspace row: a unit's tail of up to max_context_len
// tokens falls into at most ceil(max_context_len / p) + 1 pieces when every
// wave's run of the tail list is at least p tokens.
int32_t prefix_tail_slots(int32_t max_context_len, int32_t p) {
    return max_context_len > 0 ? ceil_div(max_context_len, p) + 1 : 0;
}

// The tail list the merge reads: its wave count and num_seqs + 1 offsets,
// rounded up to 16 bytes.
size_t prefix_list_bytes(int32_t num_seqs) {
    return ((size_t)num_seqs + 2) * sizeof(int32_t) + 15 & ~(size_t)15;
}


// Leading block-table entries rows a and b share, among the first `limit`.
int32_t common_blocks(const int32_t *a, const int32_t *b, int32_t limit) {
    int32_t i = 0;
    while (i < limit && a[i] == b[i]) ++i;
    return i;
}

// pkv_decode_attn_prefix over either cache: argument checks, the sizing, the launch.
int prefix_call(const void *q, const CacheDesc &cache, const int32_t *block_tables,
                int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                int32_t max_context_len, int32_t num_q_heads, float scale,
                const int32_t *group_starts, const int32_t *prefix_lens, int32_t num_groups,
                int32_t max_group_size, void *out, void *workspace, size_t workspace_bytes,
                int32_t partition_tokens, hipStream_t stream, const char *what) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_heads(num_q_heads, cache.num_kv_heads))) return rc;
    if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0 || num_groups < 0 ||
        max_group_size < 0)
        return fail(PKV_ERR_SHAPE,
                    "num_seqs %d, max_context_len %d, max_blocks_per_seq %d, num_groups %d, "
                    "max_group_size %d",
                    num_seqs, max_context_len, max_blocks_per_seq, num_groups, max_group_size);
    if (num_seqs == 0) return ok();
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlock)
        return fail(PKV_ERR_SHAPE, "max_context_len %d exceeds max_blocks_per_seq %d x 16",
                    max_context_len, max_blocks_per_seq);
    if (max_context_len > 0 && cache.num_blocks == 0)
        return fail(PKV_ERR_SHAPE, "an empty pool cannot hold a context of %d tokens",
                    max_context_len);
    if (max_group_size > num_seqs)
        return fail(PKV_ERR_SHAPE, "max_group_size %d exceeds num_seqs %d", max_group_size,
                    num_seqs);
    if (num_seqs > pkv::kMaxPrefixSeqs)
        return fail(PKV_ERR_SHAPE, "%d sequences exceed the %d of one shared-prefix call",
                    num_seqs, pkv::kMaxPrefixSeqs);
    if (!q || !out || !context_lens || (max_blocks_per_seq > 0 && !block_tables))
        return fail(PKV_ERR_NULL, "q, out, context_lens or block_tables is null");
    if (num_groups > 0 && (!group_starts || !prefix_lens))
        return fail(PKV_ERR_NULL, "group_starts or prefix_lens is null");
    if (!aligned16(q) || !aligned16(out))
        return fail(PKV_ERR_ALIGN, "q / out must be 16-byte aligned");
    if (partition_tokens < 0 || partition_tokens % kBlock != 0)
        return fail(PKV_ERR_SHAPE, "partition_tokens %d is neither 0 nor a positive multiple of 16",
                    partition_tokens);
    const int32_t p = partition_tokens
                          ? partition_tokens
                          : prefix_partition_for(num_seqs, cache.num_kv_heads, max_context_len);
    const int32_t parts = prefix_tail_slots(max_context_len, p);
    const size_t need = pkv_decode_prefix_workspace_bytes(
        num_seqs, num_q_heads, cache.num_kv_heads, cache.head_dim, max_context_len, p);
    if (!workspace || workspace_bytes < need)
        return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(PKV_ERR_ALIGN, "workspace must be 16-byte aligned");
    // the grid: tail workgroups plus prefix tiles (a tile holds at least 16
    // sequences, group size 8); 256 threads per workgroup.  Over an FP8 cache
    // two tail workgroups per compute unit, as many as can be resident (4 tail
    // waves per compute unit stream the list 13% slower on 256 sequences in 8
    // shared-prefix groups; 4 or 6 workgroups with shorter runs, 5-6% slower).
    // Over a bf16 cache six, so that three rounds of shorter runs pass through
    // each compute unit: equal runs do not take equal times (compute units
    // finished them between 100 and 170 us in a per-wave timeline), and the
    // dispatcher hands the later rounds to the compute units that finish
    // first (2% faster on the same batch).
    const int64_t qblocks = ((int64_t)max_group_size + 15) / 16;
    const int32_t tail_wgs = (cache.fp8 ? 2 : 6) * pkv::compute_units();
    const int64_t wgs = tail_wgs +
                        (int64_t)num_groups * qblocks * pkv::kMaxSegments * cache.num_kv_heads;
    if (wgs >= (int64_t)1 << 24 || (int64_t)num_seqs * num_q_heads >= (int64_t)1 << 26)
        return fail(PKV_ERR_SHAPE, "%d sequences of up to %d tokens in %d groups exceed one launch's grid",
                    num_seqs, max_context_len, num_groups);
    pkv::CascadeArgs a{};
    a.q = q;
    a.k_cache = cache.k;
    a.v_cache = cache.v;
    a.k_scale = cache.k_scale;
    a.v_scale = cache.v_scale;
    a.fp8 = cache.fp8;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.max_context_len = max_context_len;
    a.num_blocks = cache.num_blocks;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = cache.num_kv_heads;
    a.head_dim = cache.head_dim;
    a.group_starts = group_starts;
    a.prefix_lens = prefix_lens;
    a.num_groups = num_groups;
    a.max_group_size = max_group_size;
    a.partition_tokens = p;
    a.max_parts = parts;
    a.tail_workgroups = tail_wgs;
    a.scale = scale;
    a.out = out;
    float *ws = static_cast<float *>(workspace);
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)(parts + pkv::kMaxSegments);
    a.ws_out = ws;
    a.ws_ml = ws + rows * cache.head_dim;
    a.ws_list = reinterpret_cast<int32_t *>(a.ws_ml + rows * 2);
    return hip_status(pkv::launch_cascade(a, stream), what);
}

}  // namespace

extern "C" {

size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_tokens) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_context_len < 0 || partition_tokens < 0 || partition_tokens % kBlock != 0)
        return 0;
    const int32_t p = partition_tokens
                          ? partition_tokens
                          : prefix_partition_for(num_seqs, num_kv_heads, max_context_len);
    const int32_t parts = prefix_tail_slots(max_context_len, p);
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)(parts + pkv::kMaxSegments);
    return rows * (size_t)(head_dim + 2) * sizeof(float) + prefix_list_bytes(num_seqs);
}

int pkv_decode_attn_prefix(const void *q, pkv_cache cache, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, const int32_t *context_lens,
                           int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                           float scale, const int32_t *group_starts, const int32_t *prefix_lens,
                           int32_t num_groups, int32_t max_group_size, void *out, void *workspace,
                           size_t workspace_bytes, int32_t partition_tokens, hipStream_t stream) {
    return prefix_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, group_starts, prefix_lens,
                       num_groups, max_group_size, out, workspace, workspace_bytes,
                       partition_tokens, stream, "pkv_decode_attn_prefix launch");
}

int pkv_decode_attn_prefix_fp8(const void *q, pkv_cache_fp8 cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                               float scale, const int32_t *group_starts,
                               const int32_t *prefix_lens, int32_t num_groups,
                               int32_t max_group_size, void *out, void *workspace,
                               size_t workspace_bytes, int32_t partition_tokens,
                               hipStream_t stream) {
    return prefix_call(q, desc_of(cache), block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, max_context_len, num_q_heads, scale, group_starts, prefix_lens,
                       num_groups, max_group_size, out, workspace, workspace_bytes,
                       partition_tokens, stream, "pkv_decode_attn_prefix_fp8 launch");
}

int pkv_prefix_groups(const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t num_seqs, int32_t min_prefix_tokens,
                      int32_t *group_starts, int32_t *prefix_lens, int32_t *num_groups,
                      int32_t *max_group_size) {
    if (num_seqs < 0 || max_blocks_per_seq < 0 || min_prefix_tokens < 0)
        return fail(PKV_ERR_SHAPE, "num_seqs %d, max_blocks_per_seq %d, min_prefix_tokens %d",
                    num_seqs, max_blocks_per_seq, min_prefix_tokens);
    if (!group_starts || !prefix_lens || !num_groups || !max_group_size ||
        (num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_tables))))
        return fail(PKV_ERR_NULL, "a required pointer is null");
    // whole blocks of a sequence's context that a prefix may cover
    auto full_blocks = [&](int32_t s) {
        const int32_t c = context_lens[s] < 0 ? 0 : context_lens[s];
        return std::min(c / kBlock, max_blocks_per_seq);
    };
    auto row = [&](int32_t s) { return block_tables + (size_t)s * max_blocks_per_seq; };
    const int32_t min_blocks = std::max(1, (min_prefix_tokens + kBlock - 1) / kBlock);
    int32_t g = 0, biggest = 0;
    bool open_plain = false;  // the last group written shares nothing and may grow
    group_starts[0] = 0;
    for (int32_t s = 0; s < num_seqs;) {
        // the run starting at s: its prefix is what s and s + 1 share; each
        // later sequence joins while it shares at least that much with s
        int32_t e = s + 1, common = 0;
        if (e < num_seqs) {
            common = common_blocks(row(s), row(e), std::min(full_blocks(s), full_blocks(e)));
            if (common >= min_blocks) {
                ++e;
                while (e < num_seqs &&
                       common_blocks(row(s), row(e), std::min(common, full_blocks(e))) == common)
                    ++e;
            }
        }
        if (e - s >= 2) {
            prefix_lens[g] = common * kBlock;
            group_starts[++g] = e;
            biggest = std::max(biggest, e - s);
            open_plain = false;
        } else if (open_plain) {
            group_starts[g] = e;  // extend the open group of sequences that share nothing
        } else {
            prefix_lens[g] = 0;
            group_starts[++g] = e;
            open_plain = true;
        }
        s = e;
    }
    *num_groups = g;
    *max_group_size = biggest;
    return ok();
}

int pkv_debug_bounds_enabled(void) {
#ifdef PKV_DEBUG_BOUNDS
    return 1;
#else
    return 0;
#endif
}

int pkv_debug_status(uint32_t out[4], int clear) {
    if (!out) return fail(PKV_ERR_NULL, "out is null");
    out[0] = out[1] = out[2] = out[3] = 0u;
    if (!pkv_debug_bounds_enabled())
        return fail(PKV_ERR_UNSUPPORTED, "this library was built without PKV_DEBUG_BOUNDS");
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_debug_status: %s", hipGetErrorString(e));
    hipError_t (*const words[])(uint32_t *, bool) = {
        pkv::debug_word_store,   pkv::debug_word_decode,  pkv::debug_word_prefill,
        pkv::debug_word_mixed,   pkv::debug_word_cascade, pkv::debug_word_copy};
    for (auto word : words) {
        uint32_t w[4];
        e = word(w, clear != 0);
        if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_debug_status: %s", hipGetErrorString(e));
        if (out[0] == 0u && w[0] != 0u) {
            out[0] = w[0];
            out[1] = w[1];
            out[2] = w[2];
        }
        out[3] += w[3];
    }
    return ok();
}

int pkv_check_tables(const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs, int32_t max_context_len,
                     const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                     int32_t *bad_seq, int32_t *bad_index) {
    auto report = [&](int32_t s, int32_t i) {
        if (bad_seq) *bad_seq = s;
        if (bad_index) *bad_index = i;
    };
    report(-1, -1);
    if (num_seqs < 0 || max_blocks_per_seq < 0 || num_tokens < 0 || num_blocks < 0)
        return fail(PKV_ERR_SHAPE, "num_seqs %d, max_blocks_per_seq %d, num_tokens %d, num_blocks %d",
                    num_seqs, max_blocks_per_seq, num_tokens, num_blocks);
    if ((num_seqs > 0 && (!context_lens || (max_blocks_per_seq > 0 && !block_tables))) ||
        (num_tokens > 0 && !slot_mapping))
        return fail(PKV_ERR_NULL, "context_lens, block_tables or slot_mapping is null");
    const int64_t table_tokens = (int64_t)max_blocks_per_seq * kBlock;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t ctx = context_lens[s];
        if (ctx < 0 || ctx > table_tokens || (max_context_len >= 0 && ctx > max_context_len)) {
            report(s, -1);
            return fail(PKV_ERR_INDEX,
                        "context_lens[%d] = %d is outside [0, %lld] (table of %d blocks, "
                        "max_context_len %d)",
                        s, ctx, (long long)table_tokens, max_blocks_per_seq, max_context_len);
        }
        const int32_t *row = block_tables + (size_t)s * max_blocks_per_seq;
        const int32_t nb = (ctx + kBlock - 1) / kBlock;
        for (int32_t i = 0; i < nb; ++i) {
            if (row[i] < 0 || row[i] >= num_blocks) {
                report(s, i);
                return fail(PKV_ERR_INDEX,
                            "block_tables[%d][%d] = %d is outside the pool of %d blocks "
                            "(context %d)",
                            s, i, row[i], num_blocks, ctx);
            }
        }
    }
    const int64_t pool_slots = (int64_t)num_blocks * kBlock;
    std::vector<std::pair<int32_t, int32_t>> live;  // (slot, token)
    live.reserve((size_t)num_tokens);
    for (int32_t i = 0; i < num_tokens; ++i) {
        const int32_t slot = slot_mapping[i];
        if (slot < 0) continue;  // a skipped token
        if (slot >= pool_slots) {
            report(-1, i);
            return fail(PKV_ERR_INDEX, "slot_mapping[%d] = %d is outside the pool of %lld slots", i,
                        slot, (long long)pool_slots);
        }
        live.emplace_back(slot, i);
    }
    std::sort(live.begin(), live.end());
    for (size_t k = 1; k < live.size(); ++k) {
        if (live[k].first == live[k - 1].first) {
            const int32_t i = std::max(live[k].second, live[k - 1].second);
            report(-1, i);
            return fail(PKV_ERR_INDEX, "slot %d is written by tokens %d and %d", live[k].first,
                        std::min(live[k].second, live[k - 1].second), i);
        }
    }
    return ok();
}

}  // extern "C"
