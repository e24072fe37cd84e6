// pool.cpp -- the physical block pool (declared in include/pkv_pool.h).
//
// Host-only bookkeeping that turns requests into the block tables and slot
// mappings the kernels read: a global pool of uniform blocks handed out on
// demand and returned when a request ends ("Nano-vLLM engine deep-dive",
// section 2.2), logical-to-physical block tables ("LLM basics primer" part 4,
// section 17.7), and shared prefixes held once, with copy-on-write and prefix
// caching (deep-dive section 2.2; primer part 4, sections 17.6 and 17.7).
//
// Data structures, all O(1) per token except the prefix lookup (one hash of a
// block's tokens per full block):
//   ref[b]            live sequences whose table holds b
//   free list         intrusive doubly linked FIFO over block ids, so a block
//                     revived by a prefix hit leaves it in O(1)
//   handed[b]         times b has been taken from the free list; with the
//                     previous block's id it makes a cached block's identity
//                     exact, whatever order blocks are evicted in
//   prefix cache      hash of (previous block, its hand-out count, tokens) ->
//                     block ids; candidates are confirmed by comparing the
//                     stored identity, so a hash collision never gives a hit
#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"
#include "pkv_pool.h"

using pkv::fail;
using pkv::ok;

struct pkv_pool {
    struct Seq {
        std::vector<int32_t> blocks;
        std::vector<int32_t> tokens;
    };

    int32_t num_blocks = 0;
    int32_t block_size = 0;
    bool prefix_caching = false;

    std::vector<int32_t> ref, handed;
    // free list (FIFO): head is handed out next, freed blocks join at the tail
    std::vector<int32_t> next_free, prev_free;
    std::vector<uint8_t> is_free;
    int32_t head = -1, tail = -1, nfree = 0;

    // identity each block is cached under (has_key[b] == 0: none)
    std::vector<uint8_t> has_key;
    std::vector<int32_t> key_prev, key_prev_handed, key_tokens;  // key_tokens [b][block_size]
    std::unordered_multimap<uint64_t, int32_t> cache;

    std::unordered_map<int64_t, Seq> seqs;

    // -- free list ---------------------------------------------------------------
    void push_free(int32_t b) {
        prev_free[b] = tail;
        next_free[b] = -1;
        if (tail >= 0) next_free[tail] = b; else head = b;
        tail = b;
        is_free[b] = 1;
        ++nfree;
    }
    void unlink_free(int32_t b) {
        if (prev_free[b] >= 0) next_free[prev_free[b]] = next_free[b]; else head = next_free[b];
        if (next_free[b] >= 0) prev_free[next_free[b]] = prev_free[b]; else tail = prev_free[b];
        is_free[b] = 0;
        --nfree;
    }
    // Hand out the oldest free block for new content (caller checked nfree > 0).
    int32_t take_free() {
        const int32_t b = head;
        unlink_free(b);
        if (has_key[b]) uncache(b);
        ++handed[b];
        ref[b] = 1;
        return b;
    }

    // -- prefix cache --------------------------------------------------------------
    static uint64_t mix(uint64_t h, uint64_t x) {
        h ^= x + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
        h *= 0xff51afd7ed558ccdull;
        return h ^ (h >> 33);
    }
    uint64_t key_hash(int32_t prev, int32_t prev_handed, const int32_t *toks) const {
        uint64_t h = mix(0x243f6a8885a308d3ull, (uint32_t)prev);
        h = mix(h, (uint32_t)prev_handed);
        for (int32_t i = 0; i < block_size; ++i) h = mix(h, (uint32_t)toks[i]);
        return h;
    }
    // The identity of a full block whose tokens are toks and which follows
    // block prev (-1 for the first block of a sequence).
    void identity(int32_t prev, int32_t *out_prev, int32_t *out_handed) const {
        *out_prev = prev;
        *out_handed = prev >= 0 ? handed[prev] : 0;
    }
    int32_t lookup(int32_t prev, const int32_t *toks) const {
        int32_t kp, kh;
        identity(prev, &kp, &kh);
        auto range = cache.equal_range(key_hash(kp, kh, toks));
        for (auto it = range.first; it != range.second; ++it) {
            const int32_t b = it->second;
            if (key_prev[b] == kp && key_prev_handed[b] == kh &&
                memcmp(&key_tokens[(size_t)b * block_size], toks,
                       sizeof(int32_t) * block_size) == 0)
                return b;
        }
        return -1;
    }
    void uncache(int32_t b) {
        auto range = cache.equal_range(
            key_hash(key_prev[b], key_prev_handed[b], &key_tokens[(size_t)b * block_size]));
        for (auto it = range.first; it != range.second; ++it) {
            if (it->second == b) {
                cache.erase(it);
                break;
            }
        }
        has_key[b] = 0;
    }
    // Block `index` of s has just become full: cache it unless an equal block
    // is cached already.
    void register_full(const Seq &s, size_t index) {
        if (!prefix_caching) return;
        const int32_t b = s.blocks[index];
        const int32_t prev = index > 0 ? s.blocks[index - 1] : -1;
        const int32_t *toks = &s.tokens[index * block_size];
        if (has_key[b] || lookup(prev, toks) >= 0) return;
        identity(prev, &key_prev[b], &key_prev_handed[b]);
        memcpy(&key_tokens[(size_t)b * block_size], toks, sizeof(int32_t) * block_size);
        has_key[b] = 1;
        cache.emplace(key_hash(key_prev[b], key_prev_handed[b], toks), b);
    }

    int32_t slot_of(const Seq &s, int64_t t) const {
        return s.blocks[t / block_size] * block_size + (int32_t)(t % block_size);
    }
};

extern "C" {

int pkv_pool_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                    pkv_pool **out) {
    if (!out) return fail(PKV_ERR_NULL, "out is null");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0 ||
        (int64_t)num_blocks * block_size > INT32_MAX)
        return fail(PKV_ERR_SHAPE, "num_blocks %d x block_size %d: both positive, slots below 2^31",
                    num_blocks, block_size);
    pkv_pool *p = new (std::nothrow) pkv_pool;
    if (!p) return fail(PKV_ERR_SHAPE, "out of host memory");
    try {
        p->num_blocks = num_blocks;
        p->block_size = block_size;
        p->prefix_caching = prefix_caching != 0;
        p->ref.assign(num_blocks, 0);
        p->handed.assign(num_blocks, 0);
        p->next_free.assign(num_blocks, -1);
        p->prev_free.assign(num_blocks, -1);
        p->is_free.assign(num_blocks, 0);
        p->has_key.assign(num_blocks, 0);
        p->key_prev.assign(num_blocks, -1);
        p->key_prev_handed.assign(num_blocks, 0);
        if (p->prefix_caching) p->key_tokens.assign((size_t)num_blocks * block_size, 0);
    } catch (const std::bad_alloc &) {
        delete p;
        return fail(PKV_ERR_SHAPE, "out of host memory for %d blocks", num_blocks);
    }
    for (int32_t b = 0; b < num_blocks; ++b) p->push_free(b);
    *out = p;
    return ok();
}

void pkv_pool_destroy(pkv_pool *pool) { delete pool; }

int pkv_pool_add_seq(pkv_pool *pool, int64_t seq_id, const int32_t *tokens, int32_t num_tokens,
                     int32_t *slots_out, int32_t *num_cached_out) {
    if (!pool || !tokens || !slots_out || !num_cached_out)
        return fail(PKV_ERR_NULL, "pool, tokens, slots_out or num_cached_out is null");
    if (num_tokens <= 0) return fail(PKV_ERR_SHAPE, "num_tokens %d: a prompt has a token", num_tokens);
    if (pool->seqs.count(seq_id))
        return fail(PKV_ERR_SEQUENCE, "sequence %lld is live", (long long)seq_id);
    const int32_t bs = pool->block_size;
    // look the leading full blocks up first, changing nothing
    std::vector<int32_t> hits;
    int32_t revived = 0;
    if (pool->prefix_caching) {
        int32_t prev = -1;
        for (int32_t i = 0; i < (num_tokens - 1) / bs; ++i) {
            const int32_t b = pool->lookup(prev, tokens + (size_t)i * bs);
            if (b < 0) break;
            hits.push_back(b);
            revived += pool->ref[b] == 0;
            prev = b;
        }
    }
    const int32_t nblocks = (num_tokens + bs - 1) / bs;
    const int32_t need = nblocks - (int32_t)hits.size();
    if (need > pool->nfree - revived)
        return fail(PKV_ERR_CAPACITY, "sequence %lld needs %d blocks, %d free",
                    (long long)seq_id, need, pool->nfree - revived);

    pkv_pool::Seq s;
    s.blocks.reserve(nblocks);
    s.tokens.assign(tokens, tokens + num_tokens);
    for (int32_t b : hits) {
        if (pool->ref[b] == 0) pool->unlink_free(b);
        ++pool->ref[b];
        s.blocks.push_back(b);
    }
    for (int32_t i = 0; i < need; ++i) s.blocks.push_back(pool->take_free());
    for (int32_t i = (int32_t)hits.size(); i < num_tokens / bs; ++i) pool->register_full(s, i);
    const int32_t cached = (int32_t)hits.size() * bs;
    for (int32_t t = 0; t < num_tokens; ++t) slots_out[t] = t < cached ? -1 : pool->slot_of(s, t);
    *num_cached_out = cached;
    pool->seqs.emplace(seq_id, std::move(s));
    return ok();
}

int pkv_pool_append(pkv_pool *pool, const int64_t *seq_ids, const int32_t *tokens, int32_t n,
                    int32_t *slots_out, int32_t *copies_out, int32_t *num_copies_out,
                    int32_t *num_done_out) {
    if (num_done_out) *num_done_out = 0;
    if (num_copies_out) *num_copies_out = 0;
    if (!pool || !num_done_out || !num_copies_out)
        return fail(PKV_ERR_NULL, "pool, num_copies_out or num_done_out is null");
    if (n < 0) return fail(PKV_ERR_SHAPE, "n %d", n);
    if (n > 0 && (!seq_ids || !tokens || !slots_out || !copies_out))
        return fail(PKV_ERR_NULL, "seq_ids, tokens, slots_out or copies_out is null");
    const int32_t bs = pool->block_size;
    int32_t ncopies = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it == pool->seqs.end())
            return fail(PKV_ERR_SEQUENCE, "unknown sequence %lld", (long long)seq_ids[i]);
        pkv_pool::Seq &s = it->second;
        const size_t p = s.tokens.size();
        if (p % bs == 0) {
            if (pool->nfree == 0)
                return fail(PKV_ERR_CAPACITY, "no free block for sequence %lld",
                            (long long)seq_ids[i]);
            s.blocks.push_back(pool->take_free());
        } else if (pool->ref[s.blocks.back()] > 1) {
            if (pool->nfree == 0)
                return fail(PKV_ERR_CAPACITY, "no free block to copy sequence %lld's last block",
                            (long long)seq_ids[i]);
            const int32_t old = s.blocks.back();
            const int32_t fresh = pool->take_free();
            --pool->ref[old];
            s.blocks.back() = fresh;
            copies_out[2 * ncopies] = old;
            copies_out[2 * ncopies + 1] = fresh;
            *num_copies_out = ++ncopies;
        }
        s.tokens.push_back(tokens[i]);
        if ((p + 1) % bs == 0) pool->register_full(s, p / bs);
        slots_out[i] = pool->slot_of(s, (int64_t)p);
        *num_done_out = i + 1;
    }
    return ok();
}

int pkv_pool_fork(pkv_pool *pool, int64_t parent_id, int64_t child_id) {
    if (!pool) return fail(PKV_ERR_NULL, "pool is null");
    auto it = pool->seqs.find(parent_id);
    if (it == pool->seqs.end())
        return fail(PKV_ERR_SEQUENCE, "unknown sequence %lld", (long long)parent_id);
    if (pool->seqs.count(child_id))
        return fail(PKV_ERR_SEQUENCE, "sequence %lld is live", (long long)child_id);
    pkv_pool::Seq child = it->second;
    for (int32_t b : child.blocks) ++pool->ref[b];
    pool->seqs.emplace(child_id, std::move(child));
    return ok();
}

int pkv_pool_free_seq(pkv_pool *pool, int64_t seq_id) {
    if (!pool) return fail(PKV_ERR_NULL, "pool is null");
    auto it = pool->seqs.find(seq_id);
    if (it == pool->seqs.end())
        return fail(PKV_ERR_SEQUENCE, "unknown sequence %lld", (long long)seq_id);
    const std::vector<int32_t> &blocks = it->second.blocks;
    for (size_t i = blocks.size(); i-- > 0;) {
        const int32_t b = blocks[i];
        if (--pool->ref[b] == 0) pool->push_free(b);
    }
    pool->seqs.erase(it);
    return ok();
}

int pkv_pool_block_tables(const pkv_pool *pool, const int64_t *seq_ids, int32_t n,
                          int32_t max_blocks_per_seq, int32_t *block_tables_out,
                          int32_t *context_lens_out) {
    if (!pool) return fail(PKV_ERR_NULL, "pool is null");
    if (n < 0 || max_blocks_per_seq <= 0)
        return fail(PKV_ERR_SHAPE, "n %d, max_blocks_per_seq %d", n, max_blocks_per_seq);
    if (n > 0 && (!seq_ids || !block_tables_out || !context_lens_out))
        return fail(PKV_ERR_NULL, "seq_ids, block_tables_out or context_lens_out is null");
    for (int32_t i = 0; i < n; ++i) {
        auto it = pool->seqs.find(seq_ids[i]);
        if (it == pool->seqs.end())
            return fail(PKV_ERR_SEQUENCE, "unknown sequence %lld", (long long)seq_ids[i]);
        const pkv_pool::Seq &s = it->second;
        if ((int64_t)s.blocks.size() > max_blocks_per_seq)
            return fail(PKV_ERR_SHAPE, "sequence %lld holds %zu blocks, rows have %d",
                        (long long)seq_ids[i], s.blocks.size(), max_blocks_per_seq);
        int32_t *row = block_tables_out + (size_t)i * max_blocks_per_seq;
        size_t j = 0;
        for (; j < s.blocks.size(); ++j) row[j] = s.blocks[j];
        for (; j < (size_t)max_blocks_per_seq; ++j) row[j] = -1;
        context_lens_out[i] = (int32_t)s.tokens.size();
    }
    return ok();
}

int32_t pkv_pool_num_free(const pkv_pool *pool) { return pool ? pool->nfree : 0; }

int32_t pkv_pool_refcount(const pkv_pool *pool, int32_t block) {
    if (!pool || block < 0 || block >= pool->num_blocks) return -1;
    return pool->ref[block];
}

int32_t pkv_pool_seq_len(const pkv_pool *pool, int64_t seq_id) {
    if (!pool) return -1;
    auto it = pool->seqs.find(seq_id);
    return it == pool->seqs.end() ? -1 : (int32_t)it->second.tokens.size();
}

}  // extern "C"
