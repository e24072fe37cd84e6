// host_driver.cpp -- exercises the host code of libpkv (argument checks and
// sizing of every entry point, the table helpers, the block pool) for a build
// under the address and undefined-behaviour sanitizers, with the kernel
// launchers replaced by stubs (launch_stubs.cpp).  No GPU is touched: device
// pointers are aligned stand-in addresses that nothing dereferences.
// Test infrastructure only.  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <set>
#include <vector>

#include "pkv.h"
#include "pkv_pool.h"

namespace pkv {
extern int g_launches;
}

static int g_failures = 0;

#define CHECK(cond)                                                             \
    do {                                                                        \
        if (!(cond)) {                                                          \
            ++g_failures;                                                       \
            fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, \
                    __LINE__, #cond, pkv_last_error());                         \
        }                                                                       \
    } while (0)

// A status that must be an argument error, with a message.
#define REJECT(call)                                                           \
    do {                                                                       \
        const int launches_ = pkv::g_launches;                                 \
        const int st_ = (call);                                                \
        CHECK(st_ != PKV_OK);                                                  \
        CHECK(pkv_last_error()[0] != '\0');                                    \
        CHECK(pkv::g_launches == launches_); /* rejected before any launch */ \
    } while (0)
#define ACCEPT(call) CHECK((call) == PKV_OK)

static void *dev(uintptr_t a) { return reinterpret_cast<void *>(a); }

static void entry_points() {
    void *D = dev(0x100000), *MIS = dev(0x100008);
    float *DF = static_cast<float *>(dev(0x200000));
    const int32_t *DI = static_cast<const int32_t *>(dev(0x300000));
    hipStream_t st = nullptr;
    pkv_cache c{D, D, 64, 2, 128, 16};

    // ---- store
    ACCEPT(pkv_store(D, D, DI, 4, c, st));
    ACCEPT(pkv_store(nullptr, nullptr, nullptr, 0, c, st));  // empty: no-op
    REJECT(pkv_store(D, D, DI, -1, c, st));
    REJECT(pkv_store(nullptr, D, DI, 4, c, st));
    REJECT(pkv_store(MIS, D, DI, 4, c, st));
    pkv_cache bad = c;
    bad.head_dim = 96;
    REJECT(pkv_store(D, D, DI, 4, bad, st));
    bad = c;
    bad.block_size = 32;
    REJECT(pkv_store(D, D, DI, 4, bad, st));
    bad = c;
    bad.k = MIS;
    REJECT(pkv_store(D, D, DI, 4, bad, st));

    // ---- decode, its work split and workspace
    for (int32_t ctx : {1, 16, 100, 4096, 32768})
        for (int32_t s : {1, 3, 32, 256}) {
            const int32_t p = pkv_decode_partition_tokens(s, 2, ctx);
            CHECK(p != 0);
            const size_t need = pkv_decode_workspace_bytes(s, 4, 128, ctx, p);
            CHECK(p < 0 ? need == 0 : true);
            const int32_t mb = (ctx + 15) / 16;
            const int launches = pkv::g_launches;
            ACCEPT(pkv_decode_attn(D, c, DI, mb, DI, s, ctx, 4, 0.1f, D, D, need, p, st));
            CHECK(pkv::g_launches == launches + 1);
            if (need > 0) REJECT(pkv_decode_attn(D, c, DI, mb, DI, s, ctx, 4, 0.1f, D, D, need - 1, p, st));
            const int st2 = pkv_decode_attn_noalloc(D, c, DI, mb, DI, s, ctx, 4, 0.1f, D, p, st);
            CHECK(need <= pkv_decode_noalloc_max_bytes() ? st2 == PKV_OK : st2 == PKV_ERR_WORKSPACE);
        }
    REJECT(pkv_decode_attn(D, c, DI, 2, DI, 3, 33, 4, 0.1f, D, D, 1 << 20, 0, st));  // ctx past table
    REJECT(pkv_decode_attn(D, c, DI, 8, DI, 3, 100, 3, 0.1f, D, D, 1 << 20, 0, st));  // 3 % 2 heads
    REJECT(pkv_decode_attn(D, c, DI, 8, DI, 3, 100, 32, 0.1f, D, D, 1 << 20, 0, st)); // group 16
    REJECT(pkv_decode_attn(D, c, DI, 8, DI, 3, 100, 4, 0.1f, D, D, 1 << 20, 20, st)); // P not /16
    REJECT(pkv_decode_attn(D, c, DI, 8, DI, 3, 100, 4, 0.1f, D, D, 1 << 20, -9, st));
    REJECT(pkv_decode_attn(nullptr, c, DI, 8, DI, 3, 100, 4, 0.1f, D, D, 1 << 20, 0, st));
    REJECT(pkv_decode_attn(D, c, DI, 8, DI, 3, 100, 4, 0.1f, MIS, D, 1 << 20, 0, st));
    REJECT(pkv_decode_attn(D, c, DI, 8, DI, -1, 100, 4, 0.1f, D, D, 1 << 20, 0, st));
    ACCEPT(pkv_decode_attn(D, c, DI, 8, DI, 0, 100, 4, 0.1f, D, D, 0, 0, st));  // empty batch
    REJECT(pkv_decode_attn_noalloc(D, c, DI, 2048, DI, 256, 32768, 4, 0.1f, D, 16, st));

    // ---- fused store + decode, with the rotary table
    ACCEPT(pkv_store_decode_attn(D, D, DI, D, c, DI, 8, DI, 3, 100, 4, 0.1f, D, D, 1 << 20, 0, st));
    REJECT(pkv_store_decode_attn(nullptr, D, DI, D, c, DI, 8, DI, 3, 100, 4, 0.1f, D, D, 1 << 20, 0, st));
    ACCEPT(pkv_store_decode_attn_rope(D, D, DI, D, DF, 100, c, DI, 8, DI, 3, 100, 4, 0.1f, D, D,
                                      1 << 20, 0, st));
    REJECT(pkv_store_decode_attn_rope(D, D, DI, D, DF, 99, c, DI, 8, DI, 3, 100, 4, 0.1f, D, D,
                                      1 << 20, 0, st));
    REJECT(pkv_store_decode_attn_rope(D, D, DI, D, nullptr, 100, c, DI, 8, DI, 3, 100, 4, 0.1f, D,
                                      D, 1 << 20, 0, st));

    // ---- FP8 cache
    pkv_cache_fp8 c8{D, D, DF, DF, 64, 2, 128, 16};
    ACCEPT(pkv_store_fp8(D, D, DI, 4, c8, st));
    pkv_cache_fp8 b8 = c8;
    b8.k_scale = nullptr;
    REJECT(pkv_store_fp8(D, D, DI, 4, b8, st));
    const int32_t p8 = pkv_decode_partition_tokens_fp8(3, 2, 100);
    const size_t need8 = pkv_decode_workspace_bytes(3, 4, 128, 100, p8);
    ACCEPT(pkv_decode_attn_fp8(D, c8, DI, 8, DI, 3, 100, 4, 0.1f, D, D, need8 + 16, p8, st));
    ACCEPT(pkv_store_decode_attn_fp8(D, D, DI, D, c8, DI, 8, DI, 3, 100, 4, 0.1f, D, D,
                                     need8 + 16, p8, st));
    REJECT(pkv_decode_attn_fp8(D, b8, DI, 8, DI, 3, 100, 4, 0.1f, D, D, need8 + 16, p8, st));

    // ---- prefill and the mixed step
    ACCEPT(pkv_prefill_attn(D, c, DI, 8, DI, DI, 3, 64, 100, 4, 0.1f, D, st));
    REJECT(pkv_prefill_attn(D, c, DI, 8, nullptr, DI, 3, 64, 100, 4, 0.1f, D, st));
    REJECT(pkv_prefill_attn(D, c, DI, 8, DI, DI, 3, -1, 100, 4, 0.1f, D, st));
    for (int32_t nd : {0, 2, 5}) {
        const size_t mw = pkv_mixed_workspace_bytes(5, nd, 64, 4096, 4, 2, 128);
        ACCEPT(pkv_mixed_attn(D, c, DI, 256, DI, DI, nd, 5, 64, 4096, 4, 0.1f, D,
                              mw ? D : nullptr, mw, st));
    }
    REJECT(pkv_mixed_attn(D, c, DI, 256, DI, DI, 6, 5, 64, 4096, 4, 0.1f, D, nullptr, 0, st));

    // ---- shared-prefix decode
    const size_t pw = pkv_decode_prefix_workspace_bytes(64, 4, 2, 128, 4096, 0);
    CHECK(pw > 0);
    ACCEPT(pkv_decode_attn_prefix(D, c, DI, 256, DI, 64, 4096, 4, 0.1f, DI, DI, 2, 32, D, D, pw, 0,
                                  st));
    REJECT(pkv_decode_attn_prefix(D, c, DI, 256, DI, 64, 4096, 4, 0.1f, DI, DI, 2, 32, D, D, pw - 16,
                                  0, st));
    REJECT(pkv_decode_attn_prefix(D, c, DI, 256, DI, 64, 4096, 4, 0.1f, nullptr, DI, 2, 32, D, D,
                                  pw, 0, st));

    // ---- block copy and the read probe
    void *pools[3] = {D, D, D};
    ACCEPT(pkv_copy_blocks(pools, 3, 4096, 64, DI, 5, st));
    REJECT(pkv_copy_blocks(pools, 3, 4100, 64, DI, 5, st));
    REJECT(pkv_copy_blocks(nullptr, 3, 4096, 64, DI, 5, st));
    ACCEPT(pkv_read_probe(D, 1 << 20, static_cast<uint32_t *>(D), st));
    REJECT(pkv_read_probe(D, (1 << 20) + 4, static_cast<uint32_t *>(D), st));

    // ---- sizing and status strings
    CHECK(pkv_kv_bytes(32, 8, 128, 4096, 2) == 536870912ull);
    for (int s = 0; s <= 10; ++s) CHECK(pkv_status_string(s) != nullptr);
}

// Random tables through pkv_prefix_groups and pkv_check_tables.
static void table_helpers(std::mt19937 &rng) {
    for (int round = 0; round < 300; ++round) {
        const int32_t s = 1 + rng() % 40, width = 1 + rng() % 12, nb = 1 + rng() % 64;
        std::vector<int32_t> bt((size_t)s * width), ctx(s);
        const int32_t shared = rng() % (width + 1);
        for (int32_t i = 0; i < s; ++i) {
            ctx[i] = (int32_t)(rng() % (width * 16 + 1));
            for (int32_t j = 0; j < width; ++j)
                bt[(size_t)i * width + j] = (j < shared && (i % 3)) ? j : (int32_t)(rng() % nb);
        }
        if (rng() % 4 == 0) bt[rng() % bt.size()] = (rng() % 2) ? -1 : nb + 3;
        std::vector<int32_t> starts(s + 1), plens(s);
        int32_t ng = -1, mg = -1;
        ACCEPT(pkv_prefix_groups(bt.data(), width, ctx.data(), s, 16 * (1 + rng() % 3),
                                 starts.data(), plens.data(), &ng, &mg));
        CHECK(ng >= 0 && ng <= s && starts[0] == 0 && starts[ng] == s);
        for (int32_t g = 0; g < ng; ++g) CHECK(starts[g] < starts[g + 1] && plens[g] % 16 == 0);
        std::vector<int32_t> slots(rng() % 20);
        for (auto &x : slots) x = (int32_t)(rng() % (nb * 16 + 8)) - 4;
        int32_t bs = 0, bi = 0;
        const int st = pkv_check_tables(bt.data(), width, ctx.data(), s, -1, slots.data(),
                                        (int32_t)slots.size(), nb, &bs, &bi);
        CHECK(st == PKV_OK || st == PKV_ERR_INDEX);
        CHECK(st != PKV_OK || (bs == -1 && bi == -1));
    }
    REJECT(pkv_prefix_groups(nullptr, 2, nullptr, 3, 16, nullptr, nullptr, nullptr, nullptr));
}

// Random admissions, appends, forks and frees on pools with and without the
// prefix cache, with the pool's invariants checked after every operation.
static void pool_streams(std::mt19937 &rng) {
    for (int caching = 0; caching < 2; ++caching) {
        const int32_t nb = 96;
        pkv_pool *pool = nullptr;
        ACCEPT(pkv_pool_create(nb, 16, caching, &pool));
        std::vector<int64_t> live;
        int64_t next = 1;
        for (int op = 0; op < 6000; ++op) {
            const int kind = rng() % 10;
            if (kind < 3 || live.empty()) {
                const int32_t n = 1 + rng() % 70;
                std::vector<int32_t> tok(n), slots(n);
                const int32_t prompt = rng() % 3;  // a few shared prompts give cache hits
                for (int32_t i = 0; i < n; ++i) tok[i] = i < 40 ? prompt * 1000 + i : (int32_t)rng();
                int32_t cached = -1;
                const int st = pkv_pool_add_seq(pool, next, tok.data(), n, slots.data(), &cached);
                CHECK(st == PKV_OK || st == PKV_ERR_CAPACITY);
                if (st == PKV_OK) {
                    CHECK(cached >= 0 && cached % 16 == 0 && cached < n);
                    for (int32_t i = 0; i < n; ++i)
                        CHECK(i < cached ? slots[i] == -1 : (slots[i] >= 0 && slots[i] < nb * 16));
                    live.push_back(next);
                }
                ++next;
            } else if (kind < 7) {
                const int32_t n = 1 + rng() % std::min<size_t>(8, live.size());
                std::vector<int64_t> ids;
                std::set<int64_t> used;
                while ((int32_t)ids.size() < n) {
                    const int64_t id = live[rng() % live.size()];
                    if (used.insert(id).second) ids.push_back(id);
                }
                std::vector<int32_t> tok(n), slots(n), copies(2 * n);
                for (auto &t : tok) t = (int32_t)rng();
                int32_t nc = -1, done = -1;
                const int st = pkv_pool_append(pool, ids.data(), tok.data(), n, slots.data(),
                                               copies.data(), &nc, &done);
                CHECK(st == PKV_OK || st == PKV_ERR_CAPACITY);
                CHECK(done >= 0 && done <= n && nc >= 0 && nc <= done);
                for (int32_t i = 0; i < done; ++i) CHECK(slots[i] >= 0 && slots[i] < nb * 16);
            } else if (kind < 8) {
                const int64_t parent = live[rng() % live.size()];
                const int st = pkv_pool_fork(pool, parent, next);
                CHECK(st == PKV_OK || st == PKV_ERR_CAPACITY);
                if (st == PKV_OK) live.push_back(next);
                ++next;
            } else {
                const size_t i = rng() % live.size();
                ACCEPT(pkv_pool_free_seq(pool, live[i]));
                live.erase(live.begin() + (long)i);
            }
            // invariants: the free count is the number of unreferenced blocks,
            // and every live table is valid for the kernels
            int32_t unreferenced = 0;
            for (int32_t b = 0; b < nb; ++b) unreferenced += pkv_pool_refcount(pool, b) == 0;
            CHECK(pkv_pool_num_free(pool) == unreferenced);
            CHECK(pkv_pool_refcount(pool, nb) == -1);
            if (!live.empty() && op % 50 == 0) {
                const int32_t width = 64;
                std::vector<int32_t> bt(live.size() * width), ctx(live.size());
                const int st = pkv_pool_block_tables(pool, live.data(), (int32_t)live.size(), width,
                                                     bt.data(), ctx.data());
                CHECK(st == PKV_OK || st == PKV_ERR_SHAPE);
                if (st == PKV_OK)
                    ACCEPT(pkv_check_tables(bt.data(), width, ctx.data(), (int32_t)live.size(), -1,
                                            nullptr, 0, nb, nullptr, nullptr));
            }
        }
        REJECT(pkv_pool_free_seq(pool, -12345));
        REJECT(pkv_pool_fork(pool, -1, next));
        pkv_pool_destroy(pool);
    }
    REJECT(pkv_pool_create(-1, 16, 1, nullptr));
}

int main() {
    std::mt19937 rng(20261203u);
    entry_points();
    table_helpers(rng);
    pool_streams(rng);
    printf("host driver: %d check(s) failed, %d stub launch(es)\n", g_failures, pkv::g_launches);
    return g_failures ? 1 : 0;
}
