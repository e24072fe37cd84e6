"""Pins of the block-pool reference model (oracle/block_pool.py).

Each pin checks the model against something it does not compute itself:
- brute-force content tracking: every cache slot is stamped with the token
  history whose K/V a store would put there (the sequence's tokens up to and
  including that position), copies move stamps, and after every operation
  every live sequence must read exactly its own history at every position;
- reference counts recounted from the live block tables, the free list
  recounted from the counts;
- the sizes the pages print (32 requests sharing a 2048-token system prompt,
  "LLM basics primer" part 4, section 17.6) and hand-derived block counts.

Every pin takes the module under test, so the same pins run against planted
mistakes (tests/test_pool_oracle.py).
"""
from __future__ import annotations

import copy
import random


class Tracker:
    """Wraps a pool and keeps the brute-force stamp of every slot.  A stamp is
    the interned id of a token history (equal histories, equal ids), so a
    slot's stamp says whose K/V it holds."""

    def __init__(self, bp, num_blocks, block_size=16, prefix_caching=False):
        self.bp = bp
        self.pool = bp.BlockPool(num_blocks, block_size, prefix_caching)
        self.bs = block_size
        self.stamp = {}       # (block, offset) -> history id of what is stored there
        self.ids = {}         # seq id -> [history id of tokens[:t + 1] for each t]
        self.intern = {}      # (history id, token) -> history id; the empty history is 0

    def _extend(self, hid, token):
        key = (hid, token)
        if key not in self.intern:
            self.intern[key] = len(self.intern) + 1
        return self.intern[key]

    def snapshot(self):
        state = self.pool.state() if hasattr(self.pool, "state") else self.pool.__dict__
        return copy.deepcopy((state, self.stamp, self.ids))

    def add(self, sid, tokens):
        slots, cached = self.pool.add_seq(sid, tokens)
        assert len(slots) == len(tokens)
        assert cached % self.bs == 0 and 0 <= cached <= len(tokens) - 1
        ids, h = [], 0
        for t, s in enumerate(slots):
            h = self._extend(h, tokens[t])
            ids.append(h)
            assert (s == -1) == (t < cached), (t, s, cached)
            if s >= 0:
                self.stamp[(s // self.bs, s % self.bs)] = h
        self.ids[sid] = ids
        return slots, cached

    def append(self, sid, token):
        slot, cp = self.pool.append(sid, token)
        if cp is not None:
            src, dst = cp
            assert src != dst
            for o in range(self.bs):
                if (src, o) in self.stamp:
                    self.stamp[(dst, o)] = self.stamp[(src, o)]
                else:
                    self.stamp.pop((dst, o), None)
        ids = self.ids[sid]
        ids.append(self._extend(ids[-1] if ids else 0, token))
        self.stamp[(slot // self.bs, slot % self.bs)] = ids[-1]
        return slot, cp

    def fork(self, parent, child):
        self.pool.fork(parent, child)
        self.ids[child] = list(self.ids[parent])

    def free(self, sid):
        self.pool.free_seq(sid)
        del self.ids[sid]

    def check(self):
        pool, bs = self.pool, self.bs
        refs = [0] * pool.num_blocks
        for sid, ids in self.ids.items():
            table = pool.block_table(sid)
            assert pool.seq_len(sid) == len(ids)
            assert len(table) == -(-len(ids) // bs), (sid, len(table), len(ids))
            assert len(set(table)) == len(table), "a block twice in one table"
            for b in table:
                assert 0 <= b < pool.num_blocks
                refs[b] += 1
            for t, h in enumerate(ids):
                got = self.stamp.get((table[t // bs], t % bs))
                assert got == h, f"seq {sid} position {t} reads another history"
        for b in range(pool.num_blocks):
            assert pool.refcount(b) == refs[b], (b, pool.refcount(b), refs[b])
        assert pool.num_free() == sum(1 for r in refs if r == 0)


def _ops_run(bp, seed, num_blocks, prefix_caching, steps=400):
    rng = random.Random(seed)
    tr = Tracker(bp, num_blocks, 16, prefix_caching)
    prompts = [[rng.randrange(50) for _ in range(rng.choice([16, 32, 40]))] for _ in range(3)]
    live, next_id, failures = [], 0, 0
    for _ in range(steps):
        op = rng.random()
        before = tr.snapshot()
        try:
            if op < 0.3 or not live:
                base = rng.choice(prompts)
                cut = rng.randrange(1, len(base) + 1)
                tokens = base[:cut] + [rng.randrange(50) for _ in range(rng.randrange(0, 20))]
                if not tokens:
                    tokens = [1]
                tr.add(next_id, tokens)
                live.append(next_id)
                next_id += 1
            elif op < 0.75:
                tr.append(rng.choice(live), rng.randrange(50))
            elif op < 0.85:
                tr.fork(rng.choice(live), next_id)
                live.append(next_id)
                next_id += 1
            else:
                sid = rng.choice(live)
                tr.free(sid)
                live.remove(sid)
        except bp.CapacityError:
            failures += 1
            assert tr.snapshot() == before, "a refused operation changed the pool"
        tr.check()
    for sid in list(live):
        tr.free(sid)
    tr.check()
    assert tr.pool.num_free() == num_blocks
    return failures


def pin_pool_random_histories(bp):
    """Random admissions (with shared prefixes), appends, forks and frees in a
    small pool: every sequence always reads its own history, counts add up,
    and refused operations change nothing."""
    fails = 0
    for seed in range(6):
        for pc in (False, True):
            fails += _ops_run(bp, seed, num_blocks=24, prefix_caching=pc)
    assert fails > 0, "the runs never reached capacity"


def pin_pool_sizes_without_sharing(bp):
    """Without sharing a sequence of L tokens holds ceil(L / 16) blocks."""
    lens = [1, 15, 16, 17, 100, 4096]
    tr = Tracker(bp, 400)
    for i, n in enumerate(lens):
        tr.add(i, list(range(n)))
    tr.check()
    assert tr.pool.num_free() == 400 - sum(-(-n // 16) for n in lens)
    # blocks are handed out in order from a fresh pool: 0, 1, 2, ...
    assert tr.pool.block_table(0) == [0] and tr.pool.block_table(1) == [1]


def pin_pool_shared_system_prompt(bp):
    """Primer part 4, section 17.6: 32 requests of 4096 tokens that share a
    2048-token system prompt hold the prompt once: 128 + 32 x 128 = 4224
    blocks instead of 8192, each prompt block referenced 32 times."""
    rng = random.Random(7)
    system = [rng.randrange(32000) for _ in range(2048)]
    tr = Tracker(bp, 8192, 16, prefix_caching=True)
    for r in range(32):
        own = [rng.randrange(32000) for _ in range(2048)]
        _, cached = tr.add(r, system + own)
        assert cached == (0 if r == 0 else 2048), (r, cached)
    tr.check()
    assert 8192 - tr.pool.num_free() == 128 + 32 * 128
    first = tr.pool.block_table(0)
    for b in first[:128]:
        assert tr.pool.refcount(b) == 32
    for b in first[128:]:
        assert tr.pool.refcount(b) == 1
    # without prefix caching the same requests take all 8192 blocks
    tr2 = Tracker(bp, 8192)
    for r in range(32):
        tr2.add(r, system + [rng.randrange(32000) for _ in range(2048)])
    assert tr2.pool.num_free() == 0


def pin_pool_fork_copy_on_write(bp):
    """A fork shares every block; the first append into the shared, partly
    filled last block copies it, the second writes in place.  At a block
    boundary nothing is copied."""
    tr = Tracker(bp, 16)
    tr.add(0, list(range(20)))            # blocks 0, 1 (1 holds 4 tokens)
    tr.fork(0, 1)
    assert tr.pool.refcount(0) == 2 and tr.pool.refcount(1) == 2
    slot, cp = tr.append(1, 99)
    assert cp == (1, 2) and slot == 2 * 16 + 4
    slot, cp = tr.append(0, 98)
    assert cp is None and slot == 1 * 16 + 4
    tr.check()
    tr.add(2, list(range(32)))            # exactly two full blocks
    tr.fork(2, 3)
    s2, c2 = tr.append(2, 5)
    s3, c3 = tr.append(3, 6)
    assert c2 is None and c3 is None and s2 // 16 != s3 // 16
    tr.check()


def pin_pool_prefix_hits_are_exact(bp):
    """Hits need the same tokens and the same blocks before them; the final
    prompt token is never a hit."""
    tr = Tracker(bp, 64, 16, prefix_caching=True)
    a = list(range(100, 132))             # two full blocks
    tr.add(0, a + [7])
    _, c = tr.add(1, list(a))              # 32 tokens: only the first block may hit
    assert c == 16
    _, c = tr.add(2, a + [8, 9])
    assert c == 32
    b = [5] + a[1:16] + a[16:32] + [1]     # same second block, different first one
    _, c = tr.add(3, b)
    assert c == 0
    _, c = tr.add(4, a[:16] + [0] * 16 + [3])
    assert c == 16
    # the first block hits another cached prompt's; the second block's tokens
    # are cached only after a different first block: one hit, not two
    p2 = list(range(300, 316))
    tr.add(5, p2 + [1] * 16 + [2])
    _, c = tr.add(6, p2 + a[16:32] + [4])
    assert c == 16
    tr.check()


def pin_pool_eviction(bp):
    """A finished prompt's full blocks stay hittable while the pool has older
    free blocks; once they are handed out again they no longer hit."""
    tr = Tracker(bp, 8, 16, prefix_caching=True)
    p = list(range(48)) + [1]              # 3 full blocks + 1
    tr.add(0, p)
    tr.free(0)
    _, c = tr.add(1, p)
    assert c == 48                          # all three revived from the free list
    tr.free(1)
    # take every block with other content, then the old prompt must miss
    tr.add(2, [9] * 16 * 8)
    tr.free(2)
    _, c = tr.add(3, p)
    assert c == 0
    tr.check()


def pin_pool_capacity(bp):
    """Admission needs ceil(n / 16) minus the hits free blocks, counting hit
    blocks that are themselves on the free list."""
    tr = Tracker(bp, 4, 16, prefix_caching=True)
    tr.add(0, list(range(33)))             # 3 blocks
    try:
        tr.add(1, list(range(200, 233)))
        raise AssertionError("admitted beyond capacity")
    except bp.CapacityError:
        pass
    tr.free(0)
    _, c = tr.add(1, list(range(33)))       # 2 revived hits + 1 new block
    assert c == 32 and tr.pool.num_free() == 1
    tr.check()


PINS = [pin_pool_random_histories, pin_pool_sizes_without_sharing, pin_pool_shared_system_prompt,
        pin_pool_fork_copy_on_write, pin_pool_prefix_hits_are_exact, pin_pool_eviction,
        pin_pool_capacity]
