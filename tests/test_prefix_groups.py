"""pkv_prefix_groups, the host helper that finds groups of consecutive
sequences sharing leading physical blocks: hand cases, then properties on
seeded random batches -- every group's members really hold the same blocks
over its prefix, the prefix is whole blocks within every member's context,
groups tile the batch in order, and each is maximal under the documented
rule."""
import numpy as np
import pytest

from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W


@pytest.fixture(scope="module", autouse=True)
def lib():
    B.load()


def groups(bt, ctx, min_tokens=16):
    return B.pkv_prefix_groups(np.asarray(bt, np.int32), np.asarray(ctx, np.int32), min_tokens)


def test_hand_cases():
    # rows share blocks 7, 8 (two groups of two, then a loner)
    bt = [[7, 8, 1], [7, 8, 2], [9, 3, 0], [9, 3, 4], [5, 6, 0]]
    ctx = [40, 33, 32, 48, 20]
    starts, plens, mg = groups(bt, ctx)
    assert list(starts) == [0, 2, 4, 5] and list(plens) == [32, 32, 0] and mg == 2
    # the prefix stops at the shorter context's whole blocks: 20 tokens -> 1 block
    starts, plens, _ = groups([[7, 8, 1], [7, 8, 2]], [40, 20])
    assert list(plens) == [16]
    # a context of 15 tokens has no whole block to share
    starts, plens, mg = groups([[7, 8], [7, 8]], [40, 15])
    assert list(starts) == [0, 2] and list(plens) == [0] and mg == 0
    # min_prefix_tokens: 32 shared tokens are not enough for 48
    starts, plens, _ = groups(bt[:2], ctx[:2], min_tokens=48)
    assert list(plens) == [0]
    # a third row sharing only the first block ends the run of the first two
    starts, plens, _ = groups([[7, 8, 1], [7, 8, 2], [7, 9, 3]], [48, 48, 48])
    assert list(starts) == [0, 2, 3] and list(plens) == [32, 0]
    # empty batch
    starts, plens, mg = groups(np.zeros((0, 4)), [])
    assert list(starts) == [0] and len(plens) == 0 and mg == 0


def test_cont_batch_groups():
    wl = W.cont_batch()
    starts, plens, mg = groups(wl.block_tables, wl.context_lens)
    assert list(starts) == list(range(0, 257, 32)) and list(plens) == [2048] * 8 and mg == 32


def shared_blocks(bt, ctx, a, b):
    n = min(ctx[a] // 16, ctx[b] // 16)
    i = 0
    while i < n and bt[a][i] == bt[b][i]:
        i += 1
    return i


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = np.random.default_rng(seed)
    s = int(rng.integers(1, 60))
    width = 12
    # families of rows with common leading blocks of random lengths
    bt = np.zeros((s, width), np.int32)
    ctx = rng.integers(0, width * 16 + 1, size=s).astype(np.int32)
    nxt = 0
    i = 0
    while i < s:
        fam = int(rng.integers(1, 6))
        share = int(rng.integers(0, width))
        base = np.arange(nxt, nxt + width, dtype=np.int32)
        nxt += width
        for j in range(i, min(s, i + fam)):
            row = np.arange(nxt, nxt + width, dtype=np.int32)
            nxt += width
            row[:share] = base[:share]
            bt[j] = row
        i += fam
    min_tokens = int(rng.choice([16, 32, 64]))
    starts, plens, mg = groups(bt, ctx, min_tokens)
    assert starts[0] == 0 and starts[-1] == s and np.all(np.diff(starts) >= 1)
    biggest = 0
    for g in range(len(plens)):
        a, b, p = int(starts[g]), int(starts[g + 1]), int(plens[g])
        assert p % 16 == 0
        if p == 0:
            continue
        biggest = max(biggest, b - a)
        assert b - a >= 2 and p >= min_tokens
        for m in range(a, b):
            assert ctx[m] >= p and np.array_equal(bt[m][: p // 16], bt[a][: p // 16])
        # the prefix is what the first two share; the next row does not share that much
        assert p // 16 == shared_blocks(bt, ctx, a, a + 1)
        if b < s:
            assert shared_blocks(bt, ctx, a, b) < p // 16
    assert mg == biggest
    # a sequence left out of every group shares too little with its successor to start one
    for g in range(len(plens)):
        if plens[g] == 0:
            for m in range(int(starts[g]), int(starts[g + 1])):
                if m + 1 < s:
                    assert shared_blocks(bt, ctx, m, m + 1) * 16 < max(min_tokens, 16)
