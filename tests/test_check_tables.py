"""pkv_check_tables: the host-side check of a call's block tables, context
lengths and slots (CPU only: it reads host memory and launches nothing)."""
import numpy as np
import pytest

from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W


@pytest.fixture(scope="module", autouse=True)
def lib():
    return B.load()


def expect_bad(seq, index, *args, **kw):
    with pytest.raises(B.PkvError) as e:
        B.pkv_check_tables(*args, **kw)
    assert e.value.status == B.PKV_ERR_INDEX
    assert (e.value.bad_seq, e.value.bad_index) == (seq, index), str(e.value)


@pytest.mark.parametrize("name", ["tiny", "qwen_mha", "cont_batch", "chunked_prefill",
                                  "mixed_step", "mixed_tail"])
def test_generated_workloads_pass(name):
    wl = W.CONFIGS[name]()
    B.pkv_check_tables(wl.block_tables, wl.context_lens, wl.num_blocks, wl.slot_mapping,
                       max_context_len=wl.max_context_len)


def test_mistral_batch_passes():
    wl = W.mistral_gqa(num_layers=1)
    B.pkv_check_tables(wl.block_tables, wl.context_lens, wl.num_blocks, wl.slot_mapping)


def test_entries_past_the_context_are_not_read():
    bt = np.array([[4, 2, -1, 99], [0, -7, 12345, 3]], np.int32)
    B.pkv_check_tables(bt, np.array([17, 16], np.int32), 5)   # reaches 2 and 1 blocks
    B.pkv_check_tables(bt, np.array([0, 1], np.int32), 5)


def test_context_lengths():
    bt = np.zeros((3, 2), np.int32)
    expect_bad(1, -1, bt, np.array([1, -1, 4], np.int32), 1)
    expect_bad(2, -1, bt, np.array([1, 32, 33], np.int32), 1)          # past 2 blocks of 16
    expect_bad(1, -1, bt, np.array([1, 20, 3], np.int32), 1, max_context_len=19)
    B.pkv_check_tables(bt, np.array([1, 32, 3], np.int32), 1, max_context_len=32)


def test_block_ids():
    bt = np.array([[0, 1, 2], [3, 4, 5]], np.int32)
    ctx = np.array([48, 40], np.int32)
    B.pkv_check_tables(bt, ctx, 6)
    expect_bad(1, 2, bt, ctx, 5)                     # id 5 in a pool of 5
    bt[0, 1] = -1
    expect_bad(0, 1, bt, ctx, 6)                     # the first violation is reported


def test_slots():
    bt = np.array([[0, 1]], np.int32)
    ctx = np.array([20], np.int32)
    B.pkv_check_tables(bt, ctx, 2, np.array([19, -1, 3, -5, 31], np.int32))
    expect_bad(-1, 2, bt, ctx, 2, np.array([19, -1, 32], np.int32))   # pool holds 32 slots
    expect_bad(-1, 3, bt, ctx, 2, np.array([7, -1, 8, 7], np.int32))   # 7 twice
    B.pkv_check_tables(bt, ctx, 2, np.zeros(0, np.int32))


def test_unusable_arguments():
    lib = B.load()
    assert lib.pkv_check_tables(None, 2, None, -1, -1, None, 0, 4, None, None) == B.PKV_ERR_SHAPE
    assert lib.pkv_check_tables(None, 2, None, 3, -1, None, 0, 4, None, None) == B.PKV_ERR_NULL


def first_violation(bt, ctx, nb, slots, mcl):
    """Brute force of the documented order: sequences in order (length, then
    each reached entry), then slots in order (range, then the later of two
    equal slots, smallest duplicated slot first)."""
    for s in range(bt.shape[0]):
        c = int(ctx[s])
        if c < 0 or c > bt.shape[1] * 16 or (mcl >= 0 and c > mcl):
            return (s, -1)
        for i in range(-(-c // 16)):
            if not 0 <= bt[s, i] < nb:
                return (s, i)
    for i, x in enumerate(slots):
        if x >= nb * 16:
            return (-1, i)
    seen = {}
    dups = []
    for i, x in enumerate(slots):
        if x < 0:
            continue
        if x in seen:
            dups.append((int(x), i))
        else:
            seen[int(x)] = i
    if dups:
        return (-1, min(dups)[1])
    return None


@pytest.mark.parametrize("seed", range(40))
def test_random_tables_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    s, width, nb = int(rng.integers(1, 9)), int(rng.integers(1, 6)), int(rng.integers(1, 40))
    bt = rng.integers(0, nb, (s, width)).astype(np.int32)
    ctx = rng.integers(0, width * 16 + 1, s).astype(np.int32)
    slots = rng.permutation(nb * 16)[: int(rng.integers(0, 12))].astype(np.int32)
    mcl = -1 if rng.random() < 0.5 else int(rng.integers(0, width * 16 + 1))
    kind = int(rng.integers(0, 5))
    if kind == 1:
        bt[rng.integers(0, s), rng.integers(0, width)] = int(rng.choice([-1, nb, nb + 7]))
    elif kind == 2:
        ctx[rng.integers(0, s)] = int(rng.choice([-3, width * 16 + 1]))
    elif kind == 3 and len(slots) > 1:
        slots[-1] = slots[0]
    elif kind == 4 and len(slots):
        slots[rng.integers(0, len(slots))] = nb * 16 + int(rng.integers(0, 5))
    want = first_violation(bt, ctx, nb, slots, mcl)
    if want is None:
        B.pkv_check_tables(bt, ctx, nb, slots, max_context_len=mcl)
    else:
        expect_bad(*want, bt, ctx, nb, slots, max_context_len=mcl)


def test_debug_status_needs_the_debug_build():
    """The normal build records nothing and says so."""
    with pytest.raises(B.PkvError) as e:
        B.pkv_debug_status()
    assert e.value.status == B.PKV_ERR_UNSUPPORTED
    assert B.load().pkv_debug_bounds_enabled() == 0
