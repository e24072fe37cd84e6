"""The debug-bounds build (libpkv_debug.so, PKV_DEBUG_BOUNDS): kernels that
clamp a broken device-resident index also record the first one they meet,
and pkv_debug_status returns it.  Every broken index used here is one the
clamps keep inside the pools (an out-of-range block id reads block 0, an
out-of-pool slot is skipped, a long context is cut, an out-of-range copy pair
copies nothing), so no kernel reads or writes outside its buffers."""
import numpy as np
import pytest
import torch

from gpu_cases import Case, compare, say
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu

BLOCK_ID, SLOT, CONTEXT, COPY = 1, 2, 3, 4


@pytest.fixture(scope="module")
def dbg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    lib = B.load_debug()
    assert lib.pkv_debug_bounds_enabled() == 1
    with B.using_library(lib):
        B.pkv_debug_status(clear=True)
        yield lib


def decode(c, bt=None, ctx=None, max_context_len=None, part=0):
    d, wl = c.dev, c.wl
    out = torch.empty_like(d["q"])
    B.pkv_decode_attn(d["q"], d["k_caches"][0], d["v_caches"][0],
                      d["block_tables"] if bt is None else torch.from_numpy(bt).cuda(),
                      d["context_lens"] if ctx is None else torch.from_numpy(ctx).cuda(),
                      wl.scale, out, max_context_len=max_context_len or wl.max_context_len,
                      partition_tokens=part)
    return out


@pytest.mark.parametrize("part", [0, 32, -4])
def test_clean_batch_reports_nothing(dbg, part):
    wl = W.make_decode("dbg_clean", [5, 37, 300, 16], 8, 2, 128, 1201, spare_blocks=2)
    c = Case(wl)
    say(f"[gpu] debug build: clean store + decode P={part}")
    c.gpu_store()
    out = decode(c, part=part)
    assert B.pkv_debug_status() == (0, 0, 0, 0)
    c.oracle_store()
    compare(out, c.oracle_decode(), "debug-build decode")


@pytest.mark.parametrize("part", [0, 32, -4])
def test_block_id_out_of_range(dbg, part):
    wl = W.make_decode("dbg_bid", [40, 70, 20], 8, 2, 128, 1202, store=False)
    c = Case(wl, nan_fill=False)
    bt = wl.block_tables.copy()
    bt[1, 3] = wl.num_blocks + 5          # position 3 of sequence 1 (tokens 48..63)
    say(f"[gpu] debug build: block id {bt[1, 3]} in a pool of {wl.num_blocks}, P={part}")
    decode(c, bt=bt, part=part)
    kind, value, where, n = B.pkv_debug_status()
    assert (kind, value, where) == (BLOCK_ID, wl.num_blocks + 5, 3) and n >= 1
    assert B.pkv_debug_status() == (0, 0, 0, 0)   # cleared by the read


def test_negative_block_id_in_prefill(dbg):
    wl = W.make_prefill("dbg_pf", [30, 0], [40, 20], 8, 2, 128, 1203, spare_blocks=1)
    c = Case(wl, nan_fill=False)
    c.gpu_store()
    assert B.pkv_debug_status() == (0, 0, 0, 0)
    bt = wl.block_tables.copy()
    bt[0, 2] = -7
    d = c.dev
    out = torch.empty_like(d["q"])
    say("[gpu] debug build: block id -7 in chunked prefill")
    B.pkv_prefill_attn(d["q"], d["k_caches"][0], d["v_caches"][0], torch.from_numpy(bt).cuda(),
                       d["cu_new_lens"], d["context_lens"], wl.scale, out,
                       max_new_len=wl.max_new_len, max_context_len=wl.max_context_len)
    kind, value, where, _ = B.pkv_debug_status()
    assert (kind, value, where) == (BLOCK_ID, -7, 2)


def test_slot_past_the_pool(dbg):
    wl = W.make_decode("dbg_slot", [20, 33, 7], 4, 2, 64, 1204, spare_blocks=1)
    c = Case(wl)
    slots = wl.slot_mapping.copy()
    slots[2] = wl.num_blocks * 16 + 3
    d = c.dev
    say("[gpu] debug build: a slot past the pool, store and fused store + decode")
    B.pkv_store(d["k_new"], d["v_new"], torch.from_numpy(slots).cuda(), d["k_caches"][0],
                d["v_caches"][0])
    assert B.pkv_debug_status()[:3] == (SLOT, wl.num_blocks * 16 + 3, 2)
    out = torch.empty_like(d["q"])
    B.pkv_store_decode_attn(d["k_new"], d["v_new"], torch.from_numpy(slots).cuda(), d["q"],
                            d["k_caches"][0], d["v_caches"][0], d["block_tables"],
                            d["context_lens"], wl.scale, out, max_context_len=wl.max_context_len)
    assert B.pkv_debug_status()[:3] == (SLOT, wl.num_blocks * 16 + 3, 2)


@pytest.mark.parametrize("part", [0, 16, -2])
def test_context_past_the_bound(dbg, part):
    wl = W.make_decode("dbg_ctx", [40, 33, 20], 8, 2, 128, 1205, store=False, spare_blocks=2)
    c = Case(wl, nan_fill=False)
    ctx = wl.context_lens.copy()
    # sequence 0's row holds 3 valid blocks (48 tokens): a context of 41 is
    # cut to the host bound 40 and every block it then reads is valid
    ctx[0] = 41
    say(f"[gpu] debug build: context 41 past the host bound 40, P={part}")
    decode(c, ctx=ctx, max_context_len=40, part=part)
    assert B.pkv_debug_status()[:3] == (CONTEXT, 41, 0)
    ctx[1] = -1                            # a negative context reads as empty
    decode(c, ctx=ctx, max_context_len=41, part=part)
    assert B.pkv_debug_status()[:3] == (CONTEXT, -1, 1)


def test_copy_pair_outside_the_pool(dbg):
    pool = torch.zeros((8, 4096), dtype=torch.uint8, device="cuda")
    pool[3] = 7
    copies = torch.tensor([[3, 5], [2, 99]], dtype=torch.int32, device="cuda")
    say("[gpu] debug build: block copy with a pair outside the pool")
    B.pkv_copy_blocks([pool], copies)
    assert B.pkv_debug_status()[:3] == (COPY, 99, 1)
    assert int(pool[5].min()) == 7 and int(pool[2].max()) == 0


@pytest.mark.parametrize("part", [0, 32])
def test_fp8_block_id_out_of_range(dbg, part):
    """FP8 decode: an out-of-range id met by the matrix-core path (a sequence
    past 128 keys), single pass and split-KV."""
    wl = W.make_decode("dbg_bid8", [40, 300, 20], 8, 2, 128, 1206, store=False)
    c = Case(wl, nan_fill=False)
    pools = W.make_fp8_pools(wl, device="cuda", seed=1206)
    bt = wl.block_tables.copy()
    bt[1, 3] = wl.num_blocks + 5
    d = c.dev
    out = torch.empty_like(d["q"])
    say(f"[gpu] debug build: FP8 decode, block id {bt[1, 3]} in a pool of {wl.num_blocks}, P={part}")
    B.pkv_decode_attn_fp8(d["q"], *pools, torch.from_numpy(bt).cuda(), d["context_lens"], wl.scale,
                          out, max_context_len=wl.max_context_len, partition_tokens=part)
    kind, value, where, _ = B.pkv_debug_status()
    assert (kind, value, where) == (BLOCK_ID, wl.num_blocks + 5, 3)


def test_fp8_negative_block_id_in_prefill(dbg):
    wl = W.make_prefill("dbg_pf8", [30, 0], [40, 20], 8, 2, 128, 1207, spare_blocks=1)
    c = Case(wl, nan_fill=False)
    pools = W.make_fp8_pools(wl, device="cuda", seed=1207)
    bt = wl.block_tables.copy()
    bt[0, 2] = -7
    d = c.dev
    out = torch.empty_like(d["q"])
    say("[gpu] debug build: block id -7 in FP8 chunked prefill")
    B.pkv_prefill_attn_fp8(d["q"], *pools, torch.from_numpy(bt).cuda(), d["cu_new_lens"],
                           d["context_lens"], wl.scale, out, max_new_len=wl.max_new_len,
                           max_context_len=wl.max_context_len)
    kind, value, where, _ = B.pkv_debug_status()
    assert (kind, value, where) == (BLOCK_ID, -7, 2)


def test_fp8_slot_past_the_pool(dbg):
    wl = W.make_decode("dbg_slot8", [20, 33, 7], 4, 2, 64, 1208, spare_blocks=1)
    c = Case(wl)
    pools = W.make_fp8_pools(wl, device="cuda", seed=1208)
    slots = wl.slot_mapping.copy()
    slots[2] = wl.num_blocks * 16 + 3
    d = c.dev
    say("[gpu] debug build: a slot past the pool in the FP8 store")
    B.pkv_store_fp8(d["k_new"], d["v_new"], torch.from_numpy(slots).cuda(), *pools)
    assert B.pkv_debug_status()[:3] == (SLOT, wl.num_blocks * 16 + 3, 2)


def test_fp8_prefix_tail_block_id(dbg):
    """FP8 shared-prefix decode: an out-of-range id in a grouped sequence's
    tail, met by a tail wave on the matrix-core path."""
    ctx = [320 + t for t in (200, 150, 40)]
    wl = W.make_decode("dbg_px8", ctx, 8, 2, 128, 1209, prefix_groups=[[0, 1, 2]],
                       prefix_tokens=320, store=False)
    c = Case(wl, nan_fill=False)
    pools = W.make_fp8_pools(wl, device="cuda", seed=1209)
    bt = wl.block_tables.copy()
    bt[1, 22] = wl.num_blocks + 9          # block 22: tokens 352..367, in sequence 1's tail
    d = c.dev
    out = torch.empty_like(d["q"])
    say("[gpu] debug build: FP8 shared-prefix decode, a tail block id past the pool")
    B.pkv_decode_attn_prefix_fp8(d["q"], *pools, torch.from_numpy(bt).cuda(), d["context_lens"],
                                 wl.scale, out, torch.tensor([0, 3], dtype=torch.int32, device="cuda"),
                                 torch.tensor([320], dtype=torch.int32, device="cuda"), 3,
                                 max_context_len=wl.max_context_len)
    kind, value, where, _ = B.pkv_debug_status()
    assert (kind, value, where) == (BLOCK_ID, wl.num_blocks + 9, 22)
