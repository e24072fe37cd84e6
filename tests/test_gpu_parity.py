"""GPU parity: libpkv's HIP kernels against the fp64 oracle on the same seeded
inputs.  Store must be bit-exact; attention within max |err| 1e-2 and mean
|err| 1e-3 of the oracle (bf16 in, fp32 accumulate, bf16 out).
"""
import numpy as np
import pytest
import torch

from gpu_cases import (Case, assert_pool_matches, compact_for_oracle, compare, fp8_nan_pools,
                       fp8_quantized_pools, orc, say, bits, to_f64)
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    say(f"[gpu] {torch.cuda.get_device_name(0)}")


# ---------------------------------------------------------------------------
# store
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "qwen_mha", "cont_batch", "chunked_prefill"])
def test_store_bit_exact(name):
    wl = W.CONFIGS[name]()
    say(f"[gpu] store {name}: T={wl.num_tokens} pool={wl.num_blocks} blocks")
    c = Case(wl)
    c.gpu_store()
    torch.cuda.synchronize()
    c.oracle_store()
    assert np.array_equal(bits(c.dev["k_caches"][0]), c.h["kc"])
    assert np.array_equal(bits(c.dev["v_caches"][0]), c.h["vc"])


def test_store_skips_negative_and_out_of_pool_slots():
    wl = W.make_decode("store_skip", [20, 33, 7, 16], 4, 2, 128, 41, spare_blocks=2)
    wl.slot_mapping[1] = -1
    wl.slot_mapping[3] = wl.num_blocks * 16 + 5   # outside the pool: never written
    say("[gpu] store with slot -1 and an out-of-pool slot")
    c = Case(wl)
    before = bits(c.dev["k_caches"][0]).copy()
    c.gpu_store()
    torch.cuda.synchronize()
    after = bits(c.dev["k_caches"][0])
    # exactly the two valid slots changed
    for i, s in enumerate(wl.slot_mapping):
        if 0 <= s < wl.num_blocks * 16:
            assert np.array_equal(after[s // 16, :, s % 16], c.h["k_new"][i])
    changed = np.argwhere(np.any(after != before, axis=(1, 3)))
    valid = {(int(s) // 16, int(s) % 16) for s in wl.slot_mapping if 0 <= s < wl.num_blocks * 16}
    assert {(int(b), int(o)) for b, o in changed} <= valid


# ---------------------------------------------------------------------------
# decode: whole problems checked element by element
# ---------------------------------------------------------------------------

def run_decode_full(wl, partition_tokens=0, max_context_len=None):
    c = Case(wl)
    say(f"[gpu] decode {wl.name}: S={wl.num_seqs} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"d={wl.head_dim} max_ctx={wl.max_context_len} P={partition_tokens or 'auto'}")
    c.gpu_store()
    out = c.gpu_decode(partition_tokens=partition_tokens, max_context_len=max_context_len)
    torch.cuda.synchronize()
    c.oracle_store()
    ref = c.oracle_decode()
    compare(out, ref, f"decode {wl.name}")
    return c, out, ref


def test_decode_tiny():
    run_decode_full(W.tiny())


def test_decode_qwen_mha():
    run_decode_full(W.qwen_mha())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("part", [16, 64, 0, -1, -3, -8])
def test_decode_edge_lengths(d, g, part):
    lens = [1, 15, 16, 17, 32, 63, 64, 65, 129, 0, 2]
    wl = W.make_decode(f"edge_d{d}_g{g}", lens, 2 * g, 2, d, 100 + d + g, spare_blocks=3)
    run_decode_full(wl, partition_tokens=part)


def test_decode_single_token_exact():
    """One cached token: out must equal the stored V bit for bit."""
    wl = W.make_decode("ctx1", [1, 1, 1, 1], 8, 2, 128, 51, spare_blocks=1)
    c = Case(wl)
    c.gpu_store()
    out = c.gpu_decode()
    torch.cuda.synchronize()
    got = bits(out)
    for s in range(wl.num_seqs):
        for h in range(wl.num_q_heads):
            assert np.array_equal(got[s, h], c.h["v_new"][s, h // 4]), (s, h)


@pytest.mark.parametrize("part", [16, -2])
def test_decode_empty_context_is_zero(part):
    wl = W.make_decode("ctx0", [0, 40, 0], 4, 2, 64, 52, store=False)
    c = Case(wl)
    out = c.gpu_decode(partition_tokens=part)
    torch.cuda.synchronize()
    assert np.all(to_f64(out)[[0, 2]] == 0.0)
    compare(out, c.oracle_decode(), "decode ctx0")


@pytest.mark.parametrize("part", [16, 48, 256, 1024, -2, -8])
def test_decode_partition_sizes(part):
    wl = W.make_decode("parts", [300, 1000, 17, 2048], 16, 4, 128, 53)
    run_decode_full(wl, partition_tokens=part)


def test_decode_auto_many_units():
    """More (sequence, KV head) units than compute units, contexts up to 4096:
    the automatic choice is the single-pass kernel with 8 waves per unit."""
    ctx = np.random.default_rng(56).integers(1000, 4097, 40).tolist()  # 320 units
    wl = W.make_decode("many_units", ctx, 32, 8, 128, 57)
    assert B.pkv_decode_partition_tokens(wl.num_seqs, wl.num_kv_heads, wl.max_context_len) == -8
    run_decode_full(wl)


def test_decode_loose_max_context_len():
    """A host bound larger than any context only adds empty partitions."""
    wl = W.make_decode("loose", [100, 37], 8, 2, 128, 54)
    wl.block_tables = np.concatenate([wl.block_tables, np.full((2, 30), -1, np.int32)], axis=1)
    run_decode_full(wl, max_context_len=wl.max_blocks_per_seq * 16)


def test_decode_prefix_shared_equals_copied():
    """Sequences pointing at shared prefix blocks give bit-identical output to
    the same sequences with the prefix copied into private blocks."""
    lens = [64 + 20, 64 + 3, 64 + 50]
    shared = W.make_decode("shared", lens, 8, 2, 128, 55, prefix_groups=[[0, 1, 2]],
                           prefix_tokens=64, store=False)
    c = Case(shared, nan_fill=True)
    out_shared = c.gpu_decode()
    # copy: give every sequence private prefix blocks holding the same bits
    kc, vc = c.dev["k_caches"][0], c.dev["v_caches"][0]
    nb = shared.num_blocks
    pre = shared.block_tables[0, :4].copy()
    kc2 = torch.cat([kc, kc[torch.from_numpy(np.concatenate([pre, pre])).long().cuda()]], 0)
    vc2 = torch.cat([vc, vc[torch.from_numpy(np.concatenate([pre, pre])).long().cuda()]], 0)
    bt2 = shared.block_tables.copy()
    bt2[1, :4] = np.arange(nb, nb + 4)
    bt2[2, :4] = np.arange(nb + 4, nb + 8)
    out_copied = torch.empty_like(out_shared)
    B.pkv_decode_attn(c.dev["q"], kc2.contiguous(), vc2.contiguous(),
                      torch.from_numpy(bt2).cuda(), c.dev["context_lens"], shared.scale, out_copied,
                      max_context_len=shared.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_shared), bits(out_copied))
    compare(out_shared, c.oracle_decode(), "decode shared prefix")


def test_decode_block_permutation_bit_identical():
    wl = W.make_decode("perm", [200, 45, 16], 8, 2, 128, 56, spare_blocks=5)
    c = Case(wl)
    c.gpu_store()
    out = c.gpu_decode()
    perm = np.random.default_rng(9).permutation(wl.num_blocks)
    inv = torch.from_numpy(np.argsort(perm)).long().cuda()
    kc2 = c.dev["k_caches"][0][inv].contiguous()   # new block perm[b] holds old block b
    vc2 = c.dev["v_caches"][0][inv].contiguous()
    bt2 = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    out2 = torch.empty_like(out)
    B.pkv_decode_attn(c.dev["q"], kc2, vc2, torch.from_numpy(bt2).cuda(), c.dev["context_lens"],
                      wl.scale, out2, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(out2))


# ---------------------------------------------------------------------------
# decode at full size, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

def run_decode_full_size(wl, layers=1):
    """Store + decode of the whole batch on every layer; the oracle computes
    every sequence from pre-store host copies, and the pools after the store
    must equal the oracle's bit for bit."""
    seqs = range(wl.num_seqs)
    say(f"[gpu] decode {wl.name} full size: S={wl.num_seqs} max_ctx={wl.max_context_len} "
        f"pool={wl.num_blocks} blocks, {layers} layer(s); oracle on every sequence")
    t = W.make_tensors(wl, device="cuda", layers=layers, nan_fill=True)
    hosts = [compact_for_oracle(wl, t, seqs, layer=l) for l in range(layers)]
    d = {k: t[k] for k in ("q", "k_new", "v_new", "block_tables", "context_lens", "slot_mapping")}
    outs = []
    for l in range(layers):
        B.pkv_store(d["k_new"], d["v_new"], d["slot_mapping"], t["k_caches"][l], t["v_caches"][l])
        out = torch.empty_like(d["q"])
        B.pkv_decode_attn(d["q"], t["k_caches"][l], t["v_caches"][l], d["block_tables"],
                          d["context_lens"], wl.scale, out, max_context_len=wl.max_context_len)
        outs.append(out)
    torch.cuda.synchronize()
    for l, h in enumerate(hosts):
        orc().store(h["k_new"], h["v_new"], h["slots"], h["kc"], h["vc"])
        assert_pool_matches(t["k_caches"][l], h["ids"], h["kc"], f"K pool layer {l}")
        assert_pool_matches(t["v_caches"][l], h["ids"], h["vc"], f"V pool layer {l}")
        ref = orc().decode(h["q"], h["kc"], h["vc"], h["bt"], h["ctx"], wl.scale)
        compare(outs[l], ref, f"decode {wl.name} layer {l}")
    del t


def test_decode_mistral_gqa_full_size():
    """32 x 4096 GQA batch, two layers: the automatic choice is the
    single-pass kernel."""
    assert B.pkv_decode_partition_tokens(32, 8, 4096) < 0
    run_decode_full_size(W.mistral_gqa(num_layers=2), layers=2)


def test_decode_cont_batch_full_size():
    """All 256 sequences of the continuous batch (contexts 2064 .. 32768)
    through plain split-KV decode."""
    run_decode_full_size(W.cont_batch())


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_prefill_small(d, g):
    cached = [0, 37, 5, 300]
    new = [70, 16, 1, 129]
    wl = W.make_prefill(f"prefill_d{d}_g{g}", cached, new, 2 * g, 2, d, 200 + d + g, spare_blocks=2)
    c = Case(wl)
    say(f"[gpu] prefill {wl.name}: cached {cached} new {new}")
    c.gpu_store()
    out = c.gpu_prefill()
    torch.cuda.synchronize()
    c.oracle_store()
    compare(out, c.oracle_prefill(), f"prefill {wl.name}")


@pytest.mark.parametrize("g", [1, 4])
def test_prefill_precise_boundary(g):
    """Waves whose last query sits below position 128 carry P as bf16 hi + lo; the
    rest use P rounded to bf16 with the weight sum from the same rounded
    weights.  Prompts whose waves straddle 128 keys (0 cached and 200 new;
    100 cached and 60 new; 127 cached and 2 new) check both kinds against the
    oracle, including the rows just past the boundary."""
    wl = W.make_prefill(f"prefill_boundary_g{g}", [0, 100, 127], [200, 60, 2], 8 * g, 8, 128,
                        300 + g, spare_blocks=1)
    c = Case(wl)
    say(f"[gpu] prefill precise boundary G={g}")
    c.gpu_store()
    out = c.gpu_prefill()
    torch.cuda.synchronize()
    c.oracle_store()
    compare(out, c.oracle_prefill(), f"prefill boundary G={g}")


def test_prefill_chunked_full_size():
    """The 8 x 2048-token chunked prefill (cached 336 .. 3925 tokens), in the
    launch the benchmark times: every row of every prompt against the
    oracle's chunked prefill, and the store bit-exact."""
    wl = W.chunked_prefill()
    say(f"[gpu] prefill {wl.name} full size: cached {list(wl.context_lens - wl.new_lens)}; "
        f"oracle on every row")
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    h = compact_for_oracle(wl, t, range(wl.num_seqs))
    d = t
    B.pkv_store(d["k_new"], d["v_new"], d["slot_mapping"], d["k_caches"][0], d["v_caches"][0])
    out = torch.empty_like(d["q"])
    B.pkv_prefill_attn(d["q"], d["k_caches"][0], d["v_caches"][0], d["block_tables"],
                       d["cu_new_lens"], d["context_lens"], wl.scale, out,
                       max_new_len=wl.max_new_len, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    orc().store(h["k_new"], h["v_new"], h["slots"], h["kc"], h["vc"])
    assert_pool_matches(d["k_caches"][0], h["ids"], h["kc"], "K pool")
    assert_pool_matches(d["v_caches"][0], h["ids"], h["vc"], "V pool")
    cu = np.concatenate([[0], np.cumsum(h["new_lens"])]).astype(np.int32)
    ref = orc().prefill(h["q"], h["kc"], h["vc"], h["bt"], cu, h["ctx"], wl.scale)
    assert np.array_equal(h["tok"], np.arange(wl.num_tokens))
    compare(out, ref, "prefill chunked full size (every row)")


# ---------------------------------------------------------------------------
# scale edge cases: zero (every visible key weighs the same) and negative
# (prefill applies it by flipping q's sign bits).  Sharp scales push outputs
# toward single V values, some of magnitude >= 4, so the bound adds each
# element's own bf16 rounding to 1e-2.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_prefill_scale_edges(scale):
    wl = W.make_prefill("prefill_scale", [0, 37, 130], [70, 16, 65], 8, 2, 128, 61,
                        scale=scale, spare_blocks=1)
    c = Case(wl)
    say(f"[gpu] prefill scale {scale}")
    c.gpu_store()
    out = c.gpu_prefill()
    torch.cuda.synchronize()
    c.oracle_store()
    compare(out, c.oracle_prefill(), f"prefill scale {scale}", plus_floor=True)


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
@pytest.mark.parametrize("part", [0, 32])
def test_decode_scale_edges(scale, part):
    wl = W.make_decode("decode_scale", [1, 40, 300, 17], 8, 2, 128, 62, scale=scale,
                       spare_blocks=1)
    c = Case(wl)
    say(f"[gpu] decode scale {scale} P={part}")
    c.gpu_store()
    out = c.gpu_decode(partition_tokens=part)
    torch.cuda.synchronize()
    c.oracle_store()
    compare(out, c.oracle_decode(), f"decode scale {scale}", plus_floor=True)


# ---------------------------------------------------------------------------
# fused store + decode: bit-identical to pkv_store followed by pkv_decode_attn
# (same arithmetic, the new token's K/V taken from registers instead of the
# cache), and within tolerance of the oracle
# ---------------------------------------------------------------------------

def fused_vs_separate(wl, partition_tokens=0, slots=None, what=None, prep=None):
    c = Case(wl)
    if prep is not None:
        prep(c)
    d = c.dev
    slot_t = d["slot_mapping"] if slots is None else torch.from_numpy(slots).cuda()
    kc2 = [x.clone() for x in d["k_caches"]]
    vc2 = [x.clone() for x in d["v_caches"]]
    say(f"[gpu] fused store+decode {what or wl.name}: S={wl.num_seqs} G={wl.num_q_heads // wl.num_kv_heads} "
        f"d={wl.head_dim} P={partition_tokens or 'auto'}")
    # separate
    B.pkv_store(d["k_new"], d["v_new"], slot_t, d["k_caches"][0], d["v_caches"][0])
    out_sep = torch.empty_like(d["q"])
    B.pkv_decode_attn(d["q"], d["k_caches"][0], d["v_caches"][0], d["block_tables"],
                      d["context_lens"], wl.scale, out_sep, max_context_len=wl.max_context_len,
                      partition_tokens=partition_tokens)
    # fused
    out_fused = torch.empty_like(d["q"])
    B.pkv_store_decode_attn(d["k_new"], d["v_new"], slot_t, d["q"], kc2[0], vc2[0],
                            d["block_tables"], d["context_lens"], wl.scale, out_fused,
                            max_context_len=wl.max_context_len, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc2[0]), bits(d["k_caches"][0])), "fused store differs (K)"
    assert np.array_equal(bits(vc2[0]), bits(d["v_caches"][0])), "fused store differs (V)"
    assert np.array_equal(bits(out_fused), bits(out_sep)), "fused attention differs"
    return c, out_fused


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
@pytest.mark.parametrize("part", [16, 64, 0, -1, -3])
def test_fused_store_decode_matches_separate(d, g, part):
    lens = [1, 15, 16, 17, 63, 64, 65, 129, 300]
    wl = W.make_decode(f"fused_d{d}_g{g}", lens, 2 * g, 2, d, 300 + d + g, spare_blocks=2)
    c, out = fused_vs_separate(wl, part)
    c.oracle_store()
    compare(out, c.oracle_decode(), f"fused store+decode d{d} g{g} P{part}")


def test_fused_store_decode_skips_and_strays():
    """slot -1 stores nothing and attends over the cache as it is; a slot in a
    spare block is stored but is not the last position's, so attention reads
    the cache there; a sequence with no context stores and outputs zero."""
    wl = W.make_decode("fused_edges", [20, 33, 7, 0, 40], 8, 2, 128, 63, spare_blocks=2)
    spare = sorted(set(range(wl.num_blocks)) - set(wl.used_blocks().tolist()))
    assert len(spare) == 2
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    slots[2] = spare[0] * 16 + 3      # an unreferenced block: not position ctx-1's slot
    slots[3] = spare[1] * 16 + 0      # ctx 0: store only

    def cached_earlier(c):
        # sequences 1 and 2 store nothing at their last position, so it must
        # already hold a token: write one there (the generator left NaN)
        for s in (1, 2):
            slot = int(wl.slot_mapping[s])
            for cache, host, src in ((c.dev["k_caches"][0], c.h["kc"], c.dev["k_new"]),
                                     (c.dev["v_caches"][0], c.h["vc"], c.dev["v_new"])):
                row = (src[s] * 0.5).to(torch.bfloat16)
                cache[slot // 16, :, slot % 16] = row
                host[slot // 16, :, slot % 16] = bits(row)

    c, out = fused_vs_separate(wl, 0, slots=slots, what="edges", prep=cached_earlier)
    assert np.all(to_f64(out)[3] == 0.0)
    orc().store(c.h["k_new"], c.h["v_new"], slots, c.h["kc"], c.h["vc"])
    compare(out, c.oracle_decode(), "fused store+decode edges")


def test_fused_store_decode_mistral_full_size():
    """The benchmark's launch: 32 x 4096 GQA, single-pass split, two layers.
    Every sequence against the oracle, and both pools after the step (the 32
    stored K and V rows and every slot the step must leave alone) bit-exact."""
    wl = W.mistral_gqa(num_layers=2)
    seqs = range(wl.num_seqs)
    say("[gpu] fused store+decode full size, oracle on every sequence")
    t = W.make_tensors(wl, device="cuda", layers=2, nan_fill=True)
    hosts = [compact_for_oracle(wl, t, seqs, layer=l) for l in range(2)]
    outs = []
    for l in range(2):
        out = torch.empty_like(t["q"])
        B.pkv_store_decode_attn(t["k_new"], t["v_new"], t["slot_mapping"], t["q"],
                                t["k_caches"][l], t["v_caches"][l], t["block_tables"],
                                t["context_lens"], wl.scale, out,
                                max_context_len=wl.max_context_len)
        outs.append(out)
    torch.cuda.synchronize()
    for l, h in enumerate(hosts):
        orc().store(h["k_new"], h["v_new"], h["slots"], h["kc"], h["vc"])
        assert_pool_matches(t["k_caches"][l], h["ids"], h["kc"], f"K pool layer {l}")
        assert_pool_matches(t["v_caches"][l], h["ids"], h["vc"], f"V pool layer {l}")
        ref = orc().decode(h["q"], h["kc"], h["vc"], h["bt"], h["ctx"], wl.scale)
        compare(outs[l], ref, f"fused store+decode full size layer {l}")


# ---------------------------------------------------------------------------
# rotary position embedding fused into store + decode: q and the new k are
# rotated at position ctx - 1 (the oracle rotates them on the host, then stores
# and attends with the rotated rows)
# ---------------------------------------------------------------------------

def run_rope(c, table, partition_tokens=0, slots=None):
    d = c.dev
    wl = c.wl
    slot_t = d["slot_mapping"] if slots is None else torch.from_numpy(slots).cuda()
    out = torch.empty_like(d["q"])
    B.pkv_store_decode_attn_rope(d["k_new"], d["v_new"], slot_t, d["q"],
                                 torch.from_numpy(table).cuda(), d["k_caches"][0],
                                 d["v_caches"][0], d["block_tables"], d["context_lens"], wl.scale,
                                 out, max_context_len=wl.max_context_len,
                                 partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out


def oracle_rope_step(c, table, slots=None):
    """Host reference: rotate q and the new k at max(ctx - 1, 0), store the
    rotated k (and v as it is), attend with the rotated q."""
    wl, h = c.wl, c.h
    pos = np.maximum(wl.context_lens.astype(np.int32) - 1, 0).astype(np.int32)
    q_rot = orc().rope(h["q"], pos, table)
    k_rot = orc().rope(h["k_new"], pos, table)
    orc().store(k_rot, h["v_new"], wl.slot_mapping if slots is None else slots, h["kc"], h["vc"])
    return orc().decode(q_rot, h["kc"], h["vc"], wl.block_tables, wl.context_lens, wl.scale)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
@pytest.mark.parametrize("part", [16, 64, 0, -1, -3])
def test_rope_store_decode(d, g, part):
    lens = [1, 15, 16, 17, 63, 64, 65, 129, 300]
    wl = W.make_decode(f"rope_d{d}_g{g}", lens, 2 * g, 2, d, 500 + d + g, spare_blocks=2)
    table = W.rope_table(wl.max_context_len + 37, d)
    c = Case(wl)
    say(f"[gpu] rope store+decode d={d} G={g} P={part or 'auto'}")
    out = run_rope(c, table, part)
    ref = oracle_rope_step(c, table)
    assert np.array_equal(bits(c.dev["k_caches"][0]), c.h["kc"]), "rotated K store differs"
    assert np.array_equal(bits(c.dev["v_caches"][0]), c.h["vc"]), "V store differs"
    compare(out, ref, f"rope store+decode d{d} g{g} P{part}")


@pytest.mark.parametrize("part", [0, 32])
def test_rope_identity_table_is_plain_fused(part):
    """cos 1, sin 0 at every position: the rotation is exact, so the step is
    bit-identical to pkv_store_decode_attn."""
    wl = W.make_decode("rope_identity", [5, 16, 77, 200], 16, 4, 128, 71, spare_blocks=1)
    table = np.zeros((wl.max_context_len, 128), np.float32)
    table[:, :64] = 1.0
    c = Case(wl)
    kc2 = c.dev["k_caches"][0].clone()
    vc2 = c.dev["v_caches"][0].clone()
    say(f"[gpu] rope identity table P={part or 'auto'}")
    out = run_rope(c, table, part)
    d = c.dev
    plain = torch.empty_like(d["q"])
    B.pkv_store_decode_attn(d["k_new"], d["v_new"], d["slot_mapping"], d["q"], kc2, vc2,
                            d["block_tables"], d["context_lens"], wl.scale, plain,
                            max_context_len=wl.max_context_len, partition_tokens=part)
    torch.cuda.synchronize()
    assert np.array_equal(bits(kc2), bits(d["k_caches"][0]))
    assert np.array_equal(bits(vc2), bits(d["v_caches"][0]))
    assert np.array_equal(bits(plain), bits(out))


def test_rope_table_exactly_covers_context():
    """max_positions == max_context_len: the last row is the one used."""
    wl = W.make_decode("rope_exact_table", [48, 3, 48], 8, 2, 128, 72)
    table = W.rope_table(wl.max_context_len, 128)
    c = Case(wl)
    say("[gpu] rope table of exactly max_context_len rows")
    out = run_rope(c, table)
    ref = oracle_rope_step(c, table)
    assert np.array_equal(bits(c.dev["k_caches"][0]), c.h["kc"])
    compare(out, ref, "rope exact table")


def test_rope_skips_and_empty_context():
    """slot -1 stores nothing (the cached row at ctx - 1 is used as it is); a
    sequence with no context stores its k rotated at position 0 and outputs 0."""
    wl = W.make_decode("rope_edges", [20, 33, 0, 40], 8, 2, 64, 73, spare_blocks=1)
    spare = sorted(set(range(wl.num_blocks)) - set(wl.used_blocks().tolist()))
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    slots[2] = spare[0] * 16 + 5
    table = W.rope_table(64, 64)
    c = Case(wl)
    # sequence 1 stores nothing: its last position must already hold a token
    slot = int(wl.slot_mapping[1])
    for cache, host, src in ((c.dev["k_caches"][0], c.h["kc"], c.dev["k_new"]),
                             (c.dev["v_caches"][0], c.h["vc"], c.dev["v_new"])):
        row = (src[1] * 0.5).to(torch.bfloat16)
        cache[slot // 16, :, slot % 16] = row
        host[slot // 16, :, slot % 16] = bits(row)
    say("[gpu] rope edges (skip, empty context)")
    out = run_rope(c, table, 0, slots=slots)
    ref = oracle_rope_step(c, table, slots=slots)
    assert np.array_equal(bits(c.dev["k_caches"][0]), c.h["kc"])
    assert np.all(to_f64(out)[2] == 0.0)
    compare(out, ref, "rope edges")


def test_rope_mistral_full_size():
    """The benchmark's shape (32 x 4096 GQA, single pass) with the rotation
    fused: every sequence against the oracle, the pools bit-exact."""
    wl = W.mistral_gqa(num_layers=1)
    seqs = range(wl.num_seqs)
    table = W.rope_table(wl.max_context_len, wl.head_dim)
    say("[gpu] rope store+decode full size, oracle on every sequence")
    t = W.make_tensors(wl, device="cuda", layers=1, nan_fill=True)
    h = compact_for_oracle(wl, t, seqs)
    out = torch.empty_like(t["q"])
    B.pkv_store_decode_attn_rope(t["k_new"], t["v_new"], t["slot_mapping"], t["q"],
                                 torch.from_numpy(table).cuda(), t["k_caches"][0],
                                 t["v_caches"][0], t["block_tables"], t["context_lens"], wl.scale,
                                 out, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    pos = (h["ctx"] - 1).astype(np.int32)
    k_rot = orc().rope(h["k_new"], pos, table)
    orc().store(k_rot, h["v_new"], h["slots"], h["kc"], h["vc"])
    assert_pool_matches(t["k_caches"][0], h["ids"], h["kc"], "rotated K pool")
    assert_pool_matches(t["v_caches"][0], h["ids"], h["vc"], "V pool")
    ref = orc().decode(orc().rope(h["q"], pos, table), h["kc"], h["vc"], h["bt"], h["ctx"],
                       wl.scale)
    compare(out, ref, "rope store+decode full size")


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3, one fp32 scale per token and KV head) cache.
#
# Two kinds of input.  Pools of uniformly random codes and scales reach every
# code (subnormals, the extremes, NaN sentinels) but give dequantized values up
# to about 5, so rows dominated by one key have outputs whose own bf16
# rounding reaches 1.56e-2: those tests add each element's bf16 rounding to
# the 1e-2 bound.  Pools filled the serving way -- N(0,1) bf16 K/V quantized
# by the FP8 store, the GPU's pools by pkv_store_fp8 and the oracle's by its
# own store from the same bits -- are held to the plain bound.
# ---------------------------------------------------------------------------

def fp8_case(wl, nan_fill=True):
    """Host and device FP8 pools for one layer (random codes and scales)."""
    pools = W.make_fp8_pools(wl, device="cpu", nan_fill=nan_fill)
    host = [x.numpy().copy() for x in pools]
    dev = [x.cuda() for x in pools]
    return host, dev


@pytest.mark.parametrize("name", ["tiny", "qwen_mha", "chunked_prefill"])
def test_store_fp8_bit_exact(name):
    wl = W.CONFIGS[name]()
    say(f"[gpu] store fp8 {name}: T={wl.num_tokens}")
    c = Case(wl)
    host, dev = fp8_case(wl)
    slot_t = c.dev["slot_mapping"]
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], slot_t, *dev)
    torch.cuda.synchronize()
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    for got, ref, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        g = got.cpu().numpy()
        assert np.array_equal(g.view(np.uint8), ref.view(np.uint8)), what


def test_store_fp8_skips_and_d64():
    wl = W.make_decode("fp8_skip", [20, 33, 7, 16], 4, 2, 64, 71, spare_blocks=2)
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    slots[3] = wl.num_blocks * 16 + 2      # outside the pool: never written
    c = Case(wl)
    host, dev = fp8_case(wl)
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], torch.from_numpy(slots).cuda(), *dev)
    torch.cuda.synchronize()
    slots_oracle = slots.copy()
    slots_oracle[3] = -1                   # the oracle rejects out-of-pool slots
    orc().store_fp8(c.h["k_new"], c.h["v_new"], slots_oracle, *host)
    for got, ref in zip(dev, host):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
@pytest.mark.parametrize("part", [16, 64, 0, -1, -3])
def test_decode_fp8_edge_lengths(d, g, part):
    lens = [1, 15, 16, 17, 63, 64, 65, 129, 0, 300]
    wl = W.make_decode(f"fp8_d{d}_g{g}", lens, 2 * g, 2, d, 400 + d + g, spare_blocks=2,
                       store=False)
    c = Case(wl)
    host, dev = fp8_case(wl)
    say(f"[gpu] decode fp8 d={d} G={g} P={part}")
    out = torch.empty_like(c.dev["q"])
    B.pkv_decode_attn_fp8(c.dev["q"], *dev, c.dev["block_tables"], c.dev["context_lens"],
                          wl.scale, out, max_context_len=wl.max_context_len, partition_tokens=part)
    torch.cuda.synchronize()
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, f"decode fp8 d{d} g{g} P{part}", plus_floor=True)


def test_store_then_decode_fp8():
    """A decode step on an FP8 cache: quantizing store of the new tokens, then
    attention over the cache including them, against the oracle doing both."""
    wl = W.make_decode("fp8_step", [5, 37, 200, 1, 64], 8, 2, 128, 72, spare_blocks=1)
    c = Case(wl)
    host, dev = fp8_case(wl)
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], c.dev["slot_mapping"], *dev)
    out = torch.empty_like(c.dev["q"])
    B.pkv_decode_attn_fp8(c.dev["q"], *dev, c.dev["block_tables"], c.dev["context_lens"],
                          wl.scale, out, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, "store + decode fp8", plus_floor=True)


def fused_fp8_vs_separate(wl, partition_tokens=0, slots=None, what=None, nan_fill=True):
    """pkv_store_decode_attn_fp8 against pkv_store_fp8 + pkv_decode_attn_fp8
    on copies of the same pools: codes, scales and output bit for bit."""
    c = Case(wl)
    host, dev = fp8_case(wl, nan_fill=nan_fill)
    dev2 = [x.clone() for x in dev]
    d = c.dev
    slot_t = d["slot_mapping"] if slots is None else torch.from_numpy(slots).cuda()
    say(f"[gpu] fused fp8 store+decode {what or wl.name}: S={wl.num_seqs} "
        f"G={wl.num_q_heads // wl.num_kv_heads} d={wl.head_dim} P={partition_tokens or 'auto'}")
    B.pkv_store_fp8(d["k_new"], d["v_new"], slot_t, *dev)
    out_sep = torch.empty_like(d["q"])
    B.pkv_decode_attn_fp8(d["q"], *dev, d["block_tables"], d["context_lens"], wl.scale, out_sep,
                          max_context_len=wl.max_context_len, partition_tokens=partition_tokens)
    out = torch.empty_like(d["q"])
    B.pkv_store_decode_attn_fp8(d["k_new"], d["v_new"], slot_t, d["q"], *dev2,
                                d["block_tables"], d["context_lens"], wl.scale, out,
                                max_context_len=wl.max_context_len,
                                partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    for a, b, name in zip(dev2, dev, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(a.cpu().numpy().view(np.uint8), b.cpu().numpy().view(np.uint8)), \
            f"fused store differs ({name})"
    assert np.array_equal(bits(out), bits(out_sep)), "fused attention differs"
    return c, host, dev2, out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
@pytest.mark.parametrize("part", [16, 64, 0, -1, -3])
def test_fused_store_decode_fp8_matches_separate(d, g, part):
    lens = [1, 15, 16, 17, 63, 64, 65, 129, 0, 300]
    wl = W.make_decode(f"fused_fp8_d{d}_g{g}", lens, 2 * g, 2, d, 500 + d + g, spare_blocks=2)
    c, host, dev, out = fused_fp8_vs_separate(wl, part)
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    for got, ref, name in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), name
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, f"fused fp8 store+decode d{d} g{g} P{part}", plus_floor=True)


def test_fused_store_decode_fp8_skips_and_strays():
    """slot -1 stores nothing (the last position keeps its cached codes); a
    slot in an unreferenced block is stored but not attended; a sequence with
    no context only stores; a slot outside the pool is not written."""
    wl = W.make_decode("fused_fp8_edges", [20, 33, 7, 0, 40, 9], 8, 2, 128, 64, spare_blocks=2)
    spare = sorted(set(range(wl.num_blocks)) - set(wl.used_blocks().tolist()))
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    slots[2] = spare[0] * 16 + 3
    slots[3] = spare[1] * 16 + 0
    slots[5] = wl.num_blocks * 16 + 1
    # no NaN fill: the last positions of sequences 1 and 2 are not stored in
    # this step, so they must already hold a token (random codes here)
    c, host, dev, out = fused_fp8_vs_separate(wl, 0, slots=slots, what="edges", nan_fill=False)
    assert np.all(to_f64(out)[3] == 0.0)
    slots_oracle = slots.copy()
    slots_oracle[5] = -1  # the oracle rejects out-of-pool slots
    orc().store_fp8(c.h["k_new"], c.h["v_new"], slots_oracle, *host)
    for got, ref, name in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), name
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, "fused fp8 store+decode edges", plus_floor=True)


def test_decode_fp8_mistral_full_size():
    """32 x 4096 GQA over FP8 pools of random codes, in the benchmark's launch
    configuration: the oracle quantizes the 32 new tokens into host copies of
    the pools taken before the GPU store, the pools after the store must equal
    them byte for byte, and every sequence is compared."""
    wl = W.mistral_gqa(num_layers=1)
    say("[gpu] decode fp8 full size (random codes), oracle on every sequence")
    c = Case(wl, nan_fill=False)
    host, dev = fp8_case(wl)
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], c.dev["slot_mapping"], *dev)
    out = torch.empty_like(c.dev["q"])
    B.pkv_decode_attn_fp8(c.dev["q"], *dev, c.dev["block_tables"], c.dev["context_lens"],
                          wl.scale, out, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    for got, ref, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), what
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, "decode fp8 full size")


def fp8_quantized_step(wl, partition_tokens=0, fused=True):
    """A decode step over an FP8 cache filled from N(0,1) data: every cached
    token quantized by the FP8 store (GPU and oracle separately, compared),
    then the step's new tokens stored and attended -- fused or as two
    launches -- against the oracle's store_fp8 + decode_fp8."""
    c = Case(wl)
    host, dev = fp8_quantized_pools(wl, c.dev["k_caches"][0], c.dev["v_caches"][0])
    d = c.dev
    out = torch.empty_like(d["q"])
    if fused:
        B.pkv_store_decode_attn_fp8(d["k_new"], d["v_new"], d["slot_mapping"], d["q"], *dev,
                                    d["block_tables"], d["context_lens"], wl.scale, out,
                                    max_context_len=wl.max_context_len,
                                    partition_tokens=partition_tokens)
    else:
        B.pkv_store_fp8(d["k_new"], d["v_new"], d["slot_mapping"], *dev)
        B.pkv_decode_attn_fp8(d["q"], *dev, d["block_tables"], d["context_lens"], wl.scale, out,
                              max_context_len=wl.max_context_len,
                              partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    for got, ref, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), what
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    return out, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
@pytest.mark.parametrize("part", [16, 64, 0, -1, -3])
def test_fp8_quantized_normal_data(d, g, part):
    """Edge lengths over an FP8 cache holding N(0,1) data quantized by the
    store, fused store + decode, held to max 1e-2 / mean 1e-3 with no
    allowance."""
    lens = [1, 2, 15, 16, 17, 63, 64, 65, 129, 0, 300, 1000]
    wl = W.make_decode(f"fp8q_d{d}_g{g}", lens, 2 * g, 2, d, 800 + d + g, spare_blocks=2)
    say(f"[gpu] fp8 step on quantized N(0,1) data d={d} G={g} P={part or 'auto'}")
    out, ref = fp8_quantized_step(wl, part)
    compare(out, ref, f"fp8 quantized d{d} g{g} P{part}")


@pytest.mark.parametrize("d,g", [(128, 4), (64, 8)])
@pytest.mark.parametrize("part", [0, 1024, 2048, -4])
def test_fp8_quantized_long_contexts(d, g, part):
    """Contexts past the single-pass range (up to 20,000 tokens) over store-
    quantized N(0,1) data: the matrix-core path's LDS ring over hundreds of
    blocks per wave and its lazy maximum over long spans, in the split-KV
    kernel (automatic, 1024 and 2048 tokens per partition) and in the
    single-pass kernel forced to 4 waves; plain bound."""
    lens = [20000, 129, 8200, 4097, 17, 12345]
    wl = W.make_decode(f"fp8q_long_d{d}_g{g}", lens, 2 * g, 2, d, 820 + d + g, spare_blocks=1)
    say(f"[gpu] fp8 long contexts d={d} G={g} P={part or 'auto'}")
    out, ref = fp8_quantized_step(wl, part)
    compare(out, ref, f"fp8 long contexts d{d} g{g} P{part}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_fp8_quantized_scale_edges(scale):
    """Zero, negative and sharpened scales on the matrix-core path (contexts
    above 128 keys): a sharpened softmax raises the reference maximum many
    times mid-stream.  A near-one-hot row returns one cached V row whose bf16
    rounding alone can exceed 1e-2, so the per-element allowance of the
    bf16 scale-edge tests applies."""
    wl = W.make_decode("fp8q_scale", [4000, 300, 129, 1000, 1], 8, 2, 128, 830, scale=scale,
                       spare_blocks=1)
    say(f"[gpu] fp8 quantized data, scale {scale}")
    out, ref = fp8_quantized_step(wl)
    compare(out, ref, f"fp8 quantized scale {scale}", plus_floor=True)


def test_fp8_quantized_separate_launches():
    """The same over two launches (pkv_store_fp8, then pkv_decode_attn_fp8)."""
    wl = W.make_decode("fp8q_sep", [1, 5, 37, 200, 64, 2048], 8, 2, 128, 811, spare_blocks=1)
    say("[gpu] fp8 store then decode on quantized N(0,1) data")
    out, ref = fp8_quantized_step(wl, fused=False)
    compare(out, ref, "fp8 quantized separate")


def test_fp8_quantized_mistral_full_size():
    """The benchmark's FP8 step: 32 x 4096 GQA, 131,040 cached tokens
    quantized by the store on both sides (compared byte for byte), then the
    fused store + decode launch; every sequence at the plain bound."""
    wl = W.mistral_gqa(num_layers=1)
    say("[gpu] fp8 fused step full size on quantized N(0,1) data, oracle on every sequence")
    out, ref = fp8_quantized_step(wl)
    compare(out, ref, "fp8 quantized full size")


def test_read_probe_reads_only():
    """The bench's read probe streams a buffer and changes nothing but, at
    most, the first word of its sink."""
    buf = torch.arange(1 << 20, dtype=torch.int32, device="cuda")  # 4 MiB
    before = buf.clone()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    B.pkv_read_probe(buf, sink)
    B.pkv_read_probe(buf[:4], sink)  # one 16-byte chunk
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    assert int(sink[1:].abs().sum()) == 0
