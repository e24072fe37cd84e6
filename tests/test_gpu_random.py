"""Seeded random shapes through every attention entry, over bf16 and FP8
caches, against the fp64 oracle: batch sizes, context lengths (including 0, 1,
block edges and long tails), head dims, group sizes, work splits and prefix
groupings drawn from a fixed seed per case, so a failure names a reproducible
case.  FP8 caches hold N(0,1) data quantized by the store on both sides (codes
and scales compared bit for bit), held to the plain bound."""
import numpy as np
import pytest
import torch

from gpu_cases import Case, compare, fp8_quantized_pools, orc, say
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def draw_lengths(rng, n, hi):
    """A mix of edge lengths and random ones."""
    edge = [0, 1, 15, 16, 17, 63, 64, 65, hi]
    return [int(rng.choice(edge)) if rng.random() < 0.35 else int(rng.integers(1, hi + 1))
            for _ in range(n)]


def heads(rng):
    g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    return g * hkv, hkv, d


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    rng = np.random.default_rng(1000 + seed)
    hq, hkv, d = heads(rng)
    ctx = draw_lengths(rng, int(rng.integers(1, 24)), int(rng.choice([200, 1500])))
    wl = W.make_decode(f"rand_dec_{seed}", ctx, hq, hkv, d, 1100 + seed, spare_blocks=2)
    part = int(rng.choice([0, 16, 64, 256, -1, -4, -8]))
    say(f"[gpu] random decode seed {seed}: {hq}/{hkv} heads, d {d}, ctx {ctx}, split {part}")
    c = Case(wl)
    c.gpu_store()
    out = c.gpu_decode(partition_tokens=part, max_context_len=max(1, max(ctx)))
    torch.cuda.synchronize()
    c.oracle_store()
    compare(out, c.oracle_decode(), f"random decode {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_prefill_and_mixed(seed):
    rng = np.random.default_rng(2000 + seed)
    hq, hkv, d = heads(rng)
    n = int(rng.integers(1, 7))
    cached = draw_lengths(rng, n, 700)
    new = [max(1, x) for x in draw_lengths(rng, n, 150)]
    nd = int(rng.integers(0, 5))  # leading decode sequences for the mixed step
    cached = [int(rng.integers(0, 900)) for _ in range(nd)] + cached
    new = [1] * nd + new
    wl = W.make_prefill(f"rand_pf_{seed}", cached, new, hq, hkv, d, 2100 + seed, spare_blocks=2)
    say(f"[gpu] random prefill/mixed seed {seed}: {hq}/{hkv} heads, d {d}, cached {cached}, "
        f"new {new}, decode range {nd}")
    c = Case(wl)
    c.gpu_store()
    d_ = c.dev
    mnl = int(wl.new_lens[nd:].max()) if nd < wl.num_seqs else 0
    out_mixed = torch.empty_like(d_["q"])
    B.pkv_mixed_attn(d_["q"], d_["k_caches"][0], d_["v_caches"][0], d_["block_tables"],
                     d_["cu_new_lens"], d_["context_lens"], nd, wl.scale, out_mixed,
                     max_new_len=mnl, max_context_len=int(wl.context_lens.max()))
    out_pf = c.gpu_prefill()
    torch.cuda.synchronize()
    c.oracle_store()
    ref = c.oracle_prefill()
    compare(out_pf, ref, f"random prefill {seed}")
    compare(out_mixed, ref, f"random mixed {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_shared_prefix(seed):
    rng = np.random.default_rng(3000 + seed)
    hq, hkv, d = heads(rng)
    pblocks = int(rng.integers(1, 40))
    prefix = 16 * pblocks
    sizes = [int(rng.integers(1, 20)) for _ in range(int(rng.integers(1, 4)))]
    groups, ctx, s = [], [], 0
    for n in sizes:
        groups.append(list(range(s, s + n)))
        ctx += [prefix + int(rng.integers(1, 300)) for _ in range(n)]
        s += n
    ctx += [int(rng.integers(0, 400)) for _ in range(int(rng.integers(0, 3)))]  # ungrouped
    wl = W.make_decode(f"rand_prefix_{seed}", ctx, hq, hkv, d, 3100 + seed, prefix_groups=groups,
                       prefix_tokens=prefix, spare_blocks=2)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens,
                                            int(rng.choice([16, 64])))
    part = int(rng.choice([0, 16, 48, 128]))
    say(f"[gpu] random shared prefix seed {seed}: {hq}/{hkv} heads, d {d}, groups {starts.tolist()} "
        f"prefixes {plens.tolist()}, split {part}")
    c = Case(wl)
    c.gpu_store()
    out = torch.full_like(c.dev["q"], float("nan"))
    B.pkv_decode_attn_prefix(c.dev["q"], c.dev["k_caches"][0], c.dev["v_caches"][0],
                             c.dev["block_tables"], c.dev["context_lens"], wl.scale, out,
                             torch.from_numpy(starts).cuda(), torch.from_numpy(plens).cuda(), mg,
                             max_context_len=int(wl.context_lens.max()), partition_tokens=part)
    torch.cuda.synchronize()
    c.oracle_store()
    compare(out, c.oracle_decode(), f"random shared prefix {seed}")


def fp8_step(c):
    """FP8 pools of this case's cached tokens plus its new tokens, stored by
    pkv_store_fp8 (GPU) and the oracle's store_fp8 (host) and compared.
    Returns (host pools, GPU pools)."""
    wl = c.wl
    host, dev = fp8_quantized_pools(wl, c.dev["k_caches"][0], c.dev["v_caches"][0])
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], c.dev["slot_mapping"], *dev)
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    torch.cuda.synchronize()
    for got, ref, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), what
    return host, dev


@pytest.mark.parametrize("seed", range(6))
def test_random_fp8_decode(seed):
    rng = np.random.default_rng(4000 + seed)
    hq, hkv, d = heads(rng)
    ctx = draw_lengths(rng, int(rng.integers(1, 24)), int(rng.choice([200, 1500])))
    wl = W.make_decode(f"rand_dec8_{seed}", ctx, hq, hkv, d, 4100 + seed, spare_blocks=2)
    part = int(rng.choice([0, 16, 64, 256, -1, -4, -8]))
    say(f"[gpu] random fp8 decode seed {seed}: {hq}/{hkv} heads, d {d}, ctx {ctx}, split {part}")
    c = Case(wl)
    host, dev = fp8_step(c)
    out = torch.empty_like(c.dev["q"])
    B.pkv_decode_attn_fp8(c.dev["q"], *dev, c.dev["block_tables"], c.dev["context_lens"], wl.scale,
                          out, max_context_len=max(1, max(ctx)), partition_tokens=part)
    torch.cuda.synchronize()
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, f"random fp8 decode {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_fp8_prefill_and_mixed(seed):
    rng = np.random.default_rng(5000 + seed)
    hq, hkv, d = heads(rng)
    n = int(rng.integers(1, 7))
    cached = draw_lengths(rng, n, 700)
    new = [max(1, x) for x in draw_lengths(rng, n, 150)]
    nd = int(rng.integers(0, 5))
    cached = [int(rng.integers(0, 900)) for _ in range(nd)] + cached
    new = [1] * nd + new
    wl = W.make_prefill(f"rand_pf8_{seed}", cached, new, hq, hkv, d, 5100 + seed, spare_blocks=2)
    say(f"[gpu] random fp8 prefill/mixed seed {seed}: {hq}/{hkv} heads, d {d}, cached {cached}, "
        f"new {new}, decode range {nd}")
    c = Case(wl)
    host, dev = fp8_step(c)
    d_ = c.dev
    mnl = int(wl.new_lens[nd:].max()) if nd < wl.num_seqs else 0
    mcl = int(wl.context_lens.max())
    out_pf = torch.empty_like(d_["q"])
    B.pkv_prefill_attn_fp8(d_["q"], *dev, d_["block_tables"], d_["cu_new_lens"], d_["context_lens"],
                           wl.scale, out_pf, max_new_len=wl.max_new_len, max_context_len=mcl)
    out_mixed = torch.empty_like(d_["q"])
    need = B.pkv_mixed_workspace_bytes(wl.num_seqs, nd, mnl, mcl, hq, hkv, d)
    ws = torch.empty(max(16, need), dtype=torch.uint8, device="cuda")
    B.pkv_mixed_attn_fp8(d_["q"], *dev, d_["block_tables"], d_["cu_new_lens"], d_["context_lens"], nd,
                         wl.scale, out_mixed, max_new_len=mnl, max_context_len=mcl, workspace=ws)
    torch.cuda.synchronize()
    ref = orc().prefill_fp8(c.h["q"], *host, wl.block_tables, wl.cu_new_lens, wl.context_lens,
                            wl.scale)
    compare(out_pf, ref, f"random fp8 prefill {seed}")
    compare(out_mixed, ref, f"random fp8 mixed {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_fp8_shared_prefix(seed):
    rng = np.random.default_rng(6000 + seed)
    hq, hkv, d = heads(rng)
    prefix = 16 * int(rng.integers(1, 40))
    sizes = [int(rng.integers(1, 20)) for _ in range(int(rng.integers(1, 4)))]
    groups, ctx, s = [], [], 0
    for n in sizes:
        groups.append(list(range(s, s + n)))
        ctx += [prefix + int(rng.integers(1, 300)) for _ in range(n)]
        s += n
    ctx += [int(rng.integers(0, 400)) for _ in range(int(rng.integers(0, 3)))]  # ungrouped
    wl = W.make_decode(f"rand_prefix8_{seed}", ctx, hq, hkv, d, 6100 + seed, prefix_groups=groups,
                       prefix_tokens=prefix, spare_blocks=2)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens,
                                            int(rng.choice([16, 64])))
    part = int(rng.choice([0, 16, 48, 128]))
    say(f"[gpu] random fp8 shared prefix seed {seed}: {hq}/{hkv} heads, d {d}, groups "
        f"{starts.tolist()} prefixes {plens.tolist()}, split {part}")
    c = Case(wl)
    host, dev = fp8_step(c)
    out = torch.full_like(c.dev["q"], float("nan"))
    B.pkv_decode_attn_prefix_fp8(c.dev["q"], *dev, c.dev["block_tables"], c.dev["context_lens"],
                                 wl.scale, out, torch.from_numpy(starts).cuda(),
                                 torch.from_numpy(plens).cuda(), mg,
                                 max_context_len=int(wl.context_lens.max()), partition_tokens=part)
    torch.cuda.synchronize()
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, f"random fp8 shared prefix {seed}")

