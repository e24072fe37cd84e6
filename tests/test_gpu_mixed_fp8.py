"""The mixed continuous-batching step over an FP8 cache (pkv_mixed_attn_fp8):
against the oracle's FP8 prefill over the whole batch (a decode token is the
one-new-token case), and bit for bit against the separate FP8 decode and FP8
prefill launches whose arithmetic each half of the mixed kernel shares.

Caches of store-quantized N(0,1) data (GPU pools by pkv_store_fp8, host pools
by the oracle's store, compared bit for bit) are held to the plain bound; the
full-size step uses uniformly random codes, which takes the output's own bf16
rounding on top of the bound."""
import numpy as np
import pytest
import torch

from gpu_cases import (Case, bits, compare, fp8_quantized_pools, orc, random_code_pools, say)
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def run_mixed_fp8(c, dev, num_decode, workspace=None, split=True):
    d, wl = c.dev, c.wl
    prefill_new = wl.new_lens[num_decode:]
    mnl = int(prefill_new.max()) if len(prefill_new) else 0
    out = torch.full_like(d["q"], float("nan"))
    B.pkv_mixed_attn_fp8(d["q"], *dev, d["block_tables"], d["cu_new_lens"], d["context_lens"],
                         num_decode, wl.scale, out, max_new_len=mnl,
                         max_context_len=int(wl.context_lens.max()), workspace=workspace,
                         split=split)
    torch.cuda.synchronize()
    return out


def quantized_pools_after_store(c):
    """FP8 pools of store-quantized N(0,1) data: the cached tokens quantized on
    both sides, then the step's new tokens stored by pkv_store_fp8 and the
    oracle's store_fp8; codes and scales compared.  Returns (host, GPU)."""
    wl = c.wl
    host, dev = fp8_quantized_pools(wl, c.dev["k_caches"][0], c.dev["v_caches"][0])
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], c.dev["slot_mapping"], *dev)
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    torch.cuda.synchronize()
    for got, ref, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), what
    return host, dev


def oracle(c, host):
    wl = c.wl
    return orc().prefill_fp8(c.h["q"], *host, wl.block_tables, wl.cu_new_lens, wl.context_lens,
                             wl.scale)


def mixed_case(d, g, seed):
    dec_ctx = [1, 15, 16, 17, 100, 300]
    pf = [(0, 1), (0, 40), (17, 33), (100, 5), (64, 64), (0, 130)]
    cached = [x - 1 for x in dec_ctx] + [c for c, _ in pf]
    new = [1] * len(dec_ctx) + [n for _, n in pf]
    wl = W.make_prefill(f"mixed8_d{d}_g{g}", cached, new, 2 * g, 2, d, seed, spare_blocks=2)
    return wl, len(dec_ctx)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
def test_mixed_fp8_matches_oracle(d, g):
    wl, nd = mixed_case(d, g, 1000 + d + g)
    c = Case(wl)
    say(f"[gpu] fp8 mixed step d={d} G={g}: {nd} decode + {wl.num_seqs - nd} prefill sequences")
    host, dev = quantized_pools_after_store(c)
    out = run_mixed_fp8(c, dev, nd)
    compare(out, oracle(c, host), f"fp8 mixed d{d} g{g}")


@pytest.mark.parametrize("g", [1, 4, 8])
def test_mixed_fp8_halves_equal_separate_launches(g):
    """Decode rows are bit-identical to pkv_decode_attn_fp8's single pass with
    4 waves (contexts of 300 and 1000 take its matrix-core path, the rest the
    short-context one); prefill rows to pkv_prefill_attn_fp8's."""
    dec_ctx = [1, 17, 100, 129, 300, 1000]
    pf = [(0, 40), (17, 33), (200, 64)]
    wl = W.make_prefill(f"mixed8_sep_g{g}", [x - 1 for x in dec_ctx] + [c for c, _ in pf],
                        [1] * len(dec_ctx) + [n for _, n in pf], 4 * g, 4, 128, 1100 + g,
                        spare_blocks=1)
    nd = len(dec_ctx)
    c = Case(wl)
    say(f"[gpu] fp8 mixed step vs separate launches, G={g}")
    host, dev = quantized_pools_after_store(c)
    out = run_mixed_fp8(c, dev, nd)
    d = c.dev
    dec = torch.empty((nd, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    B.pkv_decode_attn_fp8(d["q"][:nd].contiguous(), *dev, d["block_tables"][:nd].contiguous(),
                          d["context_lens"][:nd].contiguous(), wl.scale, dec,
                          max_context_len=int(wl.context_lens[:nd].max()), partition_tokens=-4)
    pf_out = torch.empty_like(d["q"])
    B.pkv_prefill_attn_fp8(d["q"], *dev, d["block_tables"], d["cu_new_lens"], d["context_lens"],
                           wl.scale, pf_out, max_new_len=wl.max_new_len,
                           max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out[:nd]), bits(dec)), "decode rows differ from pkv_decode_attn_fp8"
    assert np.array_equal(bits(out[nd:]), bits(pf_out[nd:])), \
        "prefill rows differ from pkv_prefill_attn_fp8"
    compare(out, oracle(c, host), f"fp8 mixed vs separate g{g}")


@pytest.mark.parametrize("g", [1, 4])
def test_mixed_fp8_split_matches_oracle(g):
    """Few prefill chunks behind long cached contexts, split by key range over
    a workspace: twice on the same workspace (bit-identical), unsplit, and the
    oracle."""
    cached = [4095, 1000, 17] + [3000, 2500, 40]
    new = [1, 1, 1] + [40, 70, 1]
    wl = W.make_prefill(f"mixed8_split_g{g}", cached, new, 2 * g, 2, 128, 1200 + g,
                        spare_blocks=2)
    nd = 3
    need = B.pkv_mixed_workspace_bytes(wl.num_seqs, nd, int(wl.new_lens[nd:].max()),
                                       int(wl.context_lens.max()), wl.num_q_heads,
                                       wl.num_kv_heads, wl.head_dim)
    assert need > 0, "this case should split"
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    c = Case(wl)
    say(f"[gpu] fp8 mixed step with split prefill units G={g}, workspace {need} B")
    host, dev = quantized_pools_after_store(c)
    out1 = run_mixed_fp8(c, dev, nd, workspace=ws)
    out2 = run_mixed_fp8(c, dev, nd, workspace=ws)
    whole = run_mixed_fp8(c, dev, nd, split=False)
    assert np.array_equal(bits(out1), bits(out2)), "a second launch on the workspace differs"
    assert np.array_equal(bits(out1[:nd]), bits(whole[:nd])), "decode rows depend on the split"
    ref = oracle(c, host)
    compare(out1, ref, f"fp8 mixed split g{g}")
    compare(whole, ref, f"fp8 mixed unsplit g{g}")


def test_mixed_fp8_step_full_size():
    """The benchmark's iteration (32 x 4096 decode + 4 chunks of 496 new
    tokens) over an FP8 cache of random codes: every row against the oracle."""
    wl = W.mixed_step()
    nd = 32
    say("[gpu] fp8 mixed step full size, oracle on every row")
    c = Case(wl)
    host, dev = random_code_pools(wl)
    out = run_mixed_fp8(c, dev, nd)
    compare(out, oracle(c, host), "fp8 mixed full size", plus_floor=True)


@pytest.mark.parametrize("which", ["all_decode", "all_prefill"])
def test_mixed_fp8_one_kind_only(which):
    """Every sequence one kind: all decode (one past 128 keys, so both decode
    paths run) or all prefill."""
    if which == "all_decode":
        wl = W.make_prefill("mixed8_all_decode", [3, 64, 500], [1, 1, 1], 16, 4, 128, 1720)
        nd = 3
    else:
        wl = W.make_prefill("mixed8_all_prefill", [0, 31, 200], [9, 33, 64], 16, 4, 64, 1721)
        nd = 0
    c = Case(wl)
    say(f"[gpu] fp8 mixed step, {which}")
    host, dev = quantized_pools_after_store(c)
    out = run_mixed_fp8(c, dev, nd)
    compare(out, oracle(c, host), f"fp8 mixed {which}")


def test_mixed_fp8_decode_range_irregular():
    """In the decode range a sequence with 3 new tokens is still computed in
    full and one with none writes nothing; a prefill chunk of one token is
    computed as prefill."""
    cached = [40, 20, 33, 0, 7]
    new = [1, 3, 0, 1, 1]
    wl = W.make_prefill("mixed8_irregular", cached + [50, 12], new + [1, 70], 8, 2, 128, 1710)
    c = Case(wl)
    say("[gpu] fp8 mixed step, irregular decode range")
    host, dev = quantized_pools_after_store(c)
    out = run_mixed_fp8(c, dev, len(cached))
    compare(out, oracle(c, host), "fp8 mixed irregular")
