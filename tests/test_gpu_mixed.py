"""The mixed continuous-batching step (pkv_mixed_attn) on the GPU: decode
sequences and prefill chunks in one launch, against the fp64 oracle's
prefill (a decode token is the one-new-token case, pinned equal to decode),
and bit for bit against the separate decode and prefill launches, whose
arithmetic each half of the mixed kernel shares."""
import numpy as np
import pytest
import torch

from gpu_cases import Case, bits, compact_for_oracle, compare, orc, say
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def run_mixed(c, num_decode, max_new_len=None, workspace=None, split=True):
    d, wl = c.dev, c.wl
    prefill_new = wl.new_lens[num_decode:]
    mnl = max_new_len if max_new_len is not None else int(prefill_new.max()) if len(prefill_new) else 0
    out = torch.full_like(d["q"], float("nan"))
    B.pkv_mixed_attn(d["q"], d["k_caches"][0], d["v_caches"][0], d["block_tables"],
                     d["cu_new_lens"], d["context_lens"], num_decode, wl.scale, out,
                     max_new_len=mnl, max_context_len=int(wl.context_lens.max()),
                     workspace=workspace, split=split)
    torch.cuda.synchronize()
    return out


def mixed_case(d, g, seed):
    dec_ctx = [1, 15, 16, 17, 100, 300]
    pf = [(0, 1), (0, 40), (17, 33), (100, 5), (64, 64), (0, 130)]
    cached = [x - 1 for x in dec_ctx] + [c for c, _ in pf]
    new = [1] * len(dec_ctx) + [n for _, n in pf]
    wl = W.make_prefill(f"mixed_d{d}_g{g}", cached, new, 2 * g, 2, d, seed, spare_blocks=2)
    return wl, len(dec_ctx)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_mixed_matches_oracle(d, g):
    wl, nd = mixed_case(d, g, 600 + d + g)
    c = Case(wl)
    c.gpu_store()
    say(f"[gpu] mixed step d={d} G={g}: {nd} decode + {wl.num_seqs - nd} prefill sequences")
    out = run_mixed(c, nd)
    c.oracle_store()
    compare(out, c.oracle_prefill(), f"mixed d{d} g{g}")


@pytest.mark.parametrize("g", [1, 4, 8])
def test_mixed_halves_equal_separate_launches(g):
    """Decode rows are bit-identical to pkv_decode_attn's single pass with 4
    waves; prefill rows to pkv_prefill_attn's."""
    wl, nd = mixed_case(128, g, 700 + g)
    c = Case(wl)
    c.gpu_store()
    say(f"[gpu] mixed step vs separate launches, G={g}")
    out = run_mixed(c, nd)
    d = c.dev
    dec = torch.empty((nd, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    B.pkv_decode_attn(d["q"][:nd].contiguous(), d["k_caches"][0], d["v_caches"][0],
                      d["block_tables"][:nd].contiguous(), d["context_lens"][:nd].contiguous(),
                      wl.scale, dec, max_context_len=int(wl.context_lens[:nd].max()),
                      partition_tokens=-4)
    pf = c.gpu_prefill()
    torch.cuda.synchronize()
    assert np.array_equal(bits(out[:nd]), bits(dec)), "decode rows differ from pkv_decode_attn"
    assert np.array_equal(bits(out[nd:]), bits(pf[nd:])), "prefill rows differ from pkv_prefill_attn"


def test_mixed_decode_range_irregular():
    """In the decode range a sequence with 3 new tokens is still computed in
    full and one with none writes nothing; a prefill chunk of one token is
    computed as prefill."""
    cached = [40, 20, 33, 0, 7]
    new = [1, 3, 0, 1, 1]
    wl = W.make_prefill("mixed_irregular", cached + [50, 12], new + [1, 70], 8, 2, 128, 710)
    c = Case(wl)
    c.gpu_store()
    say("[gpu] mixed step, irregular decode range")
    out = run_mixed(c, len(cached))
    c.oracle_store()
    compare(out, c.oracle_prefill(), "mixed irregular")


@pytest.mark.parametrize("which", ["all_decode", "all_prefill"])
def test_mixed_one_kind_only(which):
    if which == "all_decode":
        wl = W.make_prefill("mixed_all_decode", [3, 64, 500], [1, 1, 1], 16, 4, 128, 720)
        nd = 3
    else:
        wl = W.make_prefill("mixed_all_prefill", [0, 31, 200], [9, 33, 64], 16, 4, 64, 721)
        nd = 0
    c = Case(wl)
    c.gpu_store()
    say(f"[gpu] mixed step, {which}")
    out = run_mixed(c, nd)
    c.oracle_store()
    compare(out, c.oracle_prefill(), f"mixed {which}")


def split_case(d, g, seed):
    # few prefill chunks behind long cached contexts: the units split by key range
    cached = [4095, 1000, 17] + [3000, 2500, 40]
    new = [1, 1, 1] + [40, 70, 1]
    return W.make_prefill(f"mixed_split_d{d}_g{g}", cached, new, 2 * g, 2, d, seed, spare_blocks=2), 3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
def test_mixed_split_matches_oracle(d, g):
    wl, nd = split_case(d, g, 730 + d + g)
    mnl = int(wl.new_lens[nd:].max())
    need = B.pkv_mixed_workspace_bytes(wl.num_seqs, nd, mnl, int(wl.context_lens.max()),
                                       wl.num_q_heads, wl.num_kv_heads, d)
    assert need > 0, "this case should split"
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # contents do not matter
    c = Case(wl)
    c.gpu_store()
    say(f"[gpu] mixed step with split prefill units d={d} G={g}, workspace {need} B")
    out1 = run_mixed(c, nd, workspace=ws)
    out2 = run_mixed(c, nd, workspace=ws)
    whole = run_mixed(c, nd, split=False)
    assert np.array_equal(bits(out1), bits(out2)), "a second launch on the workspace differs"
    c.oracle_store()
    ref = c.oracle_prefill()
    compare(out1, ref, f"mixed split d{d} g{g}")
    compare(whole, ref, f"mixed unsplit d{d} g{g}")
    assert np.array_equal(bits(out1[:nd]), bits(whole[:nd])), "decode rows depend on the split"


def test_mixed_step_full_size():
    """The benchmark's iteration: 32 x 4096 decode + 4 chunks of 496 new
    tokens; the oracle checks every row of both kinds."""
    wl = W.mixed_step()
    nd = 32
    seqs = range(wl.num_seqs)
    say("[gpu] mixed step full size, oracle on every sequence")
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    h = compact_for_oracle(wl, t, seqs)
    dev = {k: t[k] for k in ("q", "k_new", "v_new", "slot_mapping", "block_tables",
                             "context_lens", "cu_new_lens")}
    B.pkv_store(dev["k_new"], dev["v_new"], dev["slot_mapping"], t["k_caches"][0],
                t["v_caches"][0])
    out = torch.empty_like(dev["q"])
    B.pkv_mixed_attn(dev["q"], t["k_caches"][0], t["v_caches"][0], dev["block_tables"],
                     dev["cu_new_lens"], dev["context_lens"], nd, wl.scale, out,
                     max_new_len=int(wl.new_lens[nd:].max()),
                     max_context_len=int(wl.context_lens.max()))
    torch.cuda.synchronize()
    orc().store(h["k_new"], h["v_new"], h["slots"], h["kc"], h["vc"])
    cu = np.concatenate([[0], np.cumsum(h["new_lens"])]).astype(np.int32)
    ref = orc().prefill(h["q"], h["kc"], h["vc"], h["bt"], cu, h["ctx"], wl.scale)
    rows = torch.from_numpy(h["tok"]).cuda()
    compare(out.index_select(0, rows), ref, "mixed full size")


def test_mixed_tail_full_size_split():
    """The last 64-token chunk of a 4096-token prompt beside the 32 x 4096
    decode batch: its units split by key range; the oracle checks every
    decode sequence and the chunk."""
    wl = W.mixed_tail()
    nd = 32
    seqs = range(wl.num_seqs)
    mnl, mcl = 64, int(wl.context_lens.max())
    need = B.pkv_mixed_workspace_bytes(wl.num_seqs, nd, mnl, mcl, wl.num_q_heads,
                                       wl.num_kv_heads, wl.head_dim)
    assert need > 0
    say(f"[gpu] mixed tail full size (split, workspace {need} B), oracle on every sequence")
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    h = compact_for_oracle(wl, t, seqs)
    B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][0], t["v_caches"][0])
    out = torch.empty_like(t["q"])
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    B.pkv_mixed_attn(t["q"], t["k_caches"][0], t["v_caches"][0], t["block_tables"],
                     t["cu_new_lens"], t["context_lens"], nd, wl.scale, out, max_new_len=mnl,
                     max_context_len=mcl, workspace=ws)
    torch.cuda.synchronize()
    orc().store(h["k_new"], h["v_new"], h["slots"], h["kc"], h["vc"])
    cu = np.concatenate([[0], np.cumsum(h["new_lens"])]).astype(np.int32)
    ref = orc().prefill(h["q"], h["kc"], h["vc"], h["bt"], cu, h["ctx"], wl.scale)
    compare(out.index_select(0, torch.from_numpy(h["tok"]).cuda()), ref, "mixed tail full size")


def test_mixed_prefill_only_split():
    """With no decode sequences pkv_mixed_attn is chunked prefill whose few,
    long-context chunks split by key range: the last chunks of two long
    prompts."""
    wl = W.make_prefill("prefill_tails", [3000, 1900], [32, 17], 16, 4, 128, 740, spare_blocks=1)
    need = B.pkv_mixed_workspace_bytes(2, 0, 32, int(wl.context_lens.max()), 16, 4, 128)
    assert need > 0
    c = Case(wl)
    c.gpu_store()
    say(f"[gpu] prefill-only mixed launch with split units, workspace {need} B")
    out = run_mixed(c, 0, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    c.oracle_store()
    compare(out, c.oracle_prefill(), "prefill-only split")
