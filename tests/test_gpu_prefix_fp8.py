"""Decode with shared prefixes over an FP8 cache (pkv_decode_attn_prefix_fp8)
against the oracle's FP8 decode: the result must be plain decode attention
over each sequence's whole dequantized context, however the batch is grouped.

Caches of store-quantized N(0,1) data (GPU pools by pkv_store_fp8, host pools
by the oracle's store, compared bit for bit) are held to the plain bound; the
full-size batch uses uniformly random codes, which takes the output's own bf16
rounding on top of the bound."""
import numpy as np
import pytest
import torch

from gpu_cases import Case, compare, fp8_quantized_pools, orc, random_code_pools, say
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def run_prefix_fp8(c, dev, starts, plens, max_group_size, partition_tokens=0):
    d, wl = c.dev, c.wl
    out = torch.full_like(d["q"], float("nan"))
    B.pkv_decode_attn_prefix_fp8(d["q"], *dev, d["block_tables"], d["context_lens"], wl.scale, out,
                                 torch.tensor(np.asarray(starts), dtype=torch.int32, device="cuda"),
                                 torch.tensor(np.asarray(plens), dtype=torch.int32, device="cuda"),
                                 int(max_group_size), max_context_len=int(wl.context_lens.max()),
                                 partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out


def stored_quantized(c):
    """FP8 pools of store-quantized N(0,1) data with this step's new tokens
    stored on both sides (codes and scales compared).  Returns (host, GPU)."""
    wl = c.wl
    host, dev = fp8_quantized_pools(wl, c.dev["k_caches"][0], c.dev["v_caches"][0])
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], c.dev["slot_mapping"], *dev)
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    torch.cuda.synchronize()
    for got, ref, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), what
    return host, dev


def grouped_case(d, g, seed):
    """Three groups that truly share 320 tokens, then two sequences that share
    nothing, one of them empty; group 1 has 36 members (more than one prefix
    tile's sequences for G = 4 and 8)."""
    tails0 = [1, 17, 100, 250, 16]
    tails1 = [(7 * i) % 90 + 1 for i in range(36)]
    tails2 = [64, 3]
    ctx = [320 + t for t in tails0 + tails1 + tails2] + [45, 0]
    groups = [list(range(0, 5)), list(range(5, 41)), list(range(41, 43))]
    wl = W.make_decode(f"prefix8_d{d}_g{g}", ctx, 2 * g, 2, d, seed, prefix_groups=groups,
                       prefix_tokens=320, spare_blocks=2)
    return wl, [0, 5, 41, 43]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 4, 8])
def test_prefix_fp8_matches_oracle(d, g):
    """Declared prefixes of 320, 100 (rounded down to 96) and 48 tokens."""
    wl, starts = grouped_case(d, g, 1300 + d + g)
    c = Case(wl)
    say(f"[gpu] fp8 prefix decode d={d} G={g}")
    host, dev = stored_quantized(c)
    out = run_prefix_fp8(c, dev, starts, [320, 100, 48], 36, partition_tokens=32)
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, f"fp8 prefix decode d{d} g{g}")


@pytest.mark.parametrize("ptok", [16, 0])
def test_prefix_fp8_found_groups(ptok):
    """Groups as pkv_prefix_groups finds them (the true 320-token prefix),
    tails in 16-token runs and the automatic choice."""
    wl, _ = grouped_case(128, 4, 1350 + ptok)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    c = Case(wl)
    say(f"[gpu] fp8 prefix decode, found groups, partition_tokens {ptok}")
    host, dev = stored_quantized(c)
    out = run_prefix_fp8(c, dev, starts, plens, mg, partition_tokens=ptok)
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, f"fp8 prefix decode found groups ptok {ptok}")


def test_prefix_fp8_cont_batch_full_size():
    """256 sequences in 8 groups of 32 sharing a 2048-token prefix, over an
    FP8 cache of random codes: every sequence against the oracle."""
    wl = W.cont_batch()
    say("[gpu] fp8 prefix decode cont_batch full size")
    c = Case(wl)
    host, dev = random_code_pools(wl)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    assert list(plens) == [2048] * 8
    out = run_prefix_fp8(c, dev, starts, plens, mg)
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, "fp8 prefix decode cont_batch", plus_floor=True)


@pytest.mark.parametrize("d,nseq", [(64, 130), (128, 400)])
def test_prefix_fp8_large_batch(d, nseq):
    """A batch whose list of tail offsets leaves no room in LDS for the
    matrix-core tails (more than 123 sequences at d 64, 379 at d 128): every
    tail runs the VALU path.  Groups of 16 share 64 tokens; tails of 1 to 150
    tokens; a few sequences stand alone."""
    rng = np.random.default_rng(1400 + d)
    tails = [int(x) for x in rng.integers(1, 151, size=nseq)]
    ngroups = (nseq - 4) // 16
    groups = [list(range(16 * k, 16 * k + 16)) for k in range(ngroups)]
    ctx = [64 + t if i < 16 * ngroups else t for i, t in enumerate(tails)]
    wl = W.make_decode(f"prefix8_big_d{d}", ctx, 8, 2, d, 1400 + d, prefix_groups=groups,
                       prefix_tokens=64, spare_blocks=2)
    c = Case(wl)
    say(f"[gpu] fp8 prefix decode, {nseq} sequences, d={d}")
    host, dev = stored_quantized(c)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    assert len(starts) >= ngroups
    out = run_prefix_fp8(c, dev, starts, plens, mg)
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, f"fp8 prefix decode {nseq} seqs d{d}")


def test_prefix_fp8_whole_context_and_no_groups():
    """A member whose context is exactly the prefix (no tail), and the same
    batch with no groups at all (every sequence split-KV only)."""
    wl, starts = grouped_case(128, 4, 1360)
    wl.context_lens[3] = 320  # member 3 of group 0 keeps only the shared tokens
    wl.slot_mapping[3] = -1   # and stores nothing
    c = Case(wl)
    say("[gpu] fp8 prefix decode: a member with no tail; then without groups")
    host, dev = stored_quantized(c)
    out = run_prefix_fp8(c, dev, starts, [320, 320, 320], 36)
    plain = run_prefix_fp8(c, dev, [0], [], 0)
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    compare(out, ref, "fp8 prefix decode, empty tail")
    compare(plain, ref, "fp8 prefix decode, no groups")


def test_prefix_fp8_workspace_reuse_deterministic():
    wl, starts = grouped_case(128, 8, 1370)
    c = Case(wl)
    host, dev = stored_quantized(c)
    need = B.pkv_decode_prefix_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                               wl.head_dim, int(wl.context_lens.max()), 32)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    say(f"[gpu] fp8 prefix decode twice on one workspace of {need} B")
    d = c.dev

    def call():
        out = torch.full_like(d["q"], float("nan"))
        B.pkv_decode_attn_prefix_fp8(d["q"], *dev, d["block_tables"], d["context_lens"], wl.scale,
                                     out, torch.tensor(starts, dtype=torch.int32, device="cuda"),
                                     torch.tensor([320, 320, 320], dtype=torch.int32, device="cuda"),
                                     36, max_context_len=int(wl.context_lens.max()), workspace=ws,
                                     partition_tokens=32)
        torch.cuda.synchronize()
        return out
    a, b = call(), call()
    assert np.array_equal(a.cpu().view(torch.int16).numpy(), b.cpu().view(torch.int16).numpy())


def test_prefix_fp8_precondition_rows_are_nan():
    """A declared prefix longer than a member's context, and a group larger
    than max_group_size, give NaN for exactly the rows concerned."""
    wl, starts = grouped_case(128, 4, 1380)
    c = Case(wl)
    say("[gpu] fp8 prefix decode with broken preconditions (NaN rows expected)")
    host, dev = stored_quantized(c)
    # group 2's members have contexts 384 and 323: a 336-token prefix exceeds the second
    out = run_prefix_fp8(c, dev, starts, [320, 320, 336], 32, partition_tokens=64)
    ref = orc().decode_fp8(c.h["q"], *host, wl.block_tables, wl.context_lens, wl.scale)
    got = out.float().cpu().numpy()
    assert np.all(np.isnan(got[42])), "prefix beyond the context must give NaN"
    # max_group_size 32 with G = 4 covers 32 members of group 1 (5 .. 36)
    assert np.all(np.isnan(got[37:41])), "members past max_group_size must give NaN"
    valid = [s for s in range(wl.num_seqs) if not (37 <= s <= 40 or s == 42)]
    compare(out[valid], ref[valid], "fp8 prefix decode, valid rows")
