"""Decode with shared prefixes (pkv_decode_attn_prefix) on the GPU, against
the fp64 oracle's decode: the result must be plain decode attention over each
sequence's whole context, however the batch is grouped."""
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


def run_prefix(c, starts, plens, max_group_size, partition_tokens=0, workspace=None):
    d, wl = c.dev, c.wl
    out = torch.full_like(d["q"], float("nan"))
    B.pkv_decode_attn_prefix(d["q"], d["k_caches"][0], d["v_caches"][0], d["block_tables"],
                             d["context_lens"], wl.scale, out,
                             torch.tensor(starts, dtype=torch.int32, device="cuda"),
                             torch.tensor(plens, dtype=torch.int32, device="cuda"),
                             max_group_size, max_context_len=int(wl.context_lens.max()),
                             workspace=workspace, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out


def grouped_case(d, g, seed):
    """Three groups that truly share 320 tokens (blocks 0..19 of their rows),
    then two sequences that share nothing, one of them empty.  Group 1 has 36
    members: more than one prefix tile's sequences for G = 4 and 8."""
    tails0 = [1, 17, 100, 250, 16]
    tails1 = [(7 * i) % 90 + 1 for i in range(36)]
    tails2 = [64, 3]
    ctx = [320 + t for t in tails0 + tails1 + tails2] + [45, 0]
    groups = [list(range(0, 5)), list(range(5, 41)), list(range(41, 43))]
    wl = W.make_decode(f"prefix_d{d}_g{g}", ctx, 2 * g, 2, d, seed, prefix_groups=groups,
                       prefix_tokens=320, spare_blocks=2)
    starts = [0, 5, 41, 43]
    return wl, starts


# declared prefixes: any whole-block length up to what the rows truly share
# (100 rounds down to 96; 48 is not a multiple of the 64-key chunk)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_prefix_matches_oracle(d, g):
    wl, starts = grouped_case(d, g, 900 + d + g)
    plens = [320, 100, 48]
    c = Case(wl)
    c.gpu_store()
    say(f"[gpu] prefix decode d={d} G={g}: groups {starts} prefixes {plens}")
    out = run_prefix(c, starts, plens, max_group_size=36, partition_tokens=32)
    c.oracle_store()
    compare(out, c.oracle_decode(), f"prefix decode d{d} g{g}")


@pytest.mark.parametrize("ptok", [16, 64, 0])
def test_prefix_partition_lengths(ptok):
    """Tails cut into 16-token partitions up to the automatic choice; groups
    as pkv_prefix_groups finds them (the true 320-token prefix)."""
    wl, _ = grouped_case(128, 4, 950 + ptok)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    assert list(starts) == [0, 5, 41, 43, 45] and list(plens) == [320, 320, 320, 0] and mg == 36
    c = Case(wl)
    c.gpu_store()
    say(f"[gpu] prefix decode, partition_tokens {ptok}")
    out = run_prefix(c, starts, plens, mg, partition_tokens=ptok)
    c.oracle_store()
    compare(out, c.oracle_decode(), f"prefix decode ptok {ptok}")


def test_prefix_whole_context_and_no_groups():
    """A member whose context is exactly the prefix (no tail), and the same
    batch with no groups at all (every sequence split-KV only)."""
    wl, starts = grouped_case(128, 4, 960)
    # member 3 of group 0 keeps only the 320 shared tokens; its store is skipped
    wl.context_lens[3] = 320
    wl.slot_mapping[3] = -1
    c = Case(wl)
    c.gpu_store()
    say("[gpu] prefix decode: a member with no tail; then without groups")
    out = run_prefix(c, starts, [320, 320, 320], 36)
    plain = run_prefix(c, [0], [], 0)
    c.oracle_store()
    ref = c.oracle_decode()
    compare(out, ref, "prefix decode, empty tail")
    compare(plain, ref, "prefix decode, no groups")


def test_prefix_workspace_reuse_deterministic():
    wl, starts = grouped_case(128, 8, 970)
    c = Case(wl)
    c.gpu_store()
    need = B.pkv_decode_prefix_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                               wl.head_dim, int(wl.context_lens.max()), 32)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    say(f"[gpu] prefix decode twice on one workspace of {need} B")
    a = run_prefix(c, starts, [320, 320, 320], 36, 32, ws)
    b = run_prefix(c, starts, [320, 320, 320], 36, 32, ws)
    assert np.array_equal(bits(a), bits(b))


def test_prefix_precondition_rows_are_nan():
    """A declared prefix longer than a member's context, and a group larger
    than max_group_size, give NaN for exactly the rows concerned."""
    wl, starts = grouped_case(128, 4, 980)
    c = Case(wl)
    c.gpu_store()
    say("[gpu] prefix decode with broken preconditions (NaN rows expected)")
    # group 2's members have contexts 384 and 323: a 336-token prefix exceeds the
    # second; the first reads the prefix through its own row, so it stays exact
    out = run_prefix(c, starts, [320, 320, 336], 32, partition_tokens=64)
    c.oracle_store()
    ref = c.oracle_decode()
    got = out.float().cpu().numpy()
    assert np.all(np.isnan(got[42])), "prefix beyond the context must give NaN"
    # max_group_size 32 with G = 4 covers 32 members of group 1 (5 .. 36)
    assert np.all(np.isnan(got[37:41])), "members past max_group_size must give NaN"
    valid = [s for s in range(wl.num_seqs) if not (37 <= s <= 40 or s == 42)]
    compare(out[valid], ref[valid], "prefix decode, valid rows")


def run_prefix_full(wl, what):
    seqs = range(wl.num_seqs)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    say(f"[gpu] {what}: S={wl.num_seqs} max_ctx={wl.max_context_len}; groups "
        f"{list(starts)} prefixes {list(plens)}; oracle on every sequence")
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    h = compact_for_oracle(wl, t, seqs)
    B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][0], t["v_caches"][0])
    out = torch.empty_like(t["q"])
    B.pkv_decode_attn_prefix(t["q"], t["k_caches"][0], t["v_caches"][0], t["block_tables"],
                             t["context_lens"], wl.scale, out,
                             torch.from_numpy(starts).cuda(), torch.from_numpy(plens).cuda(), mg,
                             max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    orc().store(h["k_new"], h["v_new"], h["slots"], h["kc"], h["vc"])
    ref = orc().decode(h["q"], h["kc"], h["vc"], h["bt"], h["ctx"], wl.scale)
    compare(out, ref, what)
    return starts, plens


def test_prefix_cont_batch_full_size():
    """256 sequences in 8 groups of 32 sharing a 2048-token prefix."""
    wl = W.cont_batch()
    starts, plens = run_prefix_full(wl, "prefix decode cont_batch")
    assert list(plens) == [2048] * 8


def test_prefix_cont_batch_reading_b_sorted():
    """The other reading of the mix (only contexts over 2048 share), with each
    group's sharers listed next to each other."""
    wl = W.cont_batch(prefix_reading="B")
    bt = wl.block_tables
    first = bt[:, 0]
    order = np.argsort(first, kind="stable")
    wl.block_tables = np.ascontiguousarray(bt[order])
    wl.context_lens = np.ascontiguousarray(wl.context_lens[order])
    wl.slot_mapping = np.ascontiguousarray(wl.slot_mapping[order])
    starts, plens = run_prefix_full(wl, "prefix decode cont_batch B")
    assert (plens > 0).any()
