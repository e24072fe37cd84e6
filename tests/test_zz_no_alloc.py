"""pkv_decode_attn_noalloc, the decode entry point that allocates nothing: its
split-KV partials live in the library's own per-GPU scratch array instead of a
caller's workspace.  Checked against pkv_decode_attn with a workspace (same
kernels, so bit-identical) and against the fp64 oracle, on consecutive calls
that reuse the scratch, the second with a smaller input."""
import numpy as np
import pytest
import torch

from gpu_cases import Case, bits, compare, say
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def noalloc_vs_workspace(wl, part):
    c = Case(wl)
    c.gpu_store()
    d = c.dev
    p = part or B.pkv_decode_partition_tokens(wl.num_seqs, wl.num_kv_heads, wl.max_context_len)
    need = B.pkv_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.head_dim,
                                        wl.max_context_len, p)
    say(f"[gpu] noalloc decode {wl.name}: S={wl.num_seqs} max_ctx={wl.max_context_len} "
        f"P={p} partials {need} B of {B.pkv_decode_noalloc_max_bytes()} B")
    assert need <= B.pkv_decode_noalloc_max_bytes()
    ref = torch.empty_like(d["q"])
    B.pkv_decode_attn(d["q"], d["k_caches"][0], d["v_caches"][0], d["block_tables"],
                      d["context_lens"], wl.scale, ref, max_context_len=wl.max_context_len,
                      partition_tokens=part)
    out = torch.full_like(d["q"], float("nan"))
    B.pkv_decode_attn_noalloc(d["q"], d["k_caches"][0], d["v_caches"][0], d["block_tables"],
                              d["context_lens"], wl.scale, out,
                              max_context_len=wl.max_context_len, partition_tokens=part)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref)), "noalloc output differs from pkv_decode_attn"
    c.oracle_store()
    compare(out, c.oracle_decode(), f"noalloc decode {wl.name} P={p}")
    return need


def test_noalloc_two_calls_second_smaller():
    """A large split (many partials in the scratch), then a smaller one that
    reuses the same scratch with fewer rows and partitions."""
    big = W.make_decode("noalloc_big", np.random.default_rng(901).integers(1, 2049, 48).tolist(),
                        32, 8, 128, 902)
    need_big = noalloc_vs_workspace(big, 64)
    small = W.make_decode("noalloc_small", [5, 37, 300, 1, 0, 129], 8, 2, 64, 903,
                          spare_blocks=2)
    need_small = noalloc_vs_workspace(small, 16)
    assert 0 < need_small < need_big


def test_noalloc_automatic_and_single_pass():
    """The automatic choice (a split here: 64 units are too few for the single
    pass) and then the single pass, which uses no scratch."""
    wl = W.make_decode("noalloc_auto", [4096] * 8, 32, 8, 128, 904)
    assert B.pkv_decode_partition_tokens(8, 8, 4096) > 0
    noalloc_vs_workspace(wl, 0)
    noalloc_vs_workspace(W.make_decode("noalloc_fused", [700, 33, 2048], 16, 4, 128, 905), -4)


def test_noalloc_rejects_split_beyond_scratch():
    """A split whose partials exceed the scratch is refused before any launch."""
    wl = W.make_decode("noalloc_huge", [32768] * 4, 32, 8, 128, 906, store=False)
    need = B.pkv_decode_workspace_bytes(4, 32, 128, 32768, 16)
    assert need > B.pkv_decode_noalloc_max_bytes()
    q = torch.zeros((4, 32, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((16, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((4, 2048), dtype=torch.int32, device="cuda")
    ctx = torch.from_numpy(wl.context_lens).cuda()
    out = torch.zeros_like(q)
    with pytest.raises(B.PkvError) as e:
        B.pkv_decode_attn_noalloc(q, kc, kc, bt, ctx, wl.scale, out, max_context_len=32768,
                                  partition_tokens=16)
    assert e.value.status == B.PKV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0  # nothing ran
