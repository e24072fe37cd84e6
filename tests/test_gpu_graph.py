"""The decode step, the mixed step and the shared-prefix decode (over bf16 and
FP8 caches) and the FP8 chunked prefill captured in a HIP graph
(torch.cuda.graph) and replayed: none of their
launches records a memset, so every replay must reproduce the eager result bit
for bit, with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

from gpu_cases import bits, say
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def replay_and_check(step, outs, what, replays=3):
    """Run `step` eagerly, capture it, replay it `replays` times (clearing the
    outputs eagerly in between) and compare every replay with the eager run."""
    step()
    torch.cuda.synchronize()
    eager = [bits(o).copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for r in range(replays):
        for o in outs:
            o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(bits(o), eager[i]), f"{what}: replay {r} output {i} differs"
    say(f"    {what}: {replays} replays bit-identical to the eager run")


def test_graph_decode_layers():
    """Fused store + decode over 4 layer pools, as one graph."""
    wl = W.make_decode("graph_decode", [100, 2048, 777, 4096, 1, 3000], 32, 8, 128, 310,
                       num_layers=4)
    t = W.make_tensors(wl, device="cuda", layers=4, nan_fill=True)
    outs = [torch.empty_like(t["q"]) for _ in range(4)]
    p = B.pkv_decode_partition_tokens(wl.num_seqs, wl.num_kv_heads, wl.max_context_len)
    ws = torch.empty(max(16, B.pkv_decode_workspace_bytes(wl.num_seqs, 32, 128, wl.max_context_len, p)),
                     dtype=torch.uint8, device="cuda")
    say(f"[gpu] graph: store + decode of 4 layers, work split {p}")

    def step():
        for l in range(4):
            B.pkv_store_decode_attn(t["k_new"], t["v_new"], t["slot_mapping"], t["q"],
                                    t["k_caches"][l], t["v_caches"][l], t["block_tables"],
                                    t["context_lens"], wl.scale, outs[l],
                                    max_context_len=wl.max_context_len, workspace=ws,
                                    partition_tokens=p)
    replay_and_check(step, outs, "decode layers")


@pytest.mark.parametrize("part", [0, 256])
def test_graph_fp8_decode(part):
    """The FP8 fused store + decode (the matrix-core path above 128 keys, the
    fp32 path below) over 2 layer pools, single pass and split-KV, as one
    graph."""
    wl = W.make_decode("graph_fp8", [100, 2048, 777, 4096, 1, 3000, 129], 32, 8, 128, 312)
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    pools = [W.make_fp8_pools(wl, device="cuda", seed=312 + l) for l in range(2)]
    outs = [torch.empty_like(t["q"]) for _ in range(2)]
    p = part or B.pkv_decode_partition_tokens_fp8(wl.num_seqs, wl.num_kv_heads, wl.max_context_len)
    ws = torch.empty(max(16, B.pkv_decode_workspace_bytes(wl.num_seqs, 32, 128, wl.max_context_len, p)),
                     dtype=torch.uint8, device="cuda")
    say(f"[gpu] graph: FP8 store + decode of 2 layers, work split {p}")

    def step():
        for l in range(2):
            B.pkv_store_decode_attn_fp8(t["k_new"], t["v_new"], t["slot_mapping"], t["q"],
                                        *pools[l], t["block_tables"], t["context_lens"], wl.scale,
                                        outs[l], max_context_len=wl.max_context_len, workspace=ws,
                                        partition_tokens=p)
    replay_and_check(step, outs, f"fp8 decode P{p}")


def test_graph_fp8_prefill():
    """The FP8 quantizing store of a chunked-prefill batch and the prefill over
    the FP8 cache, as one graph."""
    wl = W.make_prefill("graph_pf8", [0, 37, 300, 1500], [70, 16, 129, 64], 32, 8, 128, 314,
                        spare_blocks=1)
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    pools = W.make_fp8_pools(wl, device="cuda", seed=314)
    out = torch.empty_like(t["q"])
    say("[gpu] graph: FP8 store + chunked prefill")

    def step():
        B.pkv_store_fp8(t["k_new"], t["v_new"], t["slot_mapping"], *pools)
        B.pkv_prefill_attn_fp8(t["q"], *pools, t["block_tables"], t["cu_new_lens"],
                               t["context_lens"], wl.scale, out, max_new_len=wl.max_new_len,
                               max_context_len=wl.max_context_len)
    replay_and_check(step, [out], "fp8 prefill")


def test_graph_split_decode():
    """Two-pass split-KV decode (partials + merge launch) in a graph."""
    wl = W.make_decode("graph_split", [5000, 17, 1200, 64], 16, 4, 64, 311)
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    out = torch.empty_like(t["q"])
    ws = torch.empty(B.pkv_decode_workspace_bytes(4, 16, 64, wl.max_context_len, 256),
                     dtype=torch.uint8, device="cuda")
    B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][0], t["v_caches"][0])
    say("[gpu] graph: split-KV decode, P = 256")

    def step():
        B.pkv_decode_attn(t["q"], t["k_caches"][0], t["v_caches"][0], t["block_tables"],
                          t["context_lens"], wl.scale, out, max_context_len=wl.max_context_len,
                          workspace=ws, partition_tokens=256)
    replay_and_check(step, [out], "split decode")


def test_graph_mixed_step_split():
    """The mixed step with a split prefill chunk (mixed + merge launches)."""
    wl = W.mixed_tail()
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    mnl, mcl = 64, int(wl.context_lens.max())
    need = B.pkv_mixed_workspace_bytes(wl.num_seqs, 32, mnl, mcl, wl.num_q_heads, wl.num_kv_heads,
                                       wl.head_dim)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][0], t["v_caches"][0])
    say("[gpu] graph: mixed step, 32 decode + one split chunk")

    def step():
        B.pkv_mixed_attn(t["q"], t["k_caches"][0], t["v_caches"][0], t["block_tables"],
                         t["cu_new_lens"], t["context_lens"], 32, wl.scale, out, max_new_len=mnl,
                         max_context_len=mcl, workspace=ws)
    replay_and_check(step, [out], "mixed step")


def test_graph_shared_prefix_decode():
    """Store + shared-prefix decode of a grouped batch."""
    ctx = [320 + x for x in (1, 40, 300, 17, 64, 9, 200)]
    wl = W.make_decode("graph_prefix", ctx, 16, 4, 128, 312, prefix_groups=[[0, 1, 2, 3], [4, 5, 6]],
                       prefix_tokens=320)
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    gs, pl = torch.from_numpy(starts).cuda(), torch.from_numpy(plens).cuda()
    ws = torch.empty(B.pkv_decode_prefix_workspace_bytes(wl.num_seqs, 16, 4, 128, wl.max_context_len, 64),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    say(f"[gpu] graph: store + shared-prefix decode, groups {starts.tolist()}")

    def step():
        B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][0], t["v_caches"][0])
        B.pkv_decode_attn_prefix(t["q"], t["k_caches"][0], t["v_caches"][0], t["block_tables"],
                                 t["context_lens"], wl.scale, out, gs, pl, mg,
                                 max_context_len=wl.max_context_len, workspace=ws,
                                 partition_tokens=64)
    replay_and_check(step, [out], "shared-prefix decode")


def test_graph_fp8_mixed_step_split():
    """The mixed step over an FP8 cache with a split prefill chunk (mixed +
    merge launches), the FP8 store of the step's tokens in the same graph."""
    wl = W.mixed_tail()
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    pools = W.make_fp8_pools(wl, device="cuda", seed=315)
    mnl, mcl = 64, int(wl.context_lens.max())
    need = B.pkv_mixed_workspace_bytes(wl.num_seqs, 32, mnl, mcl, wl.num_q_heads, wl.num_kv_heads,
                                       wl.head_dim)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    say("[gpu] graph: FP8 store + mixed step, 32 decode + one split chunk")

    def step():
        B.pkv_store_fp8(t["k_new"], t["v_new"], t["slot_mapping"], *pools)
        B.pkv_mixed_attn_fp8(t["q"], *pools, t["block_tables"], t["cu_new_lens"], t["context_lens"],
                             32, wl.scale, out, max_new_len=mnl, max_context_len=mcl, workspace=ws)
    replay_and_check(step, [out], "fp8 mixed step")


def test_graph_fp8_shared_prefix_decode():
    """FP8 store + shared-prefix decode of a grouped batch."""
    ctx = [320 + x for x in (1, 40, 300, 17, 64, 9, 200)]
    wl = W.make_decode("graph_prefix8", ctx, 16, 4, 128, 316, prefix_groups=[[0, 1, 2, 3], [4, 5, 6]],
                       prefix_tokens=320)
    t = W.make_tensors(wl, device="cuda", nan_fill=True)
    pools = W.make_fp8_pools(wl, device="cuda", seed=316)
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    gs, pl = torch.from_numpy(starts).cuda(), torch.from_numpy(plens).cuda()
    ws = torch.empty(B.pkv_decode_prefix_workspace_bytes(wl.num_seqs, 16, 4, 128, wl.max_context_len, 64),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    say(f"[gpu] graph: FP8 store + shared-prefix decode, groups {starts.tolist()}")

    def step():
        B.pkv_store_fp8(t["k_new"], t["v_new"], t["slot_mapping"], *pools)
        B.pkv_decode_attn_prefix_fp8(t["q"], *pools, t["block_tables"], t["context_lens"], wl.scale,
                                     out, gs, pl, mg, max_context_len=wl.max_context_len,
                                     workspace=ws, partition_tokens=64)
    replay_and_check(step, [out], "fp8 shared-prefix decode")
