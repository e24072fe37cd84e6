"""Seeded synthetic workloads for paged-KV-cache store + attention.

This module only builds inputs: block tables, context lengths, slot mappings
and N(0,1) bf16 data.  It holds none of the attention or store arithmetic; it
plays the part of the block manager (the KV "control plane" of the Nano-vLLM
part 2 page, §05) that hands the data plane its block tables and slots.
Both the GPU path and the fp64 oracle consume what it produces.

Configurations (shapes follow the pages' models; no dataset is involved):
  tiny            2 seqs, ctx 5 and 37, 4 q / 2 kv heads, d 64, 16 physical
                  blocks assigned by a seeded permutation, scale 1/8
  qwen_mha        32 q = 32 kv heads x 128 (the Qwen head shape of the
                  Nano-vLLM part 2 page, §4.1), 16 seqs, ctx ~ U{128..2048}
  mistral_gqa     32 q / 8 kv heads x 128 (the Mistral-7B-style example of the
                  LLM-primer page, §17.3), 32 seqs x 4096 tokens, 32 layer pools
  cont_batch      256 seqs, GQA 32/8, groups of 32 share one 2048-token prefix
                  through identical physical block ids (LLM-primer §17.6), the
                  rest of each context lognormal(median 512, sigma 1)
  chunked_prefill 8 prompts x 2048 new tokens after U{0..4096} cached ones

Conventions:
  slot = physical_block * block_size + offset   (slot < 0: skip)
  context_lens count tokens AFTER the store of this step.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BLOCK_SIZE = 16


@dataclass
class Workload:
    name: str
    kind: str  # "decode" or "prefill"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    block_tables: np.ndarray  # int32 [S][max_blocks]
    context_lens: np.ndarray  # int32 [S], after the store
    new_lens: np.ndarray      # int32 [S], tokens stored this step per sequence
    slot_mapping: np.ndarray  # int32 [T], T = sum(new_lens)
    scale: float
    seed: int
    num_layers: int = 1
    block_size: int = BLOCK_SIZE
    shared_blocks: int = 0    # physical blocks referenced by more than one sequence
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def cu_new_lens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.new_lens)
        return cu

    @property
    def max_new_len(self) -> int:
        return int(self.new_lens.max()) if self.num_seqs else 0

    def used_blocks(self) -> np.ndarray:
        """Sorted unique physical ids referenced by the live part of every table."""
        ids = []
        for s in range(self.num_seqs):
            nb = -(-int(self.context_lens[s]) // self.block_size)
            ids.append(self.block_tables[s, :nb])
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)


# --------------------------------------------------------------------------
# block tables from explicit per-sequence block lists
# --------------------------------------------------------------------------

def _table(blocks_per_seq: List[np.ndarray], width: Optional[int] = None) -> np.ndarray:
    width = width or max((len(b) for b in blocks_per_seq), default=0)
    width = max(width, 1)
    bt = np.full((len(blocks_per_seq), width), -1, dtype=np.int32)
    for s, b in enumerate(blocks_per_seq):
        bt[s, : len(b)] = b
    return bt


def _slots_for_positions(bt_row: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    return (bt_row[positions // block_size].astype(np.int64) * block_size
            + positions % block_size).astype(np.int32)


def make_decode(name, context_lens, num_q_heads, num_kv_heads, head_dim, seed,
                scale=None, num_layers=1, spare_blocks=0, block_size=BLOCK_SIZE,
                prefix_groups=None, prefix_tokens=0, store=True) -> Workload:
    """Decode workload: every sequence stores one new token at position ctx-1
    (when ``store``), then attends over its whole context.

    ``prefix_groups``: optional list of sequence-index lists; each group shares
    its first ``prefix_tokens`` tokens (a whole number of blocks) through the
    same physical block ids.  ``spare_blocks`` extra physical blocks stay
    unreferenced (filled with NaN sentinels in parity runs).
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int32)
    s_count = ctx.shape[0]
    nblk = [-(-int(c) // block_size) for c in ctx]
    if prefix_groups:
        assert prefix_tokens % block_size == 0
        pblk = prefix_tokens // block_size
        group_of = {}
        for gi, grp in enumerate(prefix_groups):
            for s in grp:
                group_of[s] = gi
                assert ctx[s] > prefix_tokens, "a shared prefix must be followed by private tokens"
        total = len(prefix_groups) * pblk + sum(
            nb - (pblk if s in group_of else 0) for s, nb in enumerate(nblk))
    else:
        pblk = 0
        group_of = {}
        total = sum(nblk)
    num_blocks = total + spare_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    prefix_ids = []
    for _ in (prefix_groups or []):
        prefix_ids.append(perm[cursor: cursor + pblk])
        cursor += pblk
    rows = []
    for s in range(s_count):
        if s in group_of:
            own = nblk[s] - pblk
            rows.append(np.concatenate([prefix_ids[group_of[s]], perm[cursor: cursor + own]]))
            cursor += own
        else:
            rows.append(perm[cursor: cursor + nblk[s]])
            cursor += nblk[s]
    bt = _table(rows)
    if store:
        new_lens = np.ones(s_count, dtype=np.int32)
        slots = np.array([_slots_for_positions(bt[s], np.array([ctx[s] - 1]), block_size)[0]
                          if ctx[s] > 0 else -1 for s in range(s_count)], dtype=np.int32)
    else:
        new_lens = np.zeros(s_count, dtype=np.int32)
        slots = np.zeros(0, dtype=np.int32)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    shared = len(prefix_groups or []) * pblk
    return Workload(name=name, kind="decode", num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, num_blocks=num_blocks, block_tables=bt, context_lens=ctx,
                    new_lens=new_lens, slot_mapping=slots, scale=float(np.float32(scale)),
                    seed=seed, num_layers=num_layers, block_size=block_size,
                    shared_blocks=shared)


def make_prefill(name, cached_lens, new_lens, num_q_heads, num_kv_heads, head_dim, seed,
                 scale=None, spare_blocks=0, block_size=BLOCK_SIZE) -> Workload:
    """Chunked prefill: prompt p has ``cached_lens[p]`` tokens already in the
    cache and stores ``new_lens[p]`` new ones at the following positions."""
    rng = np.random.default_rng(seed)
    cached = np.asarray(cached_lens, dtype=np.int32)
    new = np.asarray(new_lens, dtype=np.int32)
    ctx = (cached + new).astype(np.int32)
    nblk = [-(-int(c) // block_size) for c in ctx]
    num_blocks = sum(nblk) + spare_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)
    rows, cursor = [], 0
    for nb in nblk:
        rows.append(perm[cursor: cursor + nb])
        cursor += nb
    bt = _table(rows)
    slots = [
        _slots_for_positions(bt[p], np.arange(cached[p], ctx[p], dtype=np.int64), block_size)
        for p in range(len(ctx))
    ]
    slots = np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(head_dim)))
    return Workload(name=name, kind="prefill", num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, num_blocks=num_blocks, block_tables=bt, context_lens=ctx,
                    new_lens=new, slot_mapping=slots, scale=float(np.float32(scale)), seed=seed,
                    block_size=block_size)


# --------------------------------------------------------------------------
# the five named configurations
# --------------------------------------------------------------------------

def tiny(seed: int = 1) -> Workload:
    """2 seqs (ctx 5, 37), 4 q / 2 kv heads, d 64, 16 physical blocks from a
    seeded permutation: seq 0 gets perm[0:1], seq 1 gets perm[1:4], the other
    12 blocks stay unreferenced."""
    return make_decode("tiny", [5, 37], 4, 2, 64, seed, scale=0.125, spare_blocks=12)


def qwen_mha(seed: int = 2) -> Workload:
    rng = np.random.default_rng(seed + 1000)
    ctx = rng.integers(128, 2048, size=16, endpoint=True)
    return make_decode("qwen_mha", ctx, 32, 32, 128, seed)


def mistral_gqa(seed: int = 3, num_layers: int = 32) -> Workload:
    return make_decode("mistral_gqa", [4096] * 32, 32, 8, 128, seed, num_layers=num_layers)


def cont_batch(seed: int = 4, prefix_reading: str = "A") -> Workload:
    """256 seqs in 8 groups of 32 sharing a 2048-token prefix.

    Reading A (default): ctx = 2048 + u, u = round(lognormal(ln 512, 1.0))
    clipped to [16, 30720], so ctx <= 32768.  Reading B: ctx itself is
    lognormal clipped to [16, 32768] and only sequences longer than 2048 share
    the prefix of their group.
    """
    rng = np.random.default_rng(seed + 1000)
    draw = np.rint(rng.lognormal(mean=np.log(512.0), sigma=1.0, size=256)).astype(np.int64)
    groups = [list(range(g * 32, (g + 1) * 32)) for g in range(8)]
    if prefix_reading == "A":
        ctx = 2048 + np.clip(draw, 16, 30720)
        return make_decode("cont_batch", ctx, 32, 8, 128, seed, prefix_groups=groups,
                           prefix_tokens=2048)
    ctx = np.clip(draw, 16, 32768)
    groups = [[s for s in grp if ctx[s] > 2048] for grp in groups]
    groups = [grp for grp in groups if len(grp) > 1]
    return make_decode("cont_batch_B", ctx, 32, 8, 128, seed, prefix_groups=groups or None,
                       prefix_tokens=2048 if groups else 0)


def chunked_prefill(seed: int = 5) -> Workload:
    rng = np.random.default_rng(seed + 1000)
    cached = rng.integers(0, 4096, size=8, endpoint=True)
    return make_prefill("chunked_prefill", cached, [2048] * 8, 32, 8, 128, seed)


def mixed_step(seed: int = 6) -> Workload:
    """One continuous-batching iteration of 2016 new tokens: the 32 x 4096 GQA
    decode batch (one new token each, listed first) plus 4 prompt chunks of
    496 new tokens after 0, 512, 1536 and 3072 cached ones; 32 q / 8 kv heads,
    d 128."""
    cached = [4095] * 32 + [0, 512, 1536, 3072]
    new = [1] * 32 + [496] * 4
    return make_prefill("mixed_step", cached, new, 32, 8, 128, seed)


def mixed_tail(seed: int = 7) -> Workload:
    """A continuous-batching iteration whose only prompt work is the last
    64-token chunk of a 4096-token prompt: the 32 x 4096 GQA decode batch plus
    one chunk of 64 new tokens after 4032 cached ones; 32 q / 8 kv heads,
    d 128."""
    return make_prefill("mixed_tail", [4095] * 32 + [4032], [1] * 32 + [64], 32, 8, 128, seed)


CONFIGS = {
    "tiny": tiny,
    "qwen_mha": qwen_mha,
    "mistral_gqa": mistral_gqa,
    "cont_batch": cont_batch,
    "chunked_prefill": chunked_prefill,
    "mixed_step": mixed_step,
    "mixed_tail": mixed_tail,
}


# --------------------------------------------------------------------------
# data: N(0,1) fp32 rounded to bf16 (round-to-nearest-even, torch's .to())
# --------------------------------------------------------------------------

def _randn_bf16(torch, shape, gen, device, chunk=1 << 26):
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk):
        m = min(chunk, n - start)
        flat[start: start + m] = torch.randn(m, generator=gen, device=device,
                                             dtype=torch.float32).to(torch.bfloat16)
    return out


def live_slot_mask(wl: Workload, pre_store: bool = True) -> np.ndarray:
    """bool [num_blocks][block_size]: True where a cached token lives.

    With ``pre_store`` the slots this step writes are excluded (they hold
    sentinels before the store)."""
    mask = np.zeros((wl.num_blocks, wl.block_size), dtype=bool)
    for s in range(wl.num_seqs):
        n = int(wl.context_lens[s]) - (int(wl.new_lens[s]) if pre_store else 0)
        if n <= 0:
            continue
        pos = np.arange(n)
        ids = wl.block_tables[s, pos // wl.block_size]
        mask[ids, pos % wl.block_size] = True
    return mask


def make_tensors(wl: Workload, device="cpu", layers: Optional[int] = None, nan_fill: bool = True,
                 seed: Optional[int] = None):
    """Allocate and fill the workload's tensors with torch.

    Returns a dict: q, k_new, v_new (bf16), k_caches / v_caches (lists of bf16
    pools, one per layer), and int32 metadata tensors (block_tables,
    context_lens, slot_mapping, cu_new_lens).  With ``nan_fill`` every cache
    slot that holds no cached token (tails of last blocks, unreferenced blocks,
    and the slots this step's store will write) is set to bf16 NaN.
    """
    import torch

    layers = wl.num_layers if layers is None else layers
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed if seed is None else seed)
    rows_q = wl.num_seqs if wl.kind == "decode" else int(wl.new_lens.sum())
    q = _randn_bf16(torch, (rows_q, wl.num_q_heads, wl.head_dim), gen, device)
    k_new = _randn_bf16(torch, (wl.num_tokens, wl.num_kv_heads, wl.head_dim), gen, device)
    v_new = _randn_bf16(torch, (wl.num_tokens, wl.num_kv_heads, wl.head_dim), gen, device)
    shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    k_caches, v_caches = [], []
    dead = None
    if nan_fill:
        dead = torch.from_numpy(~live_slot_mask(wl, pre_store=True)).to(device)
        dead = dead[:, None, :, None]
    for _ in range(layers):
        kc = _randn_bf16(torch, shape, gen, device)
        vc = _randn_bf16(torch, shape, gen, device)
        if dead is not None:
            kc.masked_fill_(dead, float("nan"))
            vc.masked_fill_(dead, float("nan"))
        k_caches.append(kc)
        v_caches.append(vc)
    meta = {
        "block_tables": torch.from_numpy(wl.block_tables).to(device),
        "context_lens": torch.from_numpy(wl.context_lens).to(device),
        "slot_mapping": torch.from_numpy(wl.slot_mapping).to(device),
        "cu_new_lens": torch.from_numpy(wl.cu_new_lens).to(device),
    }
    return {"q": q, "k_new": k_new, "v_new": v_new, "k_caches": k_caches, "v_caches": v_caches,
            **meta}


def make_fp8_pools(wl: Workload, device="cpu", seed: Optional[int] = None, nan_fill: bool = True):
    """Random FP8 (OCP E4M3) pools for one layer: codes drawn uniformly from the
    finite codes (every byte but 0x7f and 0xff), scales drawn log-uniform in
    [2^-7.5, 2^-6.5), so a row's largest magnitude (448 x scale) lies between
    about 2.5 and 5, as for N(0,1) data.  With ``nan_fill`` every slot that holds
    no cached token (tails,
    unreferenced blocks, the slots this step's store writes) gets the NaN code
    and a NaN scale.  Returns (k_codes, v_codes, k_scales, v_scales) tensors:
    uint8 [NB][Hkv][bs][d] and float32 [NB][Hkv][bs]."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed((wl.seed if seed is None else seed) + 7777)
    shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    out = []
    for _ in range(2):
        c = torch.randint(0, 254, shape, generator=gen, device=device, dtype=torch.int32)
        c = c + (c >= 0x7f).to(torch.int32)          # skip 0x7f: 0..0x7e, 0x80..0xfe
        out.append(c.to(torch.uint8))
    for _ in range(2):
        e = torch.rand(shape[:3], generator=gen, device=device, dtype=torch.float32) - 7.5
        out.append(torch.exp2(e))
    if nan_fill:
        dead = torch.from_numpy(~live_slot_mask(wl, pre_store=True)).to(device)
        out[0].masked_fill_(dead[:, None, :, None], 0x7F)
        out[1].masked_fill_(dead[:, None, :, None], 0x7F)
        out[2].masked_fill_(dead[:, None, :], float("nan"))
        out[3].masked_fill_(dead[:, None, :], float("nan"))
    return tuple(out)


def rope_table(max_positions: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """fp32 [max_positions][head_dim] table of cos (first half) and sin (second
    half) of position * base^(-2i / head_dim), i < head_dim / 2, computed in
    fp64 and rounded once: the caller-side input of the rotary embedding."""
    half = head_dim // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(max_positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def bf16_bits(t) -> np.ndarray:
    """Host numpy uint16 view of a bf16 torch tensor's bits."""
    import torch

    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
