"""Shared machinery of the GPU parity tests: run a workload through libpkv on
the GPU and through the fp64 oracle on the host, on the same seeded inputs.

The oracle always starts from the generator's pre-store cache and new K/V (host
copies taken before the GPU store runs) and applies its own store, so no
expected value comes from the GPU path.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_cache_pools_amd import binding as B
from paged_kv_cache_pools_amd import workloads as W

MAX_ABS = 1e-2   # attention tolerance vs the fp64 oracle (bf16 in, fp32 accumulate, bf16 out)
MEAN_ABS = 1e-3


def say(msg):
    print(msg, flush=True)


def bits(t):
    return W.bf16_bits(t)


def to_f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def compare(got, ref, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS, plus_floor=False):
    """got: bf16 torch tensor (GPU), ref: float64 numpy.  Returns the stats.

    With ``plus_floor`` each element may also differ by its own bf16 rounding
    (|bf16(ref) - ref|) on top of ``max_abs``, and the mean by the mean of that
    rounding on top of ``mean_abs``.  A bf16 output of magnitude 2 to 4 is
    already up to 7.8e-3 from the exact value by its own rounding, and one of
    magnitude 4 or more up to 1.56e-2, so no bf16 result holds 1e-2 there; a
    batch of rows that each return about one V row of N(0,1) data averages
    about 1e-3 of rounding by itself.  Such outputs need rows dominated by one
    or two keys: sharpened or zero scales, and FP8 caches of uniformly random
    codes (|V| up to about 5).  Only those tests take the allowance; every test
    on N(0,1) data at the configured 1/sqrt(d) scale is held to the plain
    bound."""
    g = to_f64(got)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    floor = np.abs(torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy() - ref)
    stats = dict(max=float(err.max()), mean=float(err.mean()), floor_mean=float(floor.mean()),
                 max_over_floor=float((err - floor).max()))
    say(f"    {what}: max|err| {stats['max']:.3e} mean|err| {stats['mean']:.3e} "
        f"(bf16 rounding floor mean {stats['floor_mean']:.3e}; "
        f"max beyond floor {stats['max_over_floor']:.3e})")
    bound = max_abs + floor if plus_floor else max_abs
    mean_bound = mean_abs + stats["floor_mean"] if plus_floor else mean_abs
    assert np.all(err <= bound) and stats["mean"] <= mean_bound, (what, stats)
    return stats


def orc():
    return oracle.get()


class Case:
    """A workload with its tensors on the GPU plus host copies for the oracle."""

    def __init__(self, wl, device="cuda", gen_device="cpu", seed=None, nan_fill=True, layers=1):
        self.wl = wl
        t = W.make_tensors(wl, device=gen_device, layers=layers, nan_fill=nan_fill, seed=seed)
        self.host_src = gen_device == "cpu"
        self.t = t
        self.dev = {}
        for k in ("q", "k_new", "v_new", "block_tables", "context_lens", "slot_mapping",
                  "cu_new_lens"):
            self.dev[k] = t[k].to(device)
        self.dev["k_caches"] = [x.to(device) for x in t["k_caches"]]
        self.dev["v_caches"] = [x.to(device) for x in t["v_caches"]]
        if self.host_src:
            # pre-store host copies for the oracle
            self.h = {k: bits(t[k]) for k in ("q", "k_new", "v_new")}
            self.h["kc"] = bits(t["k_caches"][0]).copy()
            self.h["vc"] = bits(t["v_caches"][0]).copy()

    # -- GPU side --------------------------------------------------------------
    def gpu_store(self, layer=0):
        d = self.dev
        B.pkv_store(d["k_new"], d["v_new"], d["slot_mapping"], d["k_caches"][layer],
                    d["v_caches"][layer])

    def gpu_decode(self, layer=0, partition_tokens=0, max_context_len=None):
        d = self.dev
        out = torch.empty_like(d["q"])
        B.pkv_decode_attn(d["q"], d["k_caches"][layer], d["v_caches"][layer], d["block_tables"],
                          d["context_lens"], self.wl.scale, out,
                          max_context_len=max_context_len or self.wl.max_context_len,
                          partition_tokens=partition_tokens)
        return out

    def gpu_prefill(self, layer=0):
        d = self.dev
        out = torch.empty_like(d["q"])
        B.pkv_prefill_attn(d["q"], d["k_caches"][layer], d["v_caches"][layer], d["block_tables"],
                           d["cu_new_lens"], d["context_lens"], self.wl.scale, out,
                           max_new_len=self.wl.max_new_len,
                           max_context_len=self.wl.max_context_len)
        return out

    # -- oracle side (whole problem, host-generated inputs) ----------------------
    def oracle_store(self):
        h = self.h
        orc().store(h["k_new"], h["v_new"], self.wl.slot_mapping, h["kc"], h["vc"])

    def oracle_decode(self, nthreads=0):
        h = self.h
        return orc().decode(h["q"], h["kc"], h["vc"], self.wl.block_tables, self.wl.context_lens,
                            self.wl.scale, nthreads=nthreads)

    def oracle_prefill(self, nthreads=0):
        h = self.h
        return orc().prefill(h["q"], h["kc"], h["vc"], self.wl.block_tables, self.wl.cu_new_lens,
                             self.wl.context_lens, self.wl.scale, nthreads=nthreads)


def compact_for_oracle(wl, t, seqs, layer=0):
    """Host inputs for the oracle restricted to the sequences ``seqs``: the
    pre-store blocks they reference (renumbered), their block-table rows,
    their new tokens' K/V and slots (renumbered), and their q rows.

    ``t`` are the generator's tensors (any device), taken before the GPU store.
    """
    seqs = list(seqs)
    bs = wl.block_size
    rows = []
    for s in seqs:
        nb = -(-int(wl.context_lens[s]) // bs)
        rows.append(wl.block_tables[s, :nb])
    ids = np.unique(np.concatenate(rows))
    remap = {int(b): i for i, b in enumerate(ids)}
    width = max(len(r) for r in rows)
    bt = np.full((len(seqs), max(width, 1)), -1, np.int32)
    for i, r in enumerate(rows):
        bt[i, : len(r)] = [remap[int(b)] for b in r]
    idx = torch.from_numpy(ids.astype(np.int64)).to(t["k_caches"][layer].device)
    kc = bits(t["k_caches"][layer].index_select(0, idx)).copy()
    vc = bits(t["v_caches"][layer].index_select(0, idx)).copy()
    cu = wl.cu_new_lens
    tok = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]).astype(np.int64)
    slots = wl.slot_mapping[tok]
    new_slots = np.array([remap[int(x) // bs] * bs + int(x) % bs if x >= 0 else -1 for x in slots],
                         np.int32)
    tok_t = torch.from_numpy(tok).to(t["k_new"].device)
    k_new = bits(t["k_new"].index_select(0, tok_t))
    v_new = bits(t["v_new"].index_select(0, tok_t))
    ctx = wl.context_lens[seqs].astype(np.int32)
    new_lens = wl.new_lens[seqs].astype(np.int32)
    if wl.kind == "decode":
        q = bits(t["q"].index_select(0, torch.tensor(seqs, device=t["q"].device)))
    else:
        q = bits(t["q"].index_select(0, tok_t))
    return dict(kc=kc, vc=vc, bt=bt, ctx=ctx, new_lens=new_lens, slots=new_slots, k_new=k_new,
                v_new=v_new, q=q, tok=tok, ids=ids)


def assert_pool_matches(dev_pool, ids, host_pool, what):
    """The GPU pool's blocks ``ids`` (the compacted copy's block i is pool block
    ids[i]) equal the oracle's pool bit for bit."""
    idx = torch.from_numpy(np.asarray(ids, np.int64)).to(dev_pool.device)
    got = dev_pool.index_select(0, idx)
    if got.dtype == torch.bfloat16:
        g = bits(got)
    else:
        g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint8), host_pool.view(np.uint8)), what


# ---------------------------------------------------------------------------
# FP8 pools filled from N(0,1) data the way serving fills them: every cached
# token's bf16 K/V row quantized by the FP8 store.  The GPU pools go through
# pkv_store_fp8, the host pools through the oracle's store, from the same bf16
# bits; neither side's codes or scales come from the other.
# ---------------------------------------------------------------------------

FP8_NAN = 0x7F  # an E4M3 NaN code: slots no store wrote keep it (and a NaN scale)


def fp8_nan_pools(wl):
    """Host FP8 pools (k codes, v codes, k scales, v scales) holding only NaN."""
    shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    codes = [np.full(shape, FP8_NAN, np.uint8) for _ in range(2)]
    scales = [np.full(shape[:3], np.nan, np.float32) for _ in range(2)]
    return codes + scales


def fp8_quantized_pools(wl, k_cache, v_cache):
    """Quantize every cached token (pre-store live slots) of the bf16 pools
    ``k_cache`` / ``v_cache`` (torch, any device) into FP8 pools: returns
    (host pools written by the oracle, GPU pools written by pkv_store_fp8).
    The two are compared bit for bit before they are returned."""
    live = W.live_slot_mask(wl, pre_store=True)
    slots = np.flatnonzero(live.reshape(-1)).astype(np.int32)  # slot = block * 16 + offset
    host = fp8_nan_pools(wl)
    dev = [torch.from_numpy(x).cuda() for x in host]
    if slots.size:
        nb, hkv, bs, d = k_cache.shape
        idx = torch.from_numpy(slots.astype(np.int64)).to(k_cache.device)
        rows_k = k_cache.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d).index_select(0, idx)
        rows_v = v_cache.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d).index_select(0, idx)
        B.pkv_store_fp8(rows_k.cuda().contiguous(), rows_v.cuda().contiguous(),
                        torch.from_numpy(slots).cuda(), *dev)
        orc().store_fp8(bits(rows_k), bits(rows_v), slots, *host)
        torch.cuda.synchronize()
        for g, h, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
            assert np.array_equal(g.cpu().numpy().view(np.uint8), h.view(np.uint8)), \
                f"FP8 fill differs ({what})"
    return host, dev


def random_code_pools(wl):
    """Uniformly random codes and scales in every slot the sequences' contexts
    cover (their new tokens included, as after their store); the NaN code and
    a NaN scale everywhere else.  Returns (host pools, GPU pools)."""
    host = [x.numpy().copy() for x in W.make_fp8_pools(wl, device="cpu", nan_fill=False)]
    dead = ~W.live_slot_mask(wl, pre_store=False)
    nan = fp8_nan_pools(wl)
    for x, n in zip(host, nan):
        x.swapaxes(1, 2)[dead] = n.swapaxes(1, 2)[dead]
    return host, [torch.from_numpy(x).cuda() for x in host]

