"""The block pool driving the kernels on the GPU: block copies bit-exact
against the oracle, and whole serving steps -- prompts admitted with prefix
caching, a fork whose appends force copy-on-write, decode steps across block
boundaries, a sequence finishing and a new one admitted into its blocks --
with every cache byte and every attention output checked against the oracle
run on the same block tables."""
import numpy as np
import pytest
import torch

from gpu_cases import bits, compare, orc, say
from paged_kv_cache_pools_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _nan_pool(nb, hkv, d, gen):
    x = torch.randn((nb, hkv, 16, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    x[nb // 2:] = float("nan")     # half the pool starts as NaN sentinels
    return x


@pytest.mark.parametrize("hkv,d", [(2, 128), (8, 128), (1, 64)])
def test_copy_blocks_bit_exact(hkv, d):
    """Pools of a few layers (K and V each), FP8 code and scale pools, valid
    and invalid pairs; block sizes below, at and above the 16 KiB chunk."""
    gen = torch.Generator().manual_seed(70 + hkv + d)
    nb = 40
    pools = [_nan_pool(nb, hkv, d, gen) for _ in range(6)]
    codes = [torch.randint(0, 256, (nb, hkv, 16, d), generator=gen, dtype=torch.uint8)
             for _ in range(2)]
    scales = [torch.rand((nb, hkv, 16), generator=gen, dtype=torch.float32) for _ in range(2)]
    pairs = np.array([[3, 30], [0, 21], [7, 7], [-1, 5], [39, 2], [12, 40], [25, 26], [25, 27]],
                     np.int32)
    say(f"[gpu] copy_blocks hkv={hkv} d={d}: {len(pairs)} pairs over 6 bf16 + 2 code + 2 scale pools")
    for group in (pools, codes, scales):
        host = [g.contiguous().view(torch.uint8).numpy().copy() for g in group]
        dev = [g.cuda() for g in group]
        B.pkv_copy_blocks(dev, torch.from_numpy(pairs).cuda())
        torch.cuda.synchronize()
        orc().copy_blocks(host, pairs)
        for h, g in zip(host, dev):
            assert np.array_equal(h, g.cpu().contiguous().view(torch.uint8).numpy())


def test_copy_blocks_many_pools():
    """More pools than one launch carries (64): every pool is copied."""
    gen = torch.Generator().manual_seed(77)
    pools = [torch.randn((6, 1, 16, 64), generator=gen).to(torch.bfloat16) for _ in range(70)]
    pairs = np.array([[1, 4], [5, 0]], np.int32)
    host = [p.view(torch.int16).numpy().copy() for p in pools]
    dev = [p.cuda() for p in pools]
    say("[gpu] copy_blocks over 70 pools")
    B.pkv_copy_blocks(dev, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    orc().copy_blocks(host, pairs)
    for h, g in zip(host, dev):
        assert np.array_equal(h, g.cpu().view(torch.int16).numpy())


class Engine:
    """One GPU state and one host (oracle) state of L layer pools, advanced
    together through the pool's tables."""

    def __init__(self, nb, hq, hkv, d, layers, seed, prefix_caching=True):
        self.pool = B.BlockPool(nb, 16, prefix_caching)
        self.hq, self.hkv, self.d, self.L = hq, hkv, d, layers
        self.scale = 1.0 / np.sqrt(d)
        self.gen = torch.Generator().manual_seed(seed)
        self.kc = [_nan_pool(nb, hkv, d, self.gen) for _ in range(layers)]
        self.vc = [_nan_pool(nb, hkv, d, self.gen) for _ in range(layers)]
        self.hk = [bits(x).copy() for x in self.kc]
        self.hv = [bits(x).copy() for x in self.vc]
        self.kc = [x.cuda() for x in self.kc]
        self.vc = [x.cuda() for x in self.vc]
        self.maxb = 16
        self.shared_groups = 0  # groups with a shared prefix the decode steps met

    def rand(self, *shape):
        return torch.randn(shape, generator=self.gen).to(torch.bfloat16)

    def tables(self, ids):
        bt, ctx = self.pool.block_tables(ids, self.maxb)
        return bt, ctx

    def check_caches(self, what):
        for l in range(self.L):
            assert np.array_equal(bits(self.kc[l]), self.hk[l]), f"{what}: K cache layer {l}"
            assert np.array_equal(bits(self.vc[l]), self.hv[l]), f"{what}: V cache layer {l}"

    def prefill(self, prompts):
        """prompts: {seq id: token list}.  Admit, store the computed tokens,
        run chunked prefill from each prompt's cached prefix."""
        ids = list(prompts)
        new_slots, new_lens, cached = [], [], {}
        for sid in ids:
            slots, c = self.pool.add_seq(sid, prompts[sid])
            cached[sid] = c
            new_slots.append(slots[c:])
            new_lens.append(len(prompts[sid]) - c)
            assert np.all(slots[:c] == -1) and np.all(slots[c:] >= 0)
        slots = np.concatenate(new_slots).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int32)
        bt, ctx = self.tables(ids)
        total = int(cu[-1])
        say(f"[gpu] pool prefill: seqs {ids}, cached {[cached[s] for s in ids]}, new {new_lens}")
        for l in range(self.L):
            k, v = self.rand(total, self.hkv, self.d), self.rand(total, self.hkv, self.d)
            q = self.rand(total, self.hq, self.d)
            B.pkv_store(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), self.kc[l], self.vc[l])
            out = torch.empty((total, self.hq, self.d), dtype=torch.bfloat16, device="cuda")
            B.pkv_prefill_attn(q.cuda(), self.kc[l], self.vc[l], torch.from_numpy(bt).cuda(),
                               torch.from_numpy(cu).cuda(), torch.from_numpy(ctx).cuda(),
                               self.scale, out, max_new_len=int(max(new_lens)),
                               max_context_len=int(ctx.max()))
            torch.cuda.synchronize()
            orc().store(bits(k), bits(v), slots, self.hk[l], self.hv[l])
            ref = orc().prefill(bits(q), self.hk[l], self.hv[l], bt, cu, ctx, self.scale)
            compare(out, ref, f"pool prefill layer {l}")
        self.check_caches("prefill")
        return cached

    def decode(self, ids, tokens):
        """One decode step: append (with copy-on-write), copy, then the fused
        store + decode per layer."""
        slots, copies = self.pool.append(ids, tokens)
        bt, ctx = self.tables(ids)
        if len(copies):
            pools = [x for l in range(self.L) for x in (self.kc[l], self.vc[l])]
            B.pkv_copy_blocks(pools, torch.from_numpy(np.ascontiguousarray(copies)).cuda())
            orc().copy_blocks([x for l in range(self.L) for x in (self.hk[l], self.hv[l])], copies)
        n = len(ids)
        for l in range(self.L):
            k, v = self.rand(n, self.hkv, self.d), self.rand(n, self.hkv, self.d)
            q = self.rand(n, self.hq, self.d)
            out = torch.empty((n, self.hq, self.d), dtype=torch.bfloat16, device="cuda")
            B.pkv_store_decode_attn(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), q.cuda(),
                                    self.kc[l], self.vc[l], torch.from_numpy(bt).cuda(),
                                    torch.from_numpy(ctx).cuda(), self.scale, out,
                                    max_context_len=int(ctx.max()))
            # the same step through the shared-prefix decode, with the groups
            # the pool's tables hold (the caches now include the new tokens)
            starts, plens, mg = B.pkv_prefix_groups(bt, ctx)
            out2 = torch.empty_like(out)
            B.pkv_decode_attn_prefix(q.cuda(), self.kc[l], self.vc[l], torch.from_numpy(bt).cuda(),
                                     torch.from_numpy(ctx).cuda(), self.scale, out2,
                                     torch.from_numpy(starts).cuda(), torch.from_numpy(plens).cuda(),
                                     mg, max_context_len=int(ctx.max()), partition_tokens=16)
            torch.cuda.synchronize()
            self.shared_groups += int((plens > 0).sum())
            orc().store(bits(k), bits(v), slots, self.hk[l], self.hv[l])
            ref = orc().decode(bits(q), self.hk[l], self.hv[l], bt, ctx, self.scale)
            compare(out, ref, f"pool decode layer {l} ctx {ctx.tolist()}")
            compare(out2, ref, f"pool shared-prefix decode layer {l} groups {starts.tolist()} "
                               f"prefixes {plens.tolist()}")
        self.check_caches("decode")
        return copies


def test_pool_driven_serving_steps():
    eng = Engine(nb=48, hq=8, hkv=2, d=128, layers=2, seed=90)
    rng = np.random.default_rng(91)
    system = rng.integers(0, 1000, 32).tolist()               # two full blocks, shared
    prompts = {0: system + rng.integers(0, 1000, 20).tolist(),
               1: system + rng.integers(0, 1000, 5).tolist(),
               2: rng.integers(0, 1000, 17).tolist()}
    cached = eng.prefill(prompts)
    assert cached == {0: 0, 1: 32, 2: 0}                       # seq 1 reuses the system prompt
    assert all(eng.pool.refcount(b) == 2 for b in eng.pool.block_table(0)[:2])
    eng.pool.fork(0, 3)                                         # parallel sample of seq 0
    ids = [0, 1, 2, 3]
    copies = eng.decode(ids, [1, 2, 3, 4])
    # seq 0 appends first into the shared, partly filled block and moves to a
    # copy of it; seq 3 then holds the original alone and writes in place
    assert copies.tolist() == [[eng.pool.block_table(3)[-1], eng.pool.block_table(0)[-1]]]
    seen_boundary = False
    for step in range(14):                                      # crosses block boundaries
        eng.decode(ids, list(range(step, step + 4)))
        seen_boundary |= any(eng.pool.seq_len(s) % 16 == 1 for s in ids)
    assert seen_boundary
    eng.pool.free_seq(2)
    prompts = {4: system + rng.integers(0, 1000, 40).tolist()}
    assert eng.prefill(prompts) == {4: 32}
    eng.decode([0, 1, 3, 4], [5, 6, 7, 8])
    # the fork next to its parent: they share every full block of seq 0 from
    # before the fork; then seqs 1 and 4 share the system prompt
    eng.decode([0, 3, 1, 4], [9, 10, 11, 12])
    assert eng.shared_groups > 0
    for s in (0, 1, 3, 4):
        eng.pool.free_seq(s)
    assert eng.pool.num_free() == 48
