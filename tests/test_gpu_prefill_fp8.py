"""GPU parity of chunked causal prefill over an FP8 cache (pkv_prefill_attn_fp8)
against the oracle's prefill_fp8 on the same seeded inputs.

Caches filled the way serving fills them -- N(0,1) bf16 rows quantized by the
FP8 store, the GPU pools by pkv_store_fp8 and the host pools by the oracle's
store, compared bit for bit -- are held to max |err| 1e-2 and mean |err| 1e-3
with no allowance.  Caches of uniformly random codes (dequantized values up to
about 5) and sharpened or zero scales take the output's own bf16 rounding on
top of the bound, as the bf16 tests of such cases do.
"""
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


def gpu_prefill_fp8(c, dev):
    d = c.dev
    out = torch.empty_like(d["q"])
    B.pkv_prefill_attn_fp8(d["q"], *dev, d["block_tables"], d["cu_new_lens"], d["context_lens"],
                           c.wl.scale, out, max_new_len=c.wl.max_new_len,
                           max_context_len=c.wl.max_context_len)
    return out


def quantized_prefill(wl):
    """Chunked prefill over an FP8 cache of store-quantized N(0,1) data: the
    cached tokens quantized into both sides' pools, the new tokens stored by
    pkv_store_fp8 (GPU) and the oracle's store_fp8 (host), the stored codes and
    scales compared, then the attention on each side."""
    c = Case(wl)
    host, dev = fp8_quantized_pools(wl, c.dev["k_caches"][0], c.dev["v_caches"][0])
    B.pkv_store_fp8(c.dev["k_new"], c.dev["v_new"], c.dev["slot_mapping"], *dev)
    out = gpu_prefill_fp8(c, dev)
    torch.cuda.synchronize()
    orc().store_fp8(c.h["k_new"], c.h["v_new"], wl.slot_mapping, *host)
    for got, ref, what in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(got.cpu().numpy().view(np.uint8), ref.view(np.uint8)), what
    ref = orc().prefill_fp8(c.h["q"], *host, wl.block_tables, wl.cu_new_lens, wl.context_lens,
                            wl.scale)
    return out, ref


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_prefill_fp8_quantized(d, g):
    """Ragged prompts (0 / 37 / 5 / 300 cached, 70 / 16 / 1 / 129 new): several
    query blocks, partial last blocks and key chunks, a one-token prompt."""
    wl = W.make_prefill(f"pf8_d{d}_g{g}", [0, 37, 5, 300], [70, 16, 1, 129], 2 * g, 2, d,
                        900 + d + g, spare_blocks=2)
    say(f"[gpu] prefill fp8 quantized {wl.name}")
    out, ref = quantized_prefill(wl)
    compare(out, ref, f"prefill fp8 {wl.name}")


@pytest.mark.parametrize("g", [1, 4])
def test_prefill_fp8_precise_boundary(g):
    """Waves whose rows see at most 128 keys (hi + lo weights) beside the rest,
    over store-quantized data: prompts straddling position 128."""
    wl = W.make_prefill(f"pf8_boundary_g{g}", [0, 100, 127], [200, 60, 2], 8 * g, 8, 128,
                        950 + g, spare_blocks=1)
    say(f"[gpu] prefill fp8 precise boundary G={g}")
    out, ref = quantized_prefill(wl)
    compare(out, ref, f"prefill fp8 boundary G={g}")


def test_prefill_fp8_long_cached_context():
    """Two prompts of 300 new tokens after 2,000 and 3,500 cached ones: long
    runs of key chunks in each workgroup, store-quantized data."""
    wl = W.make_prefill("pf8_long", [2000, 3500], [300, 300], 32, 8, 128, 960, spare_blocks=1)
    say("[gpu] prefill fp8 long cached contexts")
    out, ref = quantized_prefill(wl)
    compare(out, ref, "prefill fp8 long cached contexts")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_prefill_fp8_scale_edges(scale):
    wl = W.make_prefill("pf8_scale", [0, 37, 130], [70, 16, 65], 8, 2, 128, 961, scale=scale,
                        spare_blocks=1)
    say(f"[gpu] prefill fp8 scale {scale}")
    out, ref = quantized_prefill(wl)
    compare(out, ref, f"prefill fp8 scale {scale}", plus_floor=True)


@pytest.mark.parametrize("d,g", [(64, 1), (128, 4), (128, 8)])
def test_prefill_fp8_random_codes(d, g):
    """Every finite code at random with log-uniform scales, NaN codes and
    scales in every slot outside the contexts."""
    wl = W.make_prefill(f"pf8_rand_d{d}_g{g}", [0, 37, 5, 300], [70, 16, 1, 129], 2 * g, 2, d,
                        970 + d + g, spare_blocks=2)
    say(f"[gpu] prefill fp8 random codes {wl.name}")
    c = Case(wl)
    host, dev = random_code_pools(wl)
    out = gpu_prefill_fp8(c, dev)
    torch.cuda.synchronize()
    ref = orc().prefill_fp8(c.h["q"], *host, wl.block_tables, wl.cu_new_lens, wl.context_lens,
                            wl.scale)
    compare(out, ref, f"prefill fp8 random codes {wl.name}", plus_floor=True)


def test_prefill_fp8_chunked_full_size():
    """The 8 x 2048-token chunked prefill (cached 336 .. 3925 tokens) over an
    FP8 cache of random codes, in the launch the benchmark times: every row of
    every prompt against the oracle."""
    wl = W.chunked_prefill()
    say(f"[gpu] prefill fp8 {wl.name} full size; oracle on every row")
    c = Case(wl)
    host, dev = random_code_pools(wl)
    out = gpu_prefill_fp8(c, dev)
    torch.cuda.synchronize()
    ref = orc().prefill_fp8(c.h["q"], *host, wl.block_tables, wl.cu_new_lens, wl.context_lens,
                            wl.scale)
    compare(out, ref, "prefill fp8 chunked full size (every row)", plus_floor=True)


def test_prefill_fp8_unit_scales_match_bf16_prefill():
    """With every scale 1 an FP8 cache holds bf16 values: codes drawn with
    exponent fields up to 8 (magnitudes up to 3.75, as for N(0,1) data), scales
    1.  The FP8 prefill and the bf16 prefill over the decoded values (another
    kernel path: no scales, K staged directly) both stay within the bound of
    the oracle."""
    wl = W.make_prefill("pf8_unit", [0, 37, 300], [70, 16, 129], 8, 2, 128, 980, spare_blocks=1)
    c = Case(wl)
    host, _ = random_code_pools(wl)
    rng = np.random.default_rng(981)
    for x in host[:2]:
        small = (rng.integers(0, 0x48, x.shape) | (rng.integers(0, 2, x.shape) << 7)).astype(np.uint8)
        x[...] = np.where(x == 0x7F, x, small)   # the NaN code marks the slots outside the contexts
    for x in host[2:]:
        x[np.isfinite(x)] = 1.0
    dev = [torch.from_numpy(x).cuda() for x in host]
    out = gpu_prefill_fp8(c, dev)
    kb = dev[0].view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = dev[1].view(torch.float8_e4m3fn).to(torch.bfloat16)
    out_bf16 = torch.empty_like(out)
    B.pkv_prefill_attn(c.dev["q"], kb, vb, c.dev["block_tables"], c.dev["cu_new_lens"],
                       c.dev["context_lens"], wl.scale, out_bf16, max_new_len=wl.max_new_len,
                       max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    ref = orc().prefill_fp8(c.h["q"], *host, wl.block_tables, wl.cu_new_lens, wl.context_lens,
                            wl.scale)
    compare(out, ref, "prefill fp8 unit scales")
    compare(out_bf16, ref, "prefill bf16 over the decoded codes")
