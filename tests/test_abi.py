"""Host-side checks of libpkv.so: it loads, exports every symbol include/pkv.h
declares, and its host-only logic (sizing, partitioning, argument validation
before any launch) behaves.  No GPU: no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from paged_kv_cache_pools_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def header_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libpkv.so is not built (run python -m paged_kv_cache_pools_amd.build)")
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(B.EXPORTED), names
    raw = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_debug_build_exports_every_declared_symbol(lib):
    """The debug-bounds build is the same library: a build of older sources
    (one missing a declared entry point) fails here, before any GPU test."""
    if not os.path.exists(B.LIB_DEBUG_PATH):
        pytest.skip("libpkv_debug.so not built")
    raw = ctypes.CDLL(B.LIB_DEBUG_PATH)
    for n in header_functions():
        assert hasattr(raw, n), n


def test_kv_bytes_matches_pages(lib):
    # LLM primer part 4, §17.3 and §23.2 lab 2 (tests/golden/kv_sizing.json)
    import json

    g = json.load(open(os.path.join(ROOT, "tests", "golden", "kv_sizing.json")))
    for c in g["cases"] + [g["fp8_note"], g["counter_example"]]:
        assert B.pkv_kv_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["tokens"],
                              c["bytes_per_element"]) == c["bytes"], c["cite"]
    assert B.pkv_kv_bytes(-1, 8, 128, 4096, 2) == 0


def test_status_strings(lib):
    for s, name in B.STATUS_NAMES.items():
        assert B.pkv_status_string(s).startswith(name)
    assert "unknown" in B.pkv_status_string(99)


def test_partition_heuristic(lib):
    # the 32 x 4096 GQA batch: 256 (seq, kv head) units -> single pass, 4 waves each
    assert B.pkv_decode_partition_tokens(32, 8, 4096) == -4
    # many units with long contexts, or few units: two-pass split-KV
    assert B.pkv_decode_partition_tokens(256, 8, 32768) == 512
    # many units whose longest context would leave one wave walking 6565
    # tokens alone: two-pass split-KV, not single pass with one wave each
    assert B.pkv_decode_partition_tokens(256, 8, 6565) > 0
    # the 16-sequence MHA batch (512 units, up to 2048 tokens): 4 waves of 512
    assert B.pkv_decode_partition_tokens(16, 32, 2048) == -4
    # more units than compute units and up to 4096 tokens: 8 waves of 512
    assert B.pkv_decode_partition_tokens(64, 8, 4096) == -8
    # many short units: still 4 waves each (one per SIMD)
    assert B.pkv_decode_partition_tokens(256, 8, 512) == -4
    # more units than compute units with contexts past 4096: split-KV
    assert B.pkv_decode_partition_tokens(64, 8, 4200) > 0
    for s, h, ctx in ((1, 1, 1), (2, 2, 37), (256, 8, 32768), (16, 32, 2048), (1, 1, 1 << 20),
                      (32, 8, 4096), (64, 8, 16), (256, 8, 6565)):
        p = B.pkv_decode_partition_tokens(s, h, ctx)
        assert (p % 16 == 0 and 64 <= p <= 512) or (-8 <= p <= -1), (s, h, ctx, p)
        if p < 0:  # no wave walks more than 1024 tokens (512 with more units than CUs)
            assert -(-ctx // -p) <= (1024 if s * h <= 256 else 512)
        if p < 0:  # at least one block per wave
            assert -p <= -(-ctx // 16)
    assert B.pkv_decode_partition_tokens(-1, 8, 10) == 0
    # fewer KV heads never give a longer two-pass partition: workspace(P=0) bounds every choice
    for h in (1, 2, 8, 32):
        for ctx in (100, 4096, 20000):
            p = B.pkv_decode_partition_tokens(32, h, ctx)
            if p > 0:
                assert B.pkv_decode_workspace_bytes(32, 32, 128, ctx, p) <= \
                    B.pkv_decode_workspace_bytes(32, 32, 128, ctx, 0)


def test_workspace_bytes(lib):
    assert B.pkv_decode_workspace_bytes(32, 32, 128, 4096, 256) == 32 * 32 * 16 * 130 * 4
    assert B.pkv_decode_workspace_bytes(32, 32, 128, 256, 256) == 0   # one partition
    assert B.pkv_decode_workspace_bytes(32, 32, 128, 257, 256) == 32 * 32 * 2 * 130 * 4
    assert B.pkv_decode_workspace_bytes(0, 32, 128, 4096, 256) == 0
    assert B.pkv_decode_workspace_bytes(4, 4, 64, 100, 24) == 0      # not a multiple of 16
    assert B.pkv_decode_workspace_bytes(32, 32, 128, 4096, -4) == 0  # single pass
    assert B.pkv_decode_workspace_bytes(32, 32, 128, 4096, 0) == 32 * 32 * 64 * 130 * 4


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced on these paths


def cache(nb=16, hkv=2, d=64, bs=16, k=FAKE, v=FAKE):
    return B.PkvCache(k, v, nb, hkv, d, bs)


def decode(lib, c=None, q=FAKE, out=FAKE, hq=4, s=2, max_ctx=37, max_blocks=3, ws=FAKE,
           ws_bytes=1 << 30, part=0, bt=FAKE, ctx=FAKE):
    return lib.pkv_decode_attn(q, c or cache(), bt, max_blocks, ctx, s, max_ctx, hq,
                               ctypes.c_float(0.125), out, ws, ws_bytes, part, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(c=cache(d=96)), 3),
    (dict(c=cache(bs=32)), 3),
    (dict(hq=5), 2),                       # not a multiple of 2 kv heads
    (dict(hq=6), 3),                       # group 3 unsupported
    (dict(hq=2 * 16), 3),                  # group 16 unsupported
    (dict(c=cache(hkv=3), hq=9), 3),       # group 3 unsupported
    (dict(q=0), 1),
    (dict(out=0), 1),
    (dict(q=FAKE + 8), 4),
    (dict(c=cache(k=FAKE + 2)), 4),
    (dict(max_ctx=49), 2),                 # beyond max_blocks * 16
    (dict(s=-1), 2),
    (dict(ws=0, max_ctx=37, part=16), 5),  # needs partials, no workspace
    (dict(ws_bytes=16, max_ctx=37, part=16), 5),
    (dict(part=24), 2),
    (dict(part=-9), 2),
    (dict(c=cache(nb=0)), 2),
])
def test_decode_rejects_before_launch(lib, kwargs, status):
    assert decode(lib, **kwargs) == status
    assert B.pkv_last_error() != ""


def test_decode_empty_batch_is_ok(lib):
    assert decode(lib, s=0) == 0


def test_store_validation(lib):
    st = lambda n, c=None, k=FAKE, v=FAKE, sl=FAKE: lib.pkv_store(k, v, sl, n, c or cache(), None)
    assert st(0) == 0                         # no-op, nothing launched
    assert st(-1) == 2
    assert st(4, k=0) == 1
    assert st(4, k=FAKE + 4) == 4
    assert st(4, c=cache(d=80)) == 3
    assert st(1 << 30, c=cache(hkv=64, d=128)) == 2


def test_prefill_validation(lib):
    pf = lambda **kw: lib.pkv_prefill_attn(
        kw.get("q", FAKE), kw.get("c", cache()), FAKE, kw.get("max_blocks", 4), FAKE, FAKE,
        kw.get("s", 2), kw.get("max_new", 16), kw.get("max_ctx", 40), kw.get("hq", 4),
        ctypes.c_float(0.125), kw.get("out", FAKE), None)
    assert pf(s=0) == 0 and pf(max_new=0) == 0
    assert pf(max_new=50) == 2              # more new tokens than context
    assert pf(max_ctx=80) == 2              # beyond max_blocks * 16
    assert pf(q=0) == 1
    assert pf(hq=5) == 2
    assert pf(c=cache(d=32)) == 3


def test_store_decode_validation(lib):
    sd = lambda k=FAKE, v=FAKE, sl=FAKE, s=2, q=FAKE: lib.pkv_store_decode_attn(
        k, v, sl, q, cache(), FAKE, 3, FAKE, s, 37, 4, ctypes.c_float(0.125), FAKE, FAKE, 1 << 30,
        0, None)
    assert sd(s=0) == 0                     # empty batch: nothing launched
    assert sd(k=0) == 1 and sd(v=0) == 1 and sd(sl=0) == 1
    assert sd(k=FAKE + 4) == 4
    assert sd(q=0) == 1                     # the decode checks still apply
    assert B.pkv_last_error() != ""


def test_store_decode_rope_validation(lib):
    sd = lambda cs=FAKE, mp=64, s=2, k=FAKE: lib.pkv_store_decode_attn_rope(
        k, FAKE, FAKE, FAKE, cs, mp, cache(), FAKE, 3, FAKE, s, 37, 4, ctypes.c_float(0.125),
        FAKE, FAKE, 1 << 30, 0, None)
    assert sd(s=0, cs=0, mp=0) == 0         # empty batch: nothing launched
    assert sd(cs=0) == 1 and sd(k=0) == 1
    assert sd(cs=FAKE + 4) == 4
    assert sd(mp=0) == 2 and sd(mp=36) == 2  # the table must cover max_context_len 37
    assert sd(mp=37, s=-1) == 2              # past the table check, the decode checks apply
    assert B.pkv_last_error() != ""


def test_mixed_validation(lib):
    mx = lambda nd=1, s=3, mn=16, mc=40, q=FAKE, c=None, hq=4, ws=None, wsb=0, mb=4: \
        lib.pkv_mixed_attn(q, c or cache(), FAKE, mb, FAKE, FAKE, nd, s, mn, mc, hq,
                           ctypes.c_float(0.125), FAKE, ws, wsb, None)
    assert mx(s=0, nd=0) == 0               # empty batch: nothing launched
    assert mx(nd=4) == 2 and mx(nd=-1) == 2  # more decode sequences than sequences
    assert mx(mn=50) == 2                   # more new tokens than context
    assert mx(mc=80) == 2                   # beyond max_blocks * 16
    assert mx(q=0) == 1 and mx(q=FAKE + 8) == 4
    assert mx(hq=6) == 3 and mx(c=cache(d=96)) == 3
    # a workspace too small for the split these sizes call for
    assert B.pkv_mixed_workspace_bytes(3, 1, 16, 3000, 4, 2, 64) > 0
    assert mx(ws=FAKE, wsb=16, mc=3000, mb=200) == 5
    assert mx(ws=FAKE + 4, wsb=1 << 30, mc=3000, mb=200) == 4
    assert B.pkv_last_error() != ""


def test_mixed_workspace_sizing(lib):
    # 32 decode seqs + 1 chunk of 64 after 4032 cached, GQA 32/8, d 128: 1 x 8
    # x 2 units, 8 segments each (4096 / 512), 4 waves x 32 columns x 132
    # floats per segment
    units = 1 * 8 * 2
    assert B.pkv_mixed_workspace_bytes(33, 32, 64, 4096, 32, 8, 128) == units * 8 * 4 * 2 * 16 * 132 * 4
    # 4 chunks of 496: 4 x 8 x 16 = 512 units fill the GPU: no split
    assert B.pkv_mixed_workspace_bytes(36, 32, 496, 4096, 32, 8, 128) == 0
    # many units, or short contexts, or no prefill: no split
    assert B.pkv_mixed_workspace_bytes(40, 8, 2048, 6144, 32, 8, 128) == 0
    assert B.pkv_mixed_workspace_bytes(4, 2, 64, 500, 32, 8, 128) == 0   # one segment's worth of keys
    assert B.pkv_mixed_workspace_bytes(8, 8, 1, 4096, 32, 8, 128) == 0
    assert B.pkv_mixed_workspace_bytes(4, 5, 64, 900, 32, 8, 128) == 0   # invalid: no bytes


def test_fp8_validation(lib):
    c8 = lambda ks=FAKE, vs=FAKE, d=64: B.PkvCacheFp8(FAKE, FAKE, ks, vs, 16, 2, d, 16)
    st = lambda c, n=4: lib.pkv_store_fp8(FAKE, FAKE, FAKE, n, c, None)
    assert st(c8(), 0) == 0
    assert st(c8(ks=0)) == 1
    assert st(c8(vs=FAKE + 4)) == 4
    assert st(c8(d=96)) == 3
    dec = lambda c: lib.pkv_decode_attn_fp8(FAKE, c, FAKE, 3, FAKE, 2, 37, 4,
                                            ctypes.c_float(0.125), FAKE, FAKE, 1 << 30, 0, None)
    assert dec(c8(ks=0)) == 1
    assert dec(c8(vs=FAKE + 8)) == 4
    sd = lambda c=None, k=FAKE, v=FAKE, sl=FAKE, s=2, q=FAKE: lib.pkv_store_decode_attn_fp8(
        k, v, sl, q, c or c8(), FAKE, 3, FAKE, s, 37, 4, ctypes.c_float(0.125), FAKE, FAKE,
        1 << 30, 0, None)
    assert sd(s=0) == 0                     # empty batch: nothing launched
    assert sd(k=0) == 1 and sd(v=0) == 1 and sd(sl=0) == 1
    assert sd(v=FAKE + 4) == 4
    assert sd(c=c8(ks=0)) == 1 and sd(c=c8(d=96)) == 3
    assert sd(q=0) == 1                     # the decode checks still apply
    assert B.pkv_last_error() != ""
    pf = lambda c=None, q=FAKE, s=2, mn=16, mc=40, hq=4: lib.pkv_prefill_attn_fp8(
        q, c or c8(), FAKE, 4, FAKE, FAKE, s, mn, mc, hq, ctypes.c_float(0.125), FAKE, None)
    assert pf(s=0) == 0 and pf(mn=0) == 0   # nothing to attend: nothing launched
    assert pf(c=c8(ks=0)) == 1 and pf(c=c8(vs=FAKE + 4)) == 4 and pf(c=c8(d=96)) == 3
    assert pf(mn=50) == 2 and pf(mc=80) == 2 and pf(hq=5) == 2
    assert pf(q=0) == 1
    assert "null" in B.pkv_last_error()
    mx = lambda c=None, nd=1, s=3, mn=16, mc=40, q=FAKE: lib.pkv_mixed_attn_fp8(
        q, c or c8(), FAKE, 4, FAKE, FAKE, nd, s, mn, mc, 4, ctypes.c_float(0.125), FAKE, None, 0,
        None)
    assert mx(s=0, nd=0) == 0               # empty batch: nothing launched
    assert mx(c=c8(ks=0)) == 1 and mx(c=c8(vs=FAKE + 4)) == 4 and mx(c=c8(d=96)) == 3
    assert mx(nd=4) == 2 and mx(mn=50) == 2 and mx(mc=80) == 2
    assert mx(q=0) == 1
    px = lambda c=None, s=2, q=FAKE, ws=FAKE: lib.pkv_decode_attn_prefix_fp8(
        q, c or c8(), FAKE, 3, FAKE, s, 37, 4, ctypes.c_float(0.125), FAKE, FAKE, 1, 2, FAKE, ws,
        1 << 30, 0, None)
    assert px(s=0) == 0                     # empty batch: nothing launched
    assert px(c=c8(ks=0)) == 1 and px(c=c8(vs=FAKE + 4)) == 4 and px(c=c8(d=96)) == 3
    assert px(q=0) == 1 and px(ws=0) == 5


def test_fp8_partition_heuristic(lib):
    # the 32 x 4096 GQA batch: single pass with 4 waves, as for bf16
    assert B.pkv_decode_partition_tokens_fp8(32, 8, 4096) == -4
    for s, h, ctx in ((32, 8, 4096), (64, 8, 2048), (16, 8, 1000), (3, 2, 50000)):
        assert B.pkv_decode_partition_tokens_fp8(s, h, ctx) == \
            B.pkv_decode_partition_tokens(s, h, ctx)
    for s, h, ctx in ((1, 1, 1), (2, 2, 37), (256, 8, 32768), (16, 32, 2048), (64, 8, 16)):
        p = B.pkv_decode_partition_tokens_fp8(s, h, ctx)
        assert (p % 16 == 0 and 64 <= p <= 1024) or (-8 <= p <= -1), (s, h, ctx, p)
        if p > 0:  # the P = 0 workspace bound covers the FP8 choice too
            assert B.pkv_decode_workspace_bytes(s, 4 * h, 128, ctx, p) <= \
                B.pkv_decode_workspace_bytes(s, 4 * h, 128, ctx, 0)


def test_prefix_decode_validation(lib):
    # every call here fails before a launch
    pd = lambda s=40, mc=37, mb=3, hq=4, c=None, q=FAKE, gs=FAKE, pl=FAKE, ng=2, mg=8, ws=FAKE, \
        wsb=1 << 30, p=0: lib.pkv_decode_attn_prefix(
            q, c or cache(), FAKE, mb, FAKE, s, mc, hq, ctypes.c_float(0.125), gs, pl, ng, mg, FAKE,
            ws, wsb, p, None)
    assert pd(s=-1) == 2 and pd(ng=-1) == 2 and pd(mg=-1) == 2
    assert pd(mg=41) == 2                   # a group larger than the batch
    assert pd(mc=80) == 2                   # beyond max_blocks * 16
    assert pd(s=8193) == 2                  # more sequences than one call's tail list holds
    assert pd(q=0) == 1 and pd(gs=0) == 1 and pd(pl=0) == 1
    assert pd(q=FAKE + 8) == 4
    assert pd(hq=6) == 3 and pd(c=cache(d=96)) == 3 and pd(c=cache(bs=32)) == 3
    assert pd(p=24) == 2 and pd(p=-16) == 2  # partitions: 0 or a positive multiple of 16
    assert pd(ws=0) == 5 and pd(wsb=64) == 5
    assert pd(ws=FAKE + 4) == 4
    assert B.pkv_last_error() != ""


def test_prefix_decode_workspace_sizing(lib):
    # rows x (tail pieces + 8 prefix segments) x (d + 2) floats, then the tail
    # list (wave count + num_seqs + 1 offsets) rounded up to 16 bytes; a tail
    # of up to max_context_len tokens falls into ceil(max_context_len / P) + 1
    # pieces
    lst = lambda s: ((s + 2) * 4 + 15) // 16 * 16
    assert B.pkv_decode_prefix_workspace_bytes(256, 32, 8, 128, 32768, 512) == \
        256 * 32 * (65 + 8) * 130 * 4 + lst(256)
    assert B.pkv_decode_prefix_workspace_bytes(3, 4, 2, 64, 0, 16) == 3 * 4 * 8 * 66 * 4 + lst(3)
    assert B.pkv_decode_prefix_workspace_bytes(3, 1, 2, 64, 33, 16) == \
        3 * 1 * (4 + 8) * 66 * 4 + lst(3)
    # automatic partitions: the split-KV choice, at most 256 tokens
    assert B.pkv_decode_prefix_workspace_bytes(256, 32, 8, 128, 32768, 0) == \
        256 * 32 * (129 + 8) * 130 * 4 + lst(256)
    assert B.pkv_decode_prefix_workspace_bytes(1, 32, 8, 128, 32768, 0) == \
        32 * (32768 // B.pkv_decode_partition_tokens(1, 8, 32768) + 1 + 8) * 130 * 4 + lst(1)
    assert B.pkv_decode_prefix_workspace_bytes(0, 32, 8, 128, 100, 0) == 0
    assert B.pkv_decode_prefix_workspace_bytes(4, 32, 8, 128, 100, 24) == 0


def test_read_probe_validation(lib):
    FAKE = 1 << 20  # never dereferenced: every call below fails on the host or launches nothing
    assert lib.pkv_read_probe(None, 0, None, None) == 0          # nothing to read
    assert lib.pkv_read_probe(None, 64, FAKE, None) == 1         # null buffer
    assert lib.pkv_read_probe(FAKE, 64, None, None) == 1         # null sink
    assert lib.pkv_read_probe(FAKE + 8, 64, FAKE, None) == 4     # misaligned
    assert lib.pkv_read_probe(FAKE, 72, FAKE, None) == 2         # not a multiple of 16
    assert "16" in B.pkv_last_error()
