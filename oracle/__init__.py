"""fp64 host oracle for paged-KV-cache store / decode / prefill attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg may import this package.  It wraps
``libpkv_oracle.so`` (plain C, built with gcc, see ``pkv_oracle.c`` for the
arithmetic and the passages of the pages it follows) with numpy marshalling
only.  It imports nothing from the GPU package, and the GPU package imports
nothing from it.

Arrays:
  bf16 data is passed as ``numpy.uint16`` bit patterns; results are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
LIB_PATH = os.path.join(_HERE, "libpkv_oracle.so")

# gcc in ISO C mode with contraction off: every sum is evaluated in source order.
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]

OK, ERR_ARG, ERR_RANGE, ERR_DUPLICATE, ERR_ALLOC = 0, -1, -2, -3, -4


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def build(src: str = _SRC, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc (no HIP, no GPU headers)."""
    cmd = ["gcc", *GCC_FLAGS, *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True, cwd=os.path.dirname(src))
    return out


_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def _bind(lib):
    lib.pko_kv_bytes.restype = ctypes.c_uint64
    lib.pko_kv_bytes.argtypes = [_I32, _I32, _I32, ctypes.c_int64, _I32]
    lib.pko_store.restype = ctypes.c_int
    lib.pko_store.argtypes = [_P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32]
    lib.pko_decode.restype = ctypes.c_int
    lib.pko_decode.argtypes = [_P, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32,
                               ctypes.c_float, _P, ctypes.c_int]
    lib.pko_prefill.restype = ctypes.c_int
    lib.pko_prefill.argtypes = [_P, _P, _P, _I32, _P, _I32, _P, _P, _I32, _I32, _I32, _I32,
                                _I32, ctypes.c_float, _P, ctypes.c_int]
    lib.pko_default_threads.restype = ctypes.c_int
    lib.pko_default_threads.argtypes = []
    lib.pko_copy_blocks.restype = ctypes.c_int
    lib.pko_copy_blocks.argtypes = [_P, _I32, ctypes.c_int64, _I32, _P, _I32]
    lib.pko_rope.restype = ctypes.c_int
    lib.pko_rope.argtypes = [_P, _P, _I32, _I32, _I32, _P, _I32, _P]
    lib.pko_fp8_decode.restype = ctypes.c_double
    lib.pko_fp8_decode.argtypes = [ctypes.c_uint8]
    lib.pko_fp8_encode.restype = ctypes.c_uint8
    lib.pko_fp8_encode.argtypes = [ctypes.c_float]
    lib.pko_store_fp8.restype = ctypes.c_int
    lib.pko_store_fp8.argtypes = [_P, _P, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _I32]
    lib.pko_prefill_fp8.restype = ctypes.c_int
    lib.pko_prefill_fp8.argtypes = [_P, _P, _P, _P, _P, _I32, _P, _I32, _P, _P, _I32, _I32, _I32,
                                    _I32, _I32, ctypes.c_float, _P, ctypes.c_int]
    lib.pko_decode_fp8.restype = ctypes.c_int
    lib.pko_decode_fp8.argtypes = [_P, _P, _P, _P, _P, _I32, _P, _I32, _P, _I32, _I32, _I32, _I32,
                                   _I32, ctypes.c_float, _P]
    return lib


class Oracle:
    """numpy front end over one loaded copy of the oracle library."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            build(out=lib_path)
        self.lib = _bind(ctypes.CDLL(lib_path))

    # -- sizing -----------------------------------------------------------------
    def kv_bytes(self, num_layers, num_kv_heads, head_dim, cached_tokens, bytes_per_element):
        return int(self.lib.pko_kv_bytes(num_layers, num_kv_heads, head_dim, cached_tokens,
                                         bytes_per_element))

    def default_threads(self) -> int:
        return int(self.lib.pko_default_threads())

    # -- store ------------------------------------------------------------------
    def store(self, k, v, slot_mapping, k_cache, v_cache):
        """In place: write k/v ([T][Hkv][d] uint16) into k_cache/v_cache
        ([NB][Hkv][bs][d] uint16) at slot_mapping ([T] int32)."""
        k = _u16(k)
        v = _u16(v)
        slots = _i32(slot_mapping)
        _check_inplace(k_cache, np.uint16)
        _check_inplace(v_cache, np.uint16)
        nb, hkv, bs, d = k_cache.shape
        assert v_cache.shape == k_cache.shape
        t = slots.shape[0]
        assert k.shape == (t, hkv, d) and v.shape == (t, hkv, d)
        rc = self.lib.pko_store(_ptr(k), _ptr(v), _ptr(slots), t, _ptr(k_cache), _ptr(v_cache),
                                nb, hkv, d, bs)
        if rc != OK:
            raise OracleError(rc, "store")

    # -- decode -----------------------------------------------------------------
    def decode(self, q, k_cache, v_cache, block_tables, context_lens, scale, nthreads=0):
        """q [S][Hq][d] uint16 -> out [S][Hq][d] float64."""
        q = _u16(q)
        k_cache = _u16(k_cache)
        v_cache = _u16(v_cache)
        bt = _i32(block_tables)
        ctx = _i32(context_lens)
        nb, hkv, bs, d = k_cache.shape
        s, hq, dq = q.shape
        assert dq == d and v_cache.shape == k_cache.shape
        assert bt.ndim == 2 and bt.shape[0] == s and ctx.shape == (s,)
        out = np.zeros((s, hq, d), dtype=np.float64)
        rc = self.lib.pko_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), nb, _ptr(bt), bt.shape[1],
                                 _ptr(ctx), s, hq, hkv, d, bs, float(np.float32(scale)), _ptr(out),
                                 int(nthreads))
        if rc != OK:
            raise OracleError(rc, "decode")
        return out

    # -- block copy (copy-on-write) ---------------------------------------------------
    def copy_blocks(self, pools, copies):
        """In place: for each (src, dst) row of ``copies`` ([n][2] int32), block
        dst of every pool (contiguous numpy arrays whose first axis is the
        block) becomes a byte copy of block src."""
        pairs = np.ascontiguousarray(np.asarray(copies, dtype=np.int32).reshape(-1, 2))
        if not pools:
            return
        nb = pools[0].shape[0]
        bb = pools[0].nbytes // max(nb, 1)
        for p in pools:
            _check_inplace(p, p.dtype)
            assert p.shape[0] == nb and p.nbytes == nb * bb
        ptrs = (ctypes.c_void_p * len(pools))(*[p.ctypes.data for p in pools])
        rc = self.lib.pko_copy_blocks(ctypes.cast(ptrs, ctypes.c_void_p), len(pools), bb, nb,
                                      _ptr(pairs), pairs.shape[0])
        if rc != OK:
            raise OracleError(rc, "copy_blocks")

    # -- rotary position embedding ------------------------------------------------------
    def rope(self, x, positions, cos_sin):
        """x [n][H][d] uint16 bf16 bits rotated at positions [n] with the fp32
        table cos_sin [P][d] -> new uint16 array."""
        x = _u16(x)
        pos = _i32(positions)
        cs = np.ascontiguousarray(cos_sin, np.float32)
        n, h, d = x.shape
        assert pos.shape == (n,) and cs.ndim == 2 and cs.shape[1] == d
        out = np.empty_like(x)
        rc = self.lib.pko_rope(_ptr(x), _ptr(pos), n, h, d, _ptr(cs), cs.shape[0], _ptr(out))
        if rc != OK:
            raise OracleError(rc, "rope")
        return out

    # -- FP8 (OCP E4M3, one fp32 scale per token and KV head) ------------------------
    def fp8_decode(self, code: int) -> float:
        return float(self.lib.pko_fp8_decode(int(code)))

    def fp8_encode(self, y: float) -> int:
        return int(self.lib.pko_fp8_encode(float(np.float32(y))))

    def store_fp8(self, k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales):
        """In place: quantize k/v ([T][Hkv][d] uint16 bf16 bits) into the codes
        ([NB][Hkv][bs][d] uint8) and scales ([NB][Hkv][bs] float32)."""
        k = _u16(k)
        v = _u16(v)
        slots = _i32(slot_mapping)
        for a, dt in ((k_codes, np.uint8), (v_codes, np.uint8), (k_scales, np.float32),
                      (v_scales, np.float32)):
            _check_inplace(a, dt)
        nb, hkv, bs, d = k_codes.shape
        assert v_codes.shape == k_codes.shape and k_scales.shape == (nb, hkv, bs)
        assert v_scales.shape == k_scales.shape
        t = slots.shape[0]
        assert k.shape == (t, hkv, d) and v.shape == (t, hkv, d)
        rc = self.lib.pko_store_fp8(_ptr(k), _ptr(v), _ptr(slots), t, _ptr(k_codes), _ptr(v_codes),
                                    _ptr(k_scales), _ptr(v_scales), nb, hkv, d, bs)
        if rc != OK:
            raise OracleError(rc, "store_fp8")

    def decode_fp8(self, q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                   scale):
        """q [S][Hq][d] uint16 -> out [S][Hq][d] float64 over the dequantized cache."""
        q = _u16(q)
        k_codes = np.ascontiguousarray(k_codes, np.uint8)
        v_codes = np.ascontiguousarray(v_codes, np.uint8)
        k_scales = np.ascontiguousarray(k_scales, np.float32)
        v_scales = np.ascontiguousarray(v_scales, np.float32)
        bt = _i32(block_tables)
        ctx = _i32(context_lens)
        nb, hkv, bs, d = k_codes.shape
        s, hq, dq = q.shape
        assert dq == d and v_codes.shape == k_codes.shape
        assert bt.ndim == 2 and bt.shape[0] == s and ctx.shape == (s,)
        out = np.zeros((s, hq, d), dtype=np.float64)
        rc = self.lib.pko_decode_fp8(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales),
                                     _ptr(v_scales), nb, _ptr(bt), bt.shape[1], _ptr(ctx), s, hq,
                                     hkv, d, bs, float(np.float32(scale)), _ptr(out))
        if rc != OK:
            raise OracleError(rc, "decode_fp8")
        return out

    def prefill_fp8(self, q, k_codes, v_codes, k_scales, v_scales, block_tables, cu_new_lens,
                    context_lens, scale, nthreads=0):
        """q [total_new][Hq][d] uint16 -> out [total_new][Hq][d] float64 over the
        dequantized FP8 cache (codes uint8 [NB][Hkv][16][d], scales float32
        [NB][Hkv][16])."""
        q = _u16(q)
        k_codes = np.ascontiguousarray(k_codes, np.uint8)
        v_codes = np.ascontiguousarray(v_codes, np.uint8)
        k_scales = np.ascontiguousarray(k_scales, np.float32)
        v_scales = np.ascontiguousarray(v_scales, np.float32)
        bt = _i32(block_tables)
        cu = _i32(cu_new_lens)
        ctx = _i32(context_lens)
        nb, hkv, bs, d = k_codes.shape
        total, hq, dq = q.shape
        s = ctx.shape[0]
        assert dq == d and v_codes.shape == k_codes.shape
        assert k_scales.shape == (nb, hkv, bs) and v_scales.shape == (nb, hkv, bs)
        assert bt.ndim == 2 and bt.shape[0] == s and cu.shape == (s + 1,)
        assert int(cu[-1]) == total
        out = np.zeros((total, hq, d), dtype=np.float64)
        rc = self.lib.pko_prefill_fp8(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales),
                                      _ptr(v_scales), nb, _ptr(bt), bt.shape[1], _ptr(cu),
                                      _ptr(ctx), s, hq, hkv, d, bs, float(np.float32(scale)),
                                      _ptr(out), int(nthreads))
        if rc != OK:
            raise OracleError(rc, "prefill_fp8")
        return out

    # -- prefill ----------------------------------------------------------------
    def prefill(self, q, k_cache, v_cache, block_tables, cu_new_lens, context_lens, scale,
                nthreads=0):
        """q [total_new][Hq][d] uint16 -> out [total_new][Hq][d] float64."""
        q = _u16(q)
        k_cache = _u16(k_cache)
        v_cache = _u16(v_cache)
        bt = _i32(block_tables)
        cu = _i32(cu_new_lens)
        ctx = _i32(context_lens)
        nb, hkv, bs, d = k_cache.shape
        total, hq, dq = q.shape
        s = ctx.shape[0]
        assert dq == d and v_cache.shape == k_cache.shape
        assert bt.ndim == 2 and bt.shape[0] == s and cu.shape == (s + 1,)
        assert int(cu[-1]) == total
        out = np.zeros((total, hq, d), dtype=np.float64)
        rc = self.lib.pko_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), nb, _ptr(bt), bt.shape[1],
                                  _ptr(cu), _ptr(ctx), s, hq, hkv, d, bs, float(np.float32(scale)),
                                  _ptr(out), int(nthreads))
        if rc != OK:
            raise OracleError(rc, "prefill")
        return out


def _u16(a):
    a = np.asarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _check_inplace(a, dtype):
    assert isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous, \
        "in-place oracle buffers must be C-contiguous numpy arrays of the right dtype"


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


_default = None


def get() -> Oracle:
    """The process-wide oracle instance (built on first use if needed)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
