"""ctypes binding of libpkv.so (the C ABI in include/pkv.h).

Argument marshalling only: shape, dtype, device and contiguity checks, then the
C call with raw device pointers and torch's current HIP stream.  Every step of
the computation runs in the library's kernels; there is no fallback.  If the
library is missing, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")
LIB_DEBUG_PATH = os.path.join(HERE, "libpkv_debug.so")

PKV_OK = 0
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_SHAPE", 3: "PKV_ERR_UNSUPPORTED",
                4: "PKV_ERR_ALIGN", 5: "PKV_ERR_WORKSPACE", 6: "PKV_ERR_HIP",
                7: "PKV_ERR_CAPACITY", 8: "PKV_ERR_SEQUENCE", 9: "PKV_ERR_INDEX"}
PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_UNSUPPORTED, PKV_ERR_ALIGN = 1, 2, 3, 4
PKV_ERR_WORKSPACE, PKV_ERR_HIP, PKV_ERR_CAPACITY, PKV_ERR_SEQUENCE = 5, 6, 7, 8
PKV_ERR_INDEX = 9

# every symbol include/pkv.h and include/pkv_pool.h declare
EXPORTED = ["pkv_store", "pkv_decode_partition_tokens", "pkv_decode_workspace_bytes",
            "pkv_decode_attn", "pkv_decode_attn_noalloc", "pkv_decode_noalloc_max_bytes",
            "pkv_store_decode_attn", "pkv_store_decode_attn_rope",
            "pkv_prefill_attn", "pkv_mixed_attn", "pkv_mixed_workspace_bytes", "pkv_store_fp8",
            "pkv_decode_partition_tokens_fp8", "pkv_decode_attn_fp8", "pkv_store_decode_attn_fp8",
            "pkv_prefill_attn_fp8", "pkv_mixed_attn_fp8", "pkv_decode_attn_prefix_fp8",
            "pkv_kv_bytes", "pkv_read_probe",
            "pkv_status_string", "pkv_last_error",
            "pkv_pool_create", "pkv_pool_destroy", "pkv_pool_add_seq", "pkv_pool_append",
            "pkv_pool_fork", "pkv_pool_free_seq", "pkv_pool_block_tables", "pkv_pool_num_free",
            "pkv_pool_refcount", "pkv_pool_seq_len", "pkv_copy_blocks",
            "pkv_decode_attn_prefix", "pkv_decode_prefix_workspace_bytes", "pkv_prefix_groups",
            "pkv_check_tables", "pkv_debug_bounds_enabled", "pkv_debug_status"]


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what} failed: {STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


class PkvCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32)]


class PkvCacheFp8(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32)]


_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_lib_handle = None


def load(path: str = LIB_PATH):
    """Load libpkv.so once; raise if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    _lib_handle = _open(path)
    return _lib_handle


def load_debug(path: str = LIB_DEBUG_PATH):
    """A separate handle on libpkv_debug.so, the debug-bounds build (its
    kernels also record the first out-of-range index they clamp; read it with
    pkv_debug_status).  Use it through ``using_library``."""
    return _open(path)


@contextlib.contextmanager
def using_library(lib):
    """Route this module's calls to ``lib`` (e.g. load_debug()) inside the block."""
    global _lib_handle
    old = _lib_handle
    _lib_handle = lib
    try:
        yield lib
    finally:
        _lib_handle = old


def pkv_debug_status(clear: bool = True):
    """(kind, value, where, reports) of the first out-of-range index the
    kernels of the loaded debug-bounds library recorded; kind 0 = none.
    Waits for the device."""
    out = (ctypes.c_uint32 * 4)()
    _check(load().pkv_debug_status(out, int(bool(clear))), "pkv_debug_status")
    return (int(out[0]), ctypes.c_int32(out[1]).value, ctypes.c_int32(out[2]).value, int(out[3]))


def _open(path: str):
    # torch first: its HIP runtime (same soname as ROCm's) must be the one the
    # process loads, so that libpkv launches on the runtime that owns torch's
    # memory and streams.  Loading libpkv first pulls in a second copy.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_pools_amd.build`"
                           " (the HIP library is the only implementation; there is no fallback)")
    lib = ctypes.CDLL(path)
    lib.pkv_store.restype = ctypes.c_int
    lib.pkv_store.argtypes = [_P, _P, _P, _I32, PkvCache, _P]
    lib.pkv_decode_partition_tokens.restype = _I32
    lib.pkv_decode_partition_tokens.argtypes = [_I32, _I32, _I32]
    lib.pkv_decode_partition_tokens_fp8.restype = _I32
    lib.pkv_decode_partition_tokens_fp8.argtypes = [_I32, _I32, _I32]
    lib.pkv_decode_workspace_bytes.restype = _SZ
    lib.pkv_decode_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
    lib.pkv_decode_attn.restype = ctypes.c_int
    lib.pkv_decode_attn.argtypes = [_P, PkvCache, _P, _I32, _P, _I32, _I32, _I32, ctypes.c_float,
                                    _P, _P, _SZ, _I32, _P]
    lib.pkv_store_decode_attn.restype = ctypes.c_int
    lib.pkv_decode_attn_noalloc.restype = ctypes.c_int
    lib.pkv_decode_attn_noalloc.argtypes = [_P, PkvCache, _P, _I32, _P, _I32, _I32, _I32,
                                            ctypes.c_float, _P, _I32, _P]
    lib.pkv_decode_noalloc_max_bytes.restype = _SZ
    lib.pkv_decode_noalloc_max_bytes.argtypes = []
    lib.pkv_store_decode_attn.argtypes = [_P, _P, _P, _P, PkvCache, _P, _I32, _P, _I32, _I32, _I32,
                                          ctypes.c_float, _P, _P, _SZ, _I32, _P]
    lib.pkv_store_decode_attn_rope.restype = ctypes.c_int
    lib.pkv_store_decode_attn_rope.argtypes = [_P, _P, _P, _P, _P, _I32, PkvCache, _P, _I32, _P,
                                               _I32, _I32, _I32, ctypes.c_float, _P, _P, _SZ,
                                               _I32, _P]
    lib.pkv_store_fp8.restype = ctypes.c_int
    lib.pkv_store_fp8.argtypes = [_P, _P, _P, _I32, PkvCacheFp8, _P]
    lib.pkv_decode_attn_fp8.restype = ctypes.c_int
    lib.pkv_decode_attn_fp8.argtypes = [_P, PkvCacheFp8, _P, _I32, _P, _I32, _I32, _I32,
                                        ctypes.c_float, _P, _P, _SZ, _I32, _P]
    lib.pkv_store_decode_attn_fp8.restype = ctypes.c_int
    lib.pkv_store_decode_attn_fp8.argtypes = [_P, _P, _P, _P, PkvCacheFp8, _P, _I32, _P, _I32,
                                              _I32, _I32, ctypes.c_float, _P, _P, _SZ, _I32, _P]
    lib.pkv_prefill_attn.restype = ctypes.c_int
    lib.pkv_prefill_attn.argtypes = [_P, PkvCache, _P, _I32, _P, _P, _I32, _I32, _I32, _I32,
                                     ctypes.c_float, _P, _P]
    lib.pkv_prefill_attn_fp8.restype = ctypes.c_int
    lib.pkv_prefill_attn_fp8.argtypes = [_P, PkvCacheFp8, _P, _I32, _P, _P, _I32, _I32, _I32, _I32,
                                         ctypes.c_float, _P, _P]
    lib.pkv_pool_create.restype = ctypes.c_int
    lib.pkv_pool_create.argtypes = [_I32, _I32, _I32, ctypes.POINTER(ctypes.c_void_p)]
    lib.pkv_pool_destroy.restype = None
    lib.pkv_pool_destroy.argtypes = [_P]
    lib.pkv_pool_add_seq.restype = ctypes.c_int
    lib.pkv_pool_add_seq.argtypes = [_P, _I64, _P, _I32, _P, _P]
    lib.pkv_pool_append.restype = ctypes.c_int
    lib.pkv_pool_append.argtypes = [_P, _P, _P, _I32, _P, _P, _P, _P]
    lib.pkv_pool_fork.restype = ctypes.c_int
    lib.pkv_pool_fork.argtypes = [_P, _I64, _I64]
    lib.pkv_pool_free_seq.restype = ctypes.c_int
    lib.pkv_pool_free_seq.argtypes = [_P, _I64]
    lib.pkv_pool_block_tables.restype = ctypes.c_int
    lib.pkv_pool_block_tables.argtypes = [_P, _P, _I32, _I32, _P, _P]
    lib.pkv_pool_num_free.restype = _I32
    lib.pkv_pool_num_free.argtypes = [_P]
    lib.pkv_pool_refcount.restype = _I32
    lib.pkv_pool_refcount.argtypes = [_P, _I32]
    lib.pkv_pool_seq_len.restype = _I32
    lib.pkv_pool_seq_len.argtypes = [_P, _I64]
    lib.pkv_copy_blocks.restype = ctypes.c_int
    lib.pkv_copy_blocks.argtypes = [_P, _I32, _SZ, _I32, _P, _I32, _P]
    lib.pkv_read_probe.restype = ctypes.c_int
    lib.pkv_read_probe.argtypes = [_P, _SZ, _P, _P]
    lib.pkv_mixed_attn.restype = ctypes.c_int
    lib.pkv_mixed_attn.argtypes = [_P, PkvCache, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                   ctypes.c_float, _P, _P, _SZ, _P]
    lib.pkv_mixed_attn_fp8.restype = ctypes.c_int
    lib.pkv_mixed_attn_fp8.argtypes = [_P, PkvCacheFp8, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                   ctypes.c_float, _P, _P, _SZ, _P]
    lib.pkv_mixed_workspace_bytes.restype = _SZ
    lib.pkv_mixed_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32, _I32]
    lib.pkv_decode_attn_prefix.restype = ctypes.c_int
    lib.pkv_decode_attn_prefix.argtypes = [_P, PkvCache, _P, _I32, _P, _I32, _I32, _I32,
                                           ctypes.c_float, _P, _P, _I32, _I32, _P, _P, _SZ, _I32,
                                           _P]
    lib.pkv_decode_attn_prefix_fp8.restype = ctypes.c_int
    lib.pkv_decode_attn_prefix_fp8.argtypes = [_P, PkvCacheFp8, _P, _I32, _P, _I32, _I32, _I32,
                                               ctypes.c_float, _P, _P, _I32, _I32, _P, _P, _SZ,
                                               _I32, _P]
    lib.pkv_decode_prefix_workspace_bytes.restype = _SZ
    lib.pkv_decode_prefix_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32]
    lib.pkv_prefix_groups.restype = ctypes.c_int
    lib.pkv_prefix_groups.argtypes = [_P, _I32, _P, _I32, _I32, _P, _P, _P, _P]
    lib.pkv_kv_bytes.restype = ctypes.c_uint64
    lib.pkv_debug_bounds_enabled.restype = ctypes.c_int
    lib.pkv_debug_bounds_enabled.argtypes = []
    lib.pkv_debug_status.restype = ctypes.c_int
    lib.pkv_debug_status.argtypes = [_P, ctypes.c_int]
    lib.pkv_check_tables.restype = ctypes.c_int
    lib.pkv_check_tables.argtypes = [_P, _I32, _P, _I32, _I32, _P, _I32, _I32, _P, _P]
    lib.pkv_kv_bytes.argtypes = [_I32, _I32, _I32, _I64, _I32]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    return lib


def _check(status: int, what: str):
    if status != PKV_OK:
        detail = load().pkv_last_error().decode()
        raise PkvError(status, what, detail)


def _stream(t, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, ndim=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _cache(k_cache, v_cache) -> PkvCache:
    import torch

    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError(f"k_cache {tuple(k_cache.shape)} and v_cache {tuple(v_cache.shape)} differ")
    nb, hkv, bs, d = k_cache.shape
    return PkvCache(k_cache.data_ptr(), v_cache.data_ptr(), nb, hkv, d, bs)


def _cache_fp8(k_codes, v_codes, k_scale, v_scale) -> PkvCacheFp8:
    import torch

    _need(k_codes, "k_codes", torch.uint8, 4)
    _need(v_codes, "v_codes", torch.uint8, 4)
    _need(k_scale, "k_scale", torch.float32, 3)
    _need(v_scale, "v_scale", torch.float32, 3)
    if k_codes.shape != v_codes.shape or k_scale.shape != v_scale.shape or \
            tuple(k_scale.shape) != tuple(k_codes.shape[:3]):
        raise ValueError(f"codes {tuple(k_codes.shape)} / {tuple(v_codes.shape)} and scales "
                         f"{tuple(k_scale.shape)} / {tuple(v_scale.shape)} do not match")
    nb, hkv, bs, d = k_codes.shape
    return PkvCacheFp8(k_codes.data_ptr(), v_codes.data_ptr(), k_scale.data_ptr(),
                       v_scale.data_ptr(), nb, hkv, d, bs)


# ---------------------------------------------------------------------------
# the calls
# ---------------------------------------------------------------------------

def pkv_store(k, v, slot_mapping, k_cache, v_cache, stream=None):
    """Scatter k/v ([T][Hkv][d] bf16) into the pools at slot_mapping ([T] int32)."""
    import torch

    lib = load()
    cache = _cache(k_cache, v_cache)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    t = slot_mapping.shape[0]
    want = (t, cache.num_kv_heads, cache.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k/v must be {want}, got {tuple(k.shape)} / {tuple(v.shape)}")
    _check(lib.pkv_store(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), t, cache,
                         _stream(k_cache, stream)), "pkv_store")


def pkv_decode_partition_tokens(num_seqs, num_kv_heads, max_context_len) -> int:
    return int(load().pkv_decode_partition_tokens(num_seqs, num_kv_heads, max_context_len))


def pkv_decode_partition_tokens_fp8(num_seqs, num_kv_heads, max_context_len) -> int:
    return int(load().pkv_decode_partition_tokens_fp8(num_seqs, num_kv_heads, max_context_len))


def pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                               partition_tokens=0) -> int:
    return int(load().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                                 partition_tokens))


def pkv_decode_attn(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                    max_context_len: Optional[int] = None, workspace=None, partition_tokens: int = 0,
                    stream=None):
    """out[s][h] = softmax(scale q[s][h] K^T) V over each sequence's paged cache.

    q, out: [S][Hq][d] bf16; block_tables [S][max_blocks] int32; context_lens [S]
    int32 (after the store).  ``max_context_len`` defaults to
    ``max_blocks * 16`` (no host sync); pass the true maximum to size the grid
    tightly.  ``workspace``: uint8 device tensor, allocated here when None.
    """
    import torch

    lib = load()
    cache = _cache(k_cache, v_cache)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables / context_lens do not match q's sequence count")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * cache.block_size
    p = partition_tokens or pkv_decode_partition_tokens(s, cache.num_kv_heads, max_context_len)
    need = pkv_decode_workspace_bytes(s, hq, d, max_context_len, p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_decode_attn(q.data_ptr(), cache, block_tables.data_ptr(), max_blocks,
                               context_lens.data_ptr(), s, int(max_context_len), hq,
                               float(scale), out.data_ptr(), workspace.data_ptr(),
                               workspace.numel(), int(p), _stream(q, stream)),
           "pkv_decode_attn")
    return out


def pkv_decode_attn_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                            max_context_len: Optional[int] = None, partition_tokens: int = 0,
                            stream=None):
    """pkv_decode_attn without a workspace: the split-KV partials go to the
    library's own per-GPU scratch, so nothing is allocated here or in the
    library.  Raises PkvError (PKV_ERR_WORKSPACE) when the split needs more
    than pkv_decode_noalloc_max_bytes()."""
    import torch

    lib = load()
    cache = _cache(k_cache, v_cache)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables / context_lens do not match q's sequence count")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * cache.block_size
    _check(lib.pkv_decode_attn_noalloc(q.data_ptr(), cache, block_tables.data_ptr(), max_blocks,
                                       context_lens.data_ptr(), s, int(max_context_len), hq,
                                       float(scale), out.data_ptr(), int(partition_tokens),
                                       _stream(q, stream)),
           "pkv_decode_attn_noalloc")
    return out


def pkv_decode_noalloc_max_bytes() -> int:
    return int(load().pkv_decode_noalloc_max_bytes())


def pkv_store_decode_attn(k, v, slot_mapping, q, k_cache, v_cache, block_tables, context_lens,
                          scale, out, max_context_len: Optional[int] = None, workspace=None,
                          partition_tokens: int = 0, stream=None):
    """pkv_store then pkv_decode_attn in one launch: k/v [S][Hkv][d] bf16 (one
    new token per sequence), slot_mapping [S] int32; the rest as for
    pkv_decode_attn."""
    import torch

    lib = load()
    cache = _cache(k_cache, v_cache)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    want = (s, cache.num_kv_heads, cache.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want or slot_mapping.shape[0] != s:
        raise ValueError(f"k/v must be {want} and slot_mapping [{s}], got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}, {tuple(slot_mapping.shape)}")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables / context_lens do not match q's sequence count")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * cache.block_size
    p = partition_tokens or pkv_decode_partition_tokens(s, cache.num_kv_heads, max_context_len)
    need = pkv_decode_workspace_bytes(s, hq, d, max_context_len, p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_store_decode_attn(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                     q.data_ptr(), cache, block_tables.data_ptr(), max_blocks,
                                     context_lens.data_ptr(), s, int(max_context_len), hq,
                                     float(scale), out.data_ptr(), workspace.data_ptr(),
                                     workspace.numel(), int(p), _stream(q, stream)),
           "pkv_store_decode_attn")
    return out


def pkv_store_decode_attn_rope(k, v, slot_mapping, q, cos_sin, k_cache, v_cache, block_tables,
                               context_lens, scale, out, max_context_len: Optional[int] = None,
                               workspace=None, partition_tokens: int = 0, stream=None):
    """pkv_store_decode_attn with q and the new k rotated at each sequence's
    last position by the fp32 table cos_sin [P][d] (cos, then sin)."""
    import torch

    lib = load()
    cache = _cache(k_cache, v_cache)
    for t, name, dt, nd in ((q, "q", torch.bfloat16, 3), (out, "out", torch.bfloat16, 3),
                            (k, "k", torch.bfloat16, 3), (v, "v", torch.bfloat16, 3),
                            (slot_mapping, "slot_mapping", torch.int32, 1),
                            (cos_sin, "cos_sin", torch.float32, 2),
                            (block_tables, "block_tables", torch.int32, 2),
                            (context_lens, "context_lens", torch.int32, 1)):
        _need(t, name, dt, nd)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d != cache.head_dim or cos_sin.shape[1] != d:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, cos_sin "
                         f"{tuple(cos_sin.shape)}, head_dim {cache.head_dim}")
    want = (s, cache.num_kv_heads, cache.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want or slot_mapping.shape[0] != s:
        raise ValueError(f"k/v must be {want} and slot_mapping [{s}]")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables / context_lens do not match q's sequence count")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * cache.block_size
    p = partition_tokens or pkv_decode_partition_tokens(s, cache.num_kv_heads, max_context_len)
    need = pkv_decode_workspace_bytes(s, hq, d, max_context_len, p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_store_decode_attn_rope(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                          q.data_ptr(), cos_sin.data_ptr(), cos_sin.shape[0],
                                          cache, block_tables.data_ptr(), max_blocks,
                                          context_lens.data_ptr(), s, int(max_context_len), hq,
                                          float(scale), out.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), int(p), _stream(q, stream)),
           "pkv_store_decode_attn_rope")
    return out


def pkv_prefill_attn(q, k_cache, v_cache, block_tables, cu_new_lens, context_lens, scale, out,
                     max_new_len: int, max_context_len: int, stream=None):
    """Chunked causal prefill: q/out [total_new][Hq][d] bf16, prompts packed
    by cu_new_lens ([S+1] int32); context_lens [S] int32 include the new tokens."""
    import torch

    lib = load()
    cache = _cache(k_cache, v_cache)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(cu_new_lens, "cu_new_lens", torch.int32, 1)
    _need(context_lens, "context_lens", torch.int32, 1)
    total, hq, d = q.shape
    s = context_lens.shape[0]
    if tuple(out.shape) != (total, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    if cu_new_lens.shape[0] != s + 1 or block_tables.shape[0] != s:
        raise ValueError("cu_new_lens / block_tables do not match context_lens")
    _check(lib.pkv_prefill_attn(q.data_ptr(), cache, block_tables.data_ptr(), block_tables.shape[1],
                                cu_new_lens.data_ptr(), context_lens.data_ptr(), s,
                                int(max_new_len), int(max_context_len), hq, float(scale),
                                out.data_ptr(), _stream(q, stream)),
           "pkv_prefill_attn")
    return out


def pkv_mixed_workspace_bytes(num_seqs: int, num_decode: int, max_new_len: int,
                              max_context_len: int, num_q_heads: int, num_kv_heads: int,
                              head_dim: int) -> int:
    return int(load().pkv_mixed_workspace_bytes(num_seqs, num_decode, max_new_len,
                                                max_context_len, num_q_heads, num_kv_heads,
                                                head_dim))


def pkv_mixed_attn(q, k_cache, v_cache, block_tables, cu_new_lens, context_lens, num_decode: int,
                   scale, out, max_new_len: int, max_context_len: int, workspace=None,
                   split: bool = True, stream=None):
    """One continuous-batching iteration: sequences 0 .. num_decode-1 are decode
    sequences (one new token each), the rest prefill chunks; tensors as for
    pkv_prefill_attn.  ``workspace``: a uint8 device tensor of at least
    pkv_mixed_workspace_bytes (any contents); None allocates one when
    ``split`` and the sizes call for it, ``split=False`` passes none."""
    return _mixed("pkv_mixed_attn", _cache(k_cache, v_cache), q, block_tables, cu_new_lens,
                  context_lens, num_decode, scale, out, max_new_len, max_context_len, workspace,
                  split, stream)


def pkv_mixed_attn_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, cu_new_lens,
                       context_lens, num_decode: int, scale, out, max_new_len: int,
                       max_context_len: int, workspace=None, split: bool = True, stream=None):
    """pkv_mixed_attn over an FP8 cache (see pkv_store_fp8 for its layout)."""
    return _mixed("pkv_mixed_attn_fp8", _cache_fp8(k_codes, v_codes, k_scale, v_scale), q,
                  block_tables, cu_new_lens, context_lens, num_decode, scale, out, max_new_len,
                  max_context_len, workspace, split, stream)


def _mixed(name, cache, q, block_tables, cu_new_lens, context_lens, num_decode, scale, out,
           max_new_len, max_context_len, workspace, split, stream):
    import torch

    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(cu_new_lens, "cu_new_lens", torch.int32, 1)
    _need(context_lens, "context_lens", torch.int32, 1)
    total, hq, d = q.shape
    s = context_lens.shape[0]
    if tuple(out.shape) != (total, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    if cu_new_lens.shape[0] != s + 1 or block_tables.shape[0] != s:
        raise ValueError("cu_new_lens / block_tables do not match context_lens")
    ws_ptr, ws_bytes = None, 0
    if split:
        if workspace is None:
            need = pkv_mixed_workspace_bytes(s, int(num_decode), int(max_new_len),
                                             int(max_context_len), hq, cache.num_kv_heads, d)
            if need > 0:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            _need(workspace, "workspace", torch.uint8, 1)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    _check(getattr(lib, name)(q.data_ptr(), cache, block_tables.data_ptr(), block_tables.shape[1],
                              cu_new_lens.data_ptr(), context_lens.data_ptr(), int(num_decode), s,
                              int(max_new_len), int(max_context_len), hq, float(scale),
                              out.data_ptr(), ws_ptr, ws_bytes, _stream(q, stream)),
           name)
    return out


def pkv_decode_prefix_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                      head_dim: int, max_context_len: int,
                                      partition_tokens: int = 0) -> int:
    return int(load().pkv_decode_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                        head_dim, max_context_len,
                                                        partition_tokens))


def pkv_prefix_groups(block_tables, context_lens, min_prefix_tokens: int = 16):
    """Groups of consecutive sequences that share leading blocks, from host
    (numpy int32) block tables [S][max_blocks] and context lengths [S]:
    returns (group_starts [G+1], prefix_lens [G], max_group_size)."""
    import numpy as np

    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.ndim != 2 or ctx.ndim != 1 or bt.shape[0] != ctx.shape[0]:
        raise ValueError(f"block_tables {bt.shape} / context_lens {ctx.shape}")
    s = ctx.shape[0]
    starts = np.zeros(s + 1, dtype=np.int32)
    plens = np.zeros(max(s, 1), dtype=np.int32)
    ng, mg = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().pkv_prefix_groups(_np_ptr(bt), bt.shape[1], _np_ptr(ctx), s,
                                    int(min_prefix_tokens), _np_ptr(starts), _np_ptr(plens),
                                    ctypes.byref(ng), ctypes.byref(mg)), "pkv_prefix_groups")
    return starts[: ng.value + 1].copy(), plens[: ng.value].copy(), mg.value


def pkv_check_tables(block_tables, context_lens, num_blocks: int, slot_mapping=None,
                     max_context_len: int = -1):
    """Check a call's indices on host (numpy int32) copies: block_tables
    [S][max_blocks], context_lens [S], optional slot_mapping [T].  Returns
    None when every context, reached block id and slot is in range and no slot
    repeats; raises PkvError (PKV_ERR_INDEX) naming the first violation
    otherwise, with ``bad_seq`` / ``bad_index`` set on the exception."""
    import numpy as np

    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if bt.ndim != 2 or ctx.ndim != 1 or bt.shape[0] != ctx.shape[0]:
        raise ValueError(f"block_tables {bt.shape} / context_lens {ctx.shape}")
    slots = (np.zeros(1, np.int32) if slot_mapping is None
             else np.ascontiguousarray(slot_mapping, dtype=np.int32))
    t = 0 if slot_mapping is None else slots.shape[0]
    bs, bi = ctypes.c_int32(-1), ctypes.c_int32(-1)
    lib = load()
    st = lib.pkv_check_tables(_np_ptr(bt), bt.shape[1], _np_ptr(ctx), ctx.shape[0],
                              int(max_context_len), _np_ptr(slots), t, int(num_blocks),
                              ctypes.byref(bs), ctypes.byref(bi))
    if st != 0:
        err = PkvError(st, "pkv_check_tables", lib.pkv_last_error().decode())
        err.bad_seq, err.bad_index = bs.value, bi.value
        raise err


def pkv_decode_attn_prefix(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                           group_starts, prefix_lens, max_group_size: int,
                           max_context_len: Optional[int] = None, workspace=None,
                           partition_tokens: int = 0, stream=None):
    """pkv_decode_attn for a batch whose consecutive-sequence groups share
    prefix blocks: group_starts [G+1] and prefix_lens [G] are int32 device
    tensors (see pkv_prefix_groups), ``max_group_size`` a host int bounding
    the sizes of groups with a prefix; other tensors as for pkv_decode_attn.
    ``workspace``: uint8 device tensor, allocated here when None."""
    return _prefix("pkv_decode_attn_prefix", _cache(k_cache, v_cache), q, block_tables,
                   context_lens, scale, out, group_starts, prefix_lens, max_group_size,
                   max_context_len, workspace, partition_tokens, stream)


def pkv_decode_attn_prefix_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables,
                               context_lens, scale, out, group_starts, prefix_lens,
                               max_group_size: int, max_context_len: Optional[int] = None,
                               workspace=None, partition_tokens: int = 0, stream=None):
    """pkv_decode_attn_prefix over an FP8 cache (see pkv_store_fp8 for its layout)."""
    return _prefix("pkv_decode_attn_prefix_fp8", _cache_fp8(k_codes, v_codes, k_scale, v_scale),
                   q, block_tables, context_lens, scale, out, group_starts, prefix_lens,
                   max_group_size, max_context_len, workspace, partition_tokens, stream)


def _prefix(name, cache, q, block_tables, context_lens, scale, out, group_starts, prefix_lens,
            max_group_size, max_context_len, workspace, partition_tokens, stream):
    import torch

    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    _need(group_starts, "group_starts", torch.int32, 1)
    _need(prefix_lens, "prefix_lens", torch.int32, 1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables / context_lens do not match q's sequence count")
    ng = prefix_lens.shape[0]
    if group_starts.shape[0] != ng + 1:
        raise ValueError(f"group_starts has {group_starts.shape[0]} entries, {ng + 1} expected")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * cache.block_size
    if workspace is None:
        need = pkv_decode_prefix_workspace_bytes(s, hq, cache.num_kv_heads, d,
                                                 int(max_context_len), int(partition_tokens))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(getattr(lib, name)(q.data_ptr(), cache, block_tables.data_ptr(), max_blocks,
                              context_lens.data_ptr(), s, int(max_context_len), hq, float(scale),
                              group_starts.data_ptr(), prefix_lens.data_ptr(), ng,
                              int(max_group_size), out.data_ptr(), workspace.data_ptr(),
                              workspace.numel(), int(partition_tokens), _stream(q, stream)),
           name)
    return out


def pkv_store_fp8(k, v, slot_mapping, k_codes, v_codes, k_scale, v_scale, stream=None):
    """Quantize k/v ([T][Hkv][d] bf16) into an FP8 cache (E4M3 codes uint8
    [NB][Hkv][16][d], fp32 scales [NB][Hkv][16]) at slot_mapping ([T] int32)."""
    import torch

    lib = load()
    cache = _cache_fp8(k_codes, v_codes, k_scale, v_scale)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    t = slot_mapping.shape[0]
    want = (t, cache.num_kv_heads, cache.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want:
        raise ValueError(f"k/v must be {want}, got {tuple(k.shape)} / {tuple(v.shape)}")
    _check(lib.pkv_store_fp8(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), t, cache,
                             _stream(k_codes, stream)), "pkv_store_fp8")


def pkv_prefill_attn_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, cu_new_lens,
                         context_lens, scale, out, max_new_len: int, max_context_len: int,
                         stream=None):
    """pkv_prefill_attn over an FP8 cache (see pkv_store_fp8 for its layout)."""
    import torch

    lib = load()
    cache = _cache_fp8(k_codes, v_codes, k_scale, v_scale)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(cu_new_lens, "cu_new_lens", torch.int32, 1)
    _need(context_lens, "context_lens", torch.int32, 1)
    total, hq, d = q.shape
    s = context_lens.shape[0]
    if tuple(out.shape) != (total, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    if cu_new_lens.shape[0] != s + 1 or block_tables.shape[0] != s:
        raise ValueError("cu_new_lens / block_tables do not match context_lens")
    _check(lib.pkv_prefill_attn_fp8(q.data_ptr(), cache, block_tables.data_ptr(),
                                    block_tables.shape[1], cu_new_lens.data_ptr(),
                                    context_lens.data_ptr(), s, int(max_new_len),
                                    int(max_context_len), hq, float(scale), out.data_ptr(),
                                    _stream(q, stream)),
           "pkv_prefill_attn_fp8")
    return out


def pkv_decode_attn_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, scale,
                        out, max_context_len: Optional[int] = None, workspace=None,
                        partition_tokens: int = 0, stream=None):
    """pkv_decode_attn over an FP8 cache (see pkv_store_fp8 for its layout)."""
    import torch

    lib = load()
    cache = _cache_fp8(k_codes, v_codes, k_scale, v_scale)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables / context_lens do not match q's sequence count")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * cache.block_size
    p = partition_tokens or pkv_decode_partition_tokens_fp8(s, cache.num_kv_heads,
                                                            max_context_len)
    need = pkv_decode_workspace_bytes(s, hq, d, max_context_len, p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_decode_attn_fp8(q.data_ptr(), cache, block_tables.data_ptr(), max_blocks,
                                   context_lens.data_ptr(), s, int(max_context_len), hq,
                                   float(scale), out.data_ptr(), workspace.data_ptr(),
                                   workspace.numel(), int(p), _stream(q, stream)),
           "pkv_decode_attn_fp8")
    return out


def pkv_store_decode_attn_fp8(k, v, slot_mapping, q, k_codes, v_codes, k_scale, v_scale,
                              block_tables, context_lens, scale, out,
                              max_context_len: Optional[int] = None, workspace=None,
                              partition_tokens: int = 0, stream=None):
    """pkv_store_fp8 then pkv_decode_attn_fp8 in one launch: k/v [S][Hkv][d]
    bf16 (one new token per sequence), slot_mapping [S] int32; the rest as for
    pkv_decode_attn_fp8."""
    import torch

    lib = load()
    cache = _cache_fp8(k_codes, v_codes, k_scale, v_scale)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d != cache.head_dim:
        raise ValueError(f"q {tuple(q.shape)}, out {tuple(out.shape)}, head_dim {cache.head_dim}")
    want = (s, cache.num_kv_heads, cache.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want or slot_mapping.shape[0] != s:
        raise ValueError(f"k/v must be {want} and slot_mapping [{s}], got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}, {tuple(slot_mapping.shape)}")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("block_tables / context_lens do not match q's sequence count")
    max_blocks = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = max_blocks * cache.block_size
    p = partition_tokens or pkv_decode_partition_tokens_fp8(s, cache.num_kv_heads,
                                                            max_context_len)
    need = pkv_decode_workspace_bytes(s, hq, d, max_context_len, p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_store_decode_attn_fp8(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                         q.data_ptr(), cache, block_tables.data_ptr(),
                                         max_blocks, context_lens.data_ptr(), s,
                                         int(max_context_len), hq, float(scale), out.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(), int(p),
                                         _stream(q, stream)),
           "pkv_store_decode_attn_fp8")
    return out


def pkv_kv_bytes(layers, kv_heads, head_dim, tokens, bytes_per_elem) -> int:
    return int(load().pkv_kv_bytes(layers, kv_heads, head_dim, tokens, bytes_per_elem))


def pkv_status_string(status: int) -> str:
    return load().pkv_status_string(status).decode()


def pkv_last_error() -> str:
    return load().pkv_last_error().decode()


# ---------------------------------------------------------------------------
# block pool (host) and block copy (device)
# ---------------------------------------------------------------------------

def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


class BlockPool:
    """The C++ block pool (include/pkv_pool.h): marshalling only.

    Host-side numpy int32/int64 arrays in and out; every rule lives in the
    library."""

    def __init__(self, num_blocks: int, block_size: int = 16, prefix_caching: bool = False):
        self._lib = load()
        h = ctypes.c_void_p()
        _check(self._lib.pkv_pool_create(num_blocks, block_size, int(bool(prefix_caching)),
                                         ctypes.byref(h)), "pkv_pool_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_seq(self, seq_id: int, tokens):
        """Admit a prompt -> (slots int32 [n], -1 where cached; num_cached)."""
        import numpy as np

        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(tok.shape[0], np.int32)
        cached = ctypes.c_int32(0)
        _check(self._lib.pkv_pool_add_seq(self._h, int(seq_id), _np_ptr(tok), tok.shape[0],
                                          _np_ptr(slots), ctypes.byref(cached)),
               "pkv_pool_add_seq")
        return slots, cached.value

    def append(self, seq_ids, tokens):
        """One token per sequence -> (slots int32 [n], copies int32 [k][2]).
        On failure the PkvError carries .num_done."""
        import numpy as np

        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        if ids.shape != tok.shape:
            raise ValueError("seq_ids and tokens differ in length")
        n = ids.shape[0]
        slots = np.empty(n, np.int32)
        copies = np.empty((max(n, 1), 2), np.int32)
        ncopies, done = ctypes.c_int32(0), ctypes.c_int32(0)
        st = self._lib.pkv_pool_append(self._h, _np_ptr(ids), _np_ptr(tok), n, _np_ptr(slots),
                                       _np_ptr(copies), ctypes.byref(ncopies), ctypes.byref(done))
        if st != PKV_OK:
            err = PkvError(st, "pkv_pool_append", self._lib.pkv_last_error().decode())
            err.num_done = done.value
            err.slots = slots[:done.value].copy()
            err.copies = copies[:ncopies.value].copy()
            raise err
        return slots, copies[:ncopies.value].copy()

    def fork(self, parent_id: int, child_id: int):
        _check(self._lib.pkv_pool_fork(self._h, int(parent_id), int(child_id)), "pkv_pool_fork")

    def free_seq(self, seq_id: int):
        _check(self._lib.pkv_pool_free_seq(self._h, int(seq_id)), "pkv_pool_free_seq")

    def block_tables(self, seq_ids, max_blocks_per_seq: int):
        """-> (block_tables int32 [n][max_blocks_per_seq] padded with -1,
        context_lens int32 [n])."""
        import numpy as np

        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        bt = np.empty((n, max_blocks_per_seq), np.int32)
        ctx = np.empty(n, np.int32)
        _check(self._lib.pkv_pool_block_tables(self._h, _np_ptr(ids), n, max_blocks_per_seq,
                                               _np_ptr(bt), _np_ptr(ctx)), "pkv_pool_block_tables")
        return bt, ctx

    def block_table(self, seq_id: int):
        n = self.seq_len(seq_id)
        if n < 0:
            raise PkvError(PKV_ERR_SEQUENCE, "block_table", f"unknown sequence {seq_id}")
        bt, _ = self.block_tables([seq_id], max(1, -(-n // self.block_size)))
        return [int(b) for b in bt[0] if b >= 0]

    def num_free(self) -> int:
        return self._lib.pkv_pool_num_free(self._h)

    def refcount(self, block: int) -> int:
        return self._lib.pkv_pool_refcount(self._h, block)

    def seq_len(self, seq_id: int) -> int:
        return self._lib.pkv_pool_seq_len(self._h, int(seq_id))


def pkv_copy_blocks(pools, copies, stream=None):
    """Block dst of every pool becomes a copy of block src, for each (src, dst)
    row of ``copies`` (int32 [k][2] on the device).  ``pools``: device tensors
    whose first axis is the block (a layer's K or V cache, FP8 codes or
    scales), all with the same bytes per block."""
    import torch

    lib = load()
    if len(pools) == 0 or copies.numel() == 0:
        return
    _need(copies, "copies", torch.int32, 2)
    if copies.shape[1] != 2:
        raise ValueError("copies must be [k][2]")
    nb = pools[0].shape[0]
    bb = pools[0].numel() * pools[0].element_size() // max(nb, 1)
    for i, p in enumerate(pools):
        if not isinstance(p, torch.Tensor) or not p.is_cuda or not p.is_contiguous():
            raise TypeError(f"pools[{i}] must be a contiguous device tensor")
        if p.shape[0] != nb or p.numel() * p.element_size() != nb * bb:
            raise ValueError(f"pools[{i}]: every pool must have {nb} blocks of {bb} bytes")
    ptrs = (ctypes.c_void_p * len(pools))(*[p.data_ptr() for p in pools])
    _check(lib.pkv_copy_blocks(ctypes.cast(ptrs, ctypes.c_void_p), len(pools), bb, nb,
                               copies.data_ptr(), copies.shape[0], _stream(copies, stream)),
           "pkv_copy_blocks")


def pkv_read_probe(buf, sink, stream=None):
    """Stream every byte of the contiguous device tensor ``buf`` through one
    read kernel (a measurement aid: the HBM read rate of this GPU).  ``sink``:
    a device tensor of at least 4 bytes that the kernel may write."""
    lib = load()
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda:
        raise TypeError("buf and sink must be device tensors, buf contiguous")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _check(lib.pkv_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                              _stream(buf, stream)), "pkv_read_probe")
