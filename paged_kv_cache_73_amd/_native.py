"""ctypes binding of libpa.so (include/pa.h): argument marshalling only.

Every entry point keeps its C name.  Device arguments are torch tensors (their
data pointers are passed through); the stream defaults to torch's current stream.
There is no fallback: if libpa.so is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

PA_OK = 0
PA_F32, PA_BF16 = 0, 1
STATUS = {0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_UNSUPPORTED", -3: "PA_ERR_WORKSPACE",
          -4: "PA_ERR_HIP", -5: "PA_ERR_OUT_OF_BLOCKS", -6: "PA_ERR_REFCOUNT",
          -7: "PA_ERR_METADATA"}

# bytes of the static device scratch of pa_decode_noalloc (PA_DECODE_SCRATCH_BYTES of pa.h)
PA_DECODE_SCRATCH_BYTES = 16 << 20

# every symbol include/pa.h declares
EXPORTS = [
    "pa_status_str", "pa_abi_version", "pa_source_digest", "pa_write_kv", "pa_copy_blocks",
    "pa_decode_workspace_bytes", "pa_decode", "pa_prefill_varlen",
    "pa_bm_create", "pa_bm_destroy", "pa_bm_num_free", "pa_bm_refcount", "pa_bm_free_stack",
    "pa_bm_alloc", "pa_bm_incref", "pa_bm_decref", "pa_bm_release_table", "pa_bm_share",
    "pa_bm_prepare_write", "pa_build_slot_mapping", "pa_build_cu_seqlens", "pa_pool_bytes",
    "pa_validate_decode", "pa_validate_varlen", "pa_validate_slots", "pa_probe_stream_read",
    "pa_prefix_block_hash", "pa_bm_allocate_prefix", "pa_decode_append",
    "pa_prefill_varlen_contiguous", "pa_decode_partials", "pa_decode_merge",
    "pa_prefill_workspace_bytes", "pa_prefill_varlen_splitk", "pa_decode_noalloc",
]


class PaError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)}")


class OutOfBlocks(PaError):
    pass


class RefcountError(PaError):
    pass


def _raise(code: int, what: str):
    if code == -5:
        raise OutOfBlocks(code, what)
    if code == -6:
        raise RefcountError(code, what)
    raise PaError(code, what)


class _Pool(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p)]


_lib = None
_I32P = ctypes.POINTER(ctypes.c_int32)
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32


def lib() -> ctypes.CDLL:
    """Load libpa.so once; raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(the HIP library has no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "pa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "pa_abi_version": (_I32, []),
        "pa_source_digest": (ctypes.c_char_p, []),
        "pa_write_kv": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _VP, _I32, _VP]),
        "pa_copy_blocks": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _I32, _VP]),
        "pa_decode_workspace_bytes": (ctypes.c_size_t, [_I32] * 7),
        "pa_decode": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _I32, _I32, _VP, _I32, _VP,
                                     _I32, ctypes.c_float, _I32, _VP, ctypes.c_size_t, _VP]),
        "pa_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _I32, _I32, _VP, _I32,
                                             _VP, _I32, ctypes.c_float, _I32, _VP]),
        "pa_decode_append": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _VP, _VP, _I32, _I32, _VP,
                                            _I32, _VP, _I32, ctypes.c_float, _I32, _VP,
                                            ctypes.c_size_t, _VP]),
        "pa_decode_partials": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _VP, _VP, _I32, _I32,
                                              _VP, _I32, _VP, _I32, ctypes.c_float, _I32, _VP,
                                              ctypes.c_size_t, _VP]),
        "pa_decode_merge": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _I32, _I32, _I32, _VP, _I32,
                                           _I32, _VP, ctypes.c_size_t, _VP]),
        "pa_prefill_varlen": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _I32, _I32, _VP, _VP,
                                             _I32, _I32, _VP, _I32, ctypes.c_float, _I32, _VP]),
        "pa_prefill_workspace_bytes": (ctypes.c_size_t, [_I32] * 9 + [_I32P, _I32P]),
        "pa_prefill_varlen_splitk": (ctypes.c_int, [ctypes.POINTER(_Pool), _VP, _VP, _I32, _I32, _VP,
                                                    _VP, _I32, _I32, _VP, _I32, ctypes.c_float, _I32,
                                                    _I32P, _I32P, _VP, ctypes.c_size_t, _VP]),
        "pa_prefill_varlen_contiguous": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32,
                                                        _I32, _VP, _VP, _I32, _I32, ctypes.c_float,
                                                        _I32, _VP]),
        "pa_bm_create": (ctypes.c_int, [_I32, _I32P, ctypes.POINTER(_VP)]),
        "pa_bm_destroy": (None, [_VP]),
        "pa_bm_num_free": (_I32, [_VP]),
        "pa_bm_refcount": (ctypes.c_int, [_VP, _I32]),
        "pa_bm_free_stack": (ctypes.c_int, [_VP, _I32P, _I32, _I32P]),
        "pa_bm_alloc": (ctypes.c_int, [_VP, _I32, _I32P]),
        "pa_bm_incref": (ctypes.c_int, [_VP, _I32]),
        "pa_bm_decref": (ctypes.c_int, [_VP, _I32]),
        "pa_bm_release_table": (ctypes.c_int, [_VP, _I32P, _I32]),
        "pa_bm_share": (ctypes.c_int, [_VP, _I32P, _I32, _I32P]),
        "pa_bm_prepare_write": (ctypes.c_int, [_VP, _I32, _I32P, _I32, _I32, _I32, _I32P, _I32P,
                                               _I32, _I32P]),
        "pa_build_slot_mapping": (ctypes.c_int, [_I32P, _I32, _I32, _I32P, _I32P, _I32, _I32P]),
        "pa_build_cu_seqlens": (ctypes.c_int, [_I32P, _I32, _I32P, _I32P]),
        "pa_pool_bytes": (ctypes.c_int64, [_I32, _I32, _I32, _I32]),
        "pa_validate_decode": (ctypes.c_int, [_I32P, _I32, _I32, _I32P, _I32, _I32, _I32, _I32P]),
        "pa_validate_varlen": (ctypes.c_int, [_I32P, _I32, _I32, _I32P, _I32P, _I32, _I32, _I32,
                                              _I32, _I32P]),
        "pa_validate_slots": (ctypes.c_int, [_I32P, _I32, _I32, _I32, _I32P]),
        "pa_probe_stream_read": (ctypes.c_int, [_VP, ctypes.c_size_t, _VP, _I32, _VP]),
        "pa_prefix_block_hash": (ctypes.c_uint64, [_I32P, _I32, ctypes.c_uint64]),
        "pa_bm_allocate_prefix": (ctypes.c_int, [_VP, _I32, _I32P, _I32, _I32P, _I32, _I32P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


# --------------------------------------------------------------------------------------
# host arrays
# --------------------------------------------------------------------------------------

def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


# --------------------------------------------------------------------------------------
# device arguments
# --------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev(t, what: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _meta(t, what: str) -> int:
    """Device int32 metadata (tables, lengths, offsets, slots, block ids)."""
    if t is not None and str(t.dtype) != "torch.int32":
        raise ValueError(f"{what} must be int32, got {t.dtype}")
    return _dev(t, what)


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class KVPool:
    """The two caller-owned pools [num_blocks, B, Hkv, d] (fp32 or bf16)."""

    def __init__(self, k_cache, v_cache):
        torch = _torch()
        if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.dim() != 4:
            raise ValueError("k_cache and v_cache must both be [num_blocks, B, Hkv, d] of one dtype")
        dt = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}.get(k_cache.dtype)
        if dt is None:
            raise ValueError(f"unsupported pool dtype {k_cache.dtype}")
        nb, bs, hkv, d = k_cache.shape
        self.k_cache, self.v_cache = k_cache, v_cache
        self.struct = _Pool(dt, nb, bs, hkv, d, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"))

    @property
    def num_blocks(self):
        return self.struct.num_blocks

    @property
    def block_size(self):
        return self.struct.block_size


def pa_status_str(code: int) -> str:
    return lib().pa_status_str(code).decode()


def pa_abi_version() -> int:
    return lib().pa_abi_version()


def pa_source_digest() -> str:
    return lib().pa_source_digest().decode()


def pa_write_kv(pool: KVPool, k_new, v_new, slot_mapping, stream=None) -> None:
    n = int(slot_mapping.shape[0])
    st = lib().pa_write_kv(ctypes.byref(pool.struct), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                           _meta(slot_mapping, "slot_mapping"), n, _stream(stream))
    if st:
        _raise(st, "pa_write_kv")


def pa_copy_blocks(pool: KVPool, src, dst, stream=None) -> None:
    n = int(src.shape[0])
    st = lib().pa_copy_blocks(ctypes.byref(pool.struct), _meta(src, "src"), _meta(dst, "dst"), n,
                              _stream(stream))
    if st:
        _raise(st, "pa_copy_blocks")


def pa_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_seqlen_k,
                              partition_tokens, block_size) -> int:
    return int(lib().pa_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim,
                                               max_seqlen_k, partition_tokens, block_size))


def pa_decode(pool: KVPool, out, q, block_table, seqlens_k, max_seqlen_k: int,
              softmax_scale: float, partition_tokens: int = 0, workspace=None,
              stream=None) -> None:
    batch, hq = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_decode(ctypes.byref(pool.struct), _dev(out, "out"), _dev(q, "q"), batch, hq,
                         _meta(block_table, "block_table"), int(block_table.shape[1]),
                         _meta(seqlens_k, "seqlens_k"), int(max_seqlen_k), float(softmax_scale),
                         int(partition_tokens), _dev(workspace, "workspace"), ws_bytes,
                         _stream(stream))
    if st:
        _raise(st, "pa_decode")


def pa_decode_noalloc(pool: KVPool, out, q, block_table, seqlens_k, max_seqlen_k: int,
                      softmax_scale: float, partition_tokens: int = 0, stream=None) -> None:
    batch, hq = int(q.shape[0]), int(q.shape[1])
    st = lib().pa_decode_noalloc(ctypes.byref(pool.struct), _dev(out, "out"), _dev(q, "q"), batch,
                                 hq, _meta(block_table, "block_table"), int(block_table.shape[1]),
                                 _meta(seqlens_k, "seqlens_k"), int(max_seqlen_k),
                                 float(softmax_scale), int(partition_tokens), _stream(stream))
    if st:
        _raise(st, "pa_decode_noalloc")


def pa_decode_append(pool: KVPool, out, q, k_new, v_new, block_table, seqlens_k,
                     max_seqlen_k: int, softmax_scale: float, partition_tokens: int = 0,
                     workspace=None, stream=None) -> None:
    batch, hq = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_decode_append(ctypes.byref(pool.struct), _dev(out, "out"), _dev(q, "q"),
                                _dev(k_new, "k_new"), _dev(v_new, "v_new"), batch, hq,
                                _meta(block_table, "block_table"), int(block_table.shape[1]),
                                _meta(seqlens_k, "seqlens_k"), int(max_seqlen_k),
                                float(softmax_scale), int(partition_tokens),
                                _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    if st:
        _raise(st, "pa_decode_append")


def pa_decode_partials(pool: KVPool, out, q, block_table, seqlens_k, max_seqlen_k: int,
                       softmax_scale: float, partition_tokens: int = 0, workspace=None,
                       k_new=None, v_new=None, stream=None) -> None:
    """Pass 1 of pa_decode (optionally with the fused append); pa_decode_merge follows."""
    batch, hq = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_decode_partials(ctypes.byref(pool.struct), _dev(out, "out"), _dev(q, "q"),
                                  _dev(k_new, "k_new"), _dev(v_new, "v_new"), batch, hq,
                                  _meta(block_table, "block_table"), int(block_table.shape[1]),
                                  _meta(seqlens_k, "seqlens_k"), int(max_seqlen_k),
                                  float(softmax_scale), int(partition_tokens),
                                  _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    if st:
        _raise(st, "pa_decode_partials")


def pa_decode_merge(pool: KVPool, out, block_table, seqlens_k, max_seqlen_k: int,
                    partition_tokens: int = 0, workspace=None, stream=None) -> None:
    """Pass 2 of pa_decode, with the arguments of the pa_decode_partials call before it."""
    batch, hq = int(out.shape[0]), int(out.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_decode_merge(ctypes.byref(pool.struct), _dev(out, "out"), batch, hq,
                               int(block_table.shape[1]), _meta(seqlens_k, "seqlens_k"),
                               int(max_seqlen_k), int(partition_tokens),
                               _dev(workspace, "workspace"), ws_bytes, _stream(stream))
    if st:
        _raise(st, "pa_decode_merge")


def pa_prefill_varlen(pool: KVPool, out, q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                      max_seqlen_k: int, block_table, softmax_scale: float, causal: bool = True,
                      stream=None) -> None:
    batch = int(cu_seqlens_q.shape[0]) - 1
    st = lib().pa_prefill_varlen(ctypes.byref(pool.struct), _dev(out, "out"), _dev(q, "q"), batch,
                                 int(q.shape[1]), _meta(cu_seqlens_q, "cu_seqlens_q"),
                                 _meta(cu_seqlens_k, "cu_seqlens_k"), int(max_seqlen_q),
                                 int(max_seqlen_k), _meta(block_table, "block_table"),
                                 int(block_table.shape[1]), float(softmax_scale), int(bool(causal)),
                                 _stream(stream))
    if st:
        _raise(st, "pa_prefill_varlen")


def _host_i32(a):
    """A host int32 array for an optional host-side copy of metadata (None stays None)."""
    if a is None:
        return None
    arr = (ctypes.c_int32 * len(a))(*[int(x) for x in a])
    return arr


def pa_prefill_workspace_bytes(dtype: int, batch: int, num_heads: int, num_kv_heads: int,
                               head_dim: int, block_size: int, max_seqlen_q: int,
                               max_seqlen_k: int, causal: bool = True, host_cu_seqlens_q=None,
                               host_cu_seqlens_k=None) -> int:
    """Workspace of pa_prefill_varlen_splitk; host_cu_seqlens_q/k: optional host lists."""
    return int(lib().pa_prefill_workspace_bytes(int(dtype), int(batch), int(num_heads),
                                                int(num_kv_heads), int(head_dim), int(block_size),
                                                int(max_seqlen_q), int(max_seqlen_k),
                                                int(bool(causal)), _host_i32(host_cu_seqlens_q),
                                                _host_i32(host_cu_seqlens_k)))


def pa_prefill_varlen_splitk(pool: KVPool, out, q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                             max_seqlen_k: int, block_table, softmax_scale: float,
                             causal: bool = True, workspace=None, host_cu_seqlens_q=None,
                             host_cu_seqlens_k=None, stream=None) -> None:
    batch = int(cu_seqlens_q.shape[0]) - 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().pa_prefill_varlen_splitk(ctypes.byref(pool.struct), _dev(out, "out"), _dev(q, "q"),
                                        batch, int(q.shape[1]), _meta(cu_seqlens_q, "cu_seqlens_q"),
                                        _meta(cu_seqlens_k, "cu_seqlens_k"), int(max_seqlen_q),
                                        int(max_seqlen_k), _meta(block_table, "block_table"),
                                        int(block_table.shape[1]), float(softmax_scale),
                                        int(bool(causal)), _host_i32(host_cu_seqlens_q),
                                        _host_i32(host_cu_seqlens_k), _dev(workspace, "workspace"),
                                        ws_bytes, _stream(stream))
    if st:
        _raise(st, "pa_prefill_varlen_splitk")


def pa_prefill_varlen_contiguous(out, q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                                 max_seqlen_k: int, softmax_scale: float, causal: bool = True,
                                 stream=None) -> None:
    """Packed q [total_q, Hq, d] against packed k, v [total_k, Hkv, d] (no block table)."""
    torch = _torch()
    if k.shape != v.shape or k.dtype != v.dtype or k.dtype != q.dtype or k.dim() != 3:
        raise ValueError("k and v must both be [total_k, Hkv, d] of q's dtype")
    dt = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    batch = int(cu_seqlens_q.shape[0]) - 1
    st = lib().pa_prefill_varlen_contiguous(
        _dev(out, "out"), _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), dt, batch, int(q.shape[1]),
        int(k.shape[1]), int(k.shape[2]), _meta(cu_seqlens_q, "cu_seqlens_q"),
        _meta(cu_seqlens_k, "cu_seqlens_k"), int(max_seqlen_q), int(max_seqlen_k),
        float(softmax_scale), int(bool(causal)), _stream(stream))
    if st:
        _raise(st, "pa_prefill_varlen_contiguous")


def pa_probe_stream_read(buf, sink, grid: int, stream=None) -> None:
    st = lib().pa_probe_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                    _dev(sink, "sink"), int(grid), _stream(stream))
    if st:
        _raise(st, "pa_probe_stream_read")


# --------------------------------------------------------------------------------------
# host block manager and builders
# --------------------------------------------------------------------------------------

class BlockManager:
    """The library's reference-counted free stack (pa_bm_*).  ``prepare_write``
    mutates the given row (a Python list) in place, like the C call."""

    def __init__(self, num_blocks: int, initial_order=None):
        self._h = _VP()
        order = None if initial_order is None else _i32(initial_order)
        st = lib().pa_bm_create(num_blocks, None if order is None else _ptr(order),
                                ctypes.byref(self._h))
        if st:
            _raise(st, "pa_bm_create")
        self.num_blocks = num_blocks

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pa_bm_destroy(self._h)
            self._h = None

    def num_free(self) -> int:
        return lib().pa_bm_num_free(self._h)

    def refcount(self, block: int) -> int:
        r = lib().pa_bm_refcount(self._h, block)
        if r < 0:
            _raise(r, "pa_bm_refcount")
        return r

    @property
    def refs(self) -> list[int]:
        return [self.refcount(i) for i in range(self.num_blocks)]

    @property
    def free(self) -> list[int]:
        """Free stack as a list whose end is handed out next (like the oracle's)."""
        out = np.zeros(max(1, self.num_blocks), dtype=np.int32)
        cnt = ctypes.c_int32()
        st = lib().pa_bm_free_stack(self._h, _ptr(out), len(out), ctypes.byref(cnt))
        if st:
            _raise(st, "pa_bm_free_stack")
        return list(reversed(out[:cnt.value].tolist()))

    def alloc(self, n: int) -> list[int]:
        ids = np.zeros(max(1, n), dtype=np.int32)
        st = lib().pa_bm_alloc(self._h, n, _ptr(ids))
        if st:
            _raise(st, "pa_bm_alloc")
        return ids[:n].tolist()

    def incref(self, block: int) -> None:
        st = lib().pa_bm_incref(self._h, block)
        if st:
            _raise(st, "pa_bm_incref")

    def decref(self, block: int) -> None:
        st = lib().pa_bm_decref(self._h, block)
        if st:
            _raise(st, "pa_bm_decref")

    def release_table(self, row) -> None:
        r = _i32(row)
        st = lib().pa_bm_release_table(self._h, _ptr(r), len(r))
        if st:
            _raise(st, "pa_bm_release_table")

    def share(self, row) -> list[int]:
        r = _i32(row)
        out = np.zeros_like(r)
        st = lib().pa_bm_share(self._h, _ptr(r), len(r), _ptr(out))
        if st:
            _raise(st, "pa_bm_share")
        return out.tolist()

    def allocate_prefix(self, tokens, block_size: int, width: int):
        t = _i32(tokens)
        row = np.full(max(1, width), -1, dtype=np.int32)
        hits = ctypes.c_int32()
        st = lib().pa_bm_allocate_prefix(self._h, block_size, _ptr(t), len(t), _ptr(row), width,
                                         ctypes.byref(hits))
        if st:
            _raise(st, "pa_bm_allocate_prefix")
        return row[:width].tolist(), hits.value

    def prepare_write(self, row: list, start: int, count: int, block_size: int):
        r = _i32(row)
        cap = len(r)
        src = np.zeros(max(1, cap), dtype=np.int32)
        dst = np.zeros(max(1, cap), dtype=np.int32)
        n = ctypes.c_int32()
        st = lib().pa_bm_prepare_write(self._h, block_size, _ptr(r), len(r), start, count,
                                       _ptr(src), _ptr(dst), cap, ctypes.byref(n))
        if st:
            _raise(st, "pa_bm_prepare_write")
        row[:] = r.tolist()
        return list(zip(src[:n.value].tolist(), dst[:n.value].tolist()))


def pa_prefix_block_hash(tokens, prefix_hash: int) -> int:
    t = _i32(tokens)
    return int(lib().pa_prefix_block_hash(_ptr(t), len(t), prefix_hash))


def pa_build_slot_mapping(table, block_size: int, seq, pos) -> np.ndarray:
    t = _i32(table)
    if t.ndim == 1:
        t = t[None]
    s, p = _i32(seq), _i32(pos)
    out = np.zeros(max(1, len(s)), dtype=np.int32)
    st = lib().pa_build_slot_mapping(_ptr(t), t.shape[1], block_size, _ptr(s), _ptr(p), len(s),
                                     _ptr(out))
    if st:
        _raise(st, "pa_build_slot_mapping")
    return out[:len(s)]


def pa_build_cu_seqlens(lengths) -> tuple[np.ndarray, int]:
    lens = _i32(lengths)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    mx = ctypes.c_int32()
    st = lib().pa_build_cu_seqlens(_ptr(lens), len(lens), _ptr(cu), ctypes.byref(mx))
    if st:
        _raise(st, "pa_build_cu_seqlens")
    return cu, mx.value


def pa_pool_bytes(num_blocks, block_size, kv_dim, elem_bytes) -> int:
    return int(lib().pa_pool_bytes(num_blocks, block_size, kv_dim, elem_bytes))


def pa_validate_decode(table, seqlens, max_seqlen_k, num_blocks, block_size):
    t, s = _i32(table), _i32(seqlens)
    bad = ctypes.c_int32()
    st = lib().pa_validate_decode(_ptr(t), t.shape[0], t.shape[1], _ptr(s), max_seqlen_k,
                                  num_blocks, block_size, ctypes.byref(bad))
    return st, bad.value


def pa_validate_varlen(table, cu_q, cu_k, max_seqlen_q, max_seqlen_k, num_blocks, block_size):
    t, q, k = _i32(table), _i32(cu_q), _i32(cu_k)
    bad = ctypes.c_int32()
    st = lib().pa_validate_varlen(_ptr(t), len(q) - 1, t.shape[1], _ptr(q), _ptr(k), max_seqlen_q,
                                  max_seqlen_k, num_blocks, block_size, ctypes.byref(bad))
    return st, bad.value


def pa_validate_slots(slots, num_blocks, block_size):
    s = _i32(slots)
    bad = ctypes.c_int32()
    st = lib().pa_validate_slots(_ptr(s), len(s), num_blocks, block_size, ctypes.byref(bad))
    return st, bad.value
