"""Python binding of libpagedkv.so, the C-ABI paged KV-cache attention library.

Argument marshalling only: every step runs in the library's host code or HIP
kernels.  Functions keep the C names (see include/pagedkv.h for the contract
of each).  Device buffers are torch tensors on a ROCm device; the stream is
torch's current stream unless one is given.

The library is loaded at import; if it has not been built the import fails
(there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loads the HIP runtime the library shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK, PKV_EINVAL, PKV_ENOMEM_BLOCKS, PKV_EUNSUPPORTED, PKV_EHIP, PKV_ESTATE = 0, -1, -2, -3, -4, -5
PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
BLOCK_SIZE = 16

# 8-bit pools are uint8 (or float8_e4m3fn) tensors holding E4M3 codes
_TORCH_CODE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
               torch.uint8: PKV_FP8_E4M3, torch.float8_e4m3fn: PKV_FP8_E4M3}
_NAME_CODE = {"f32": PKV_F32, "f16": PKV_F16, "bf16": PKV_BF16, "fp8_e4m3": PKV_FP8_E4M3}
CODE_TORCH = {PKV_F32: torch.float32, PKV_F16: torch.float16, PKV_BF16: torch.bfloat16,
              PKV_FP8_E4M3: torch.uint8}


class PagedKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class OutOfBlocks(PagedKVError):
    pass


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(python paged_kv_cache_gather_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_pi32, _pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)


class pkv_pool_desc(ctypes.Structure):
    _fields_ = [("num_blocks", _i64), ("block_size", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("dtype", _i32), ("n_layers", _i32), ("reserved", _i32),
                ("initial_free_order", _P)]


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_sig("pkv_last_error", ctypes.c_char_p)
_sig("paged_kv_bytes_per_token", ctypes.c_int, _i32, _i32, _i32, _i32, _pi64)
_sig("paged_kv_blocks_for_budget", ctypes.c_int, _i64, _i32, _i32, _i32, _i32, _i32, _pi64)
_sig("paged_kv_alloc", ctypes.c_int, ctypes.POINTER(pkv_pool_desc), ctypes.POINTER(_P))
_sig("paged_kv_pool_bytes", ctypes.c_int, ctypes.POINTER(pkv_pool_desc), _pi64, _pi64)
_sig("paged_kv_destroy", ctypes.c_int, _P)
_sig("paged_kv_seq_create", ctypes.c_int, _P, _pi64)
_sig("paged_kv_seq_fork", ctypes.c_int, _P, _i64, _i64, _pi64)
_sig("paged_kv_seq_append", ctypes.c_int, _P, _i64, _i64, _P, _P, _i32, _pi32)
_sig("paged_kv_seqs_append", ctypes.c_int, _P, _P, _i32, _P, _P, _P, _i32, _pi32, _pi32)
_sig("paged_kv_seq_blocks_needed", ctypes.c_int, _P, _i64, _i64, _pi64)
_sig("paged_kv_seq_free", ctypes.c_int, _P, _i64)
_sig("paged_kv_seq_len", ctypes.c_int, _P, _i64, _pi64)
_sig("paged_kv_seq_table", ctypes.c_int, _P, _i64, _P, _i64, _pi64)
_sig("paged_kv_block_tables", ctypes.c_int, _P, _P, _i32, _i32, _P, _P)
_sig("paged_kv_num_free", ctypes.c_int, _P, _pi64)
_sig("paged_kv_block_refcount", ctypes.c_int, _P, _i64, _pi32)
_sig("paged_kv_free_queue", ctypes.c_int, _P, _P, _i64, _pi64)
_sig("paged_kv_prefix_cache_enable", ctypes.c_int, _P, _i32)
_sig("paged_kv_seq_create_cached", ctypes.c_int, _P, _P, _i64, _pi64, _pi64)
_sig("paged_kv_seq_append_tokens", ctypes.c_int, _P, _i64, _P, _i64, _P, _P, _i32, _pi32)
_sig("paged_kv_prefix_cache_stats", ctypes.c_int, _P, _pi64, _pi64, _pi64)
_sig("paged_kv_swap_space", ctypes.c_int, _P, _i64)
_sig("paged_kv_seq_swap_out", ctypes.c_int, _P, _i64, _P, _i64, _pi64)
_sig("paged_kv_seq_swap_in", ctypes.c_int, _P, _i64, _P, _i64, _pi64)
_sig("paged_kv_seq_is_swapped", ctypes.c_int, _P, _i64, _pi32)
_sig("paged_kv_cpu_free_queue", ctypes.c_int, _P, _P, _i64, _pi64)
_sig("paged_kv_swap_blocks", ctypes.c_int, _P, _P, _i64, _P, _P, _i64, _P, _i32, _i32, _i32, _i32, _i32, _P)
_sig("reshape_and_cache", ctypes.c_int, _P, _P, _i64, _i64, _P, _P, _P, _i64, _i64, _i32, _i32,
     _i32, _i32, _P)
_sig("reshape_and_cache_fp8", ctypes.c_int, _P, _P, _i32, _i64, _i64, _P, _P, _P, _i64, _i64, _i32, _i32, _i32,
     _f32, _f32, _P)
_sig("paged_kv_copy_blocks", ctypes.c_int, _P, _P, _P, _i32, _i64, _i32, _i32, _i32, _i32, _P)
_sig("paged_attention_decode_partition_size", _i32)
_sig("paged_attention_decode_workspace_bytes", _i64, _i32, _i32, _i32, _i32)
_sig("paged_attention_decode", ctypes.c_int, _P, _i32, _P, _P, _P, _P, _i32, _P, _i32, _i32, _i32,
     _i32, _i32, _i64, _i32, _f32, _i32, _P, _i64, _P)
_sig("paged_attention_decode_fp8_append", ctypes.c_int, _P, _i32, _P, _i32, _P, _P, _i64, _i64, _P, _P, _P, _f32,
     _f32, _P, _i32, _P, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32, _P, _i64, _P)
_sig("paged_attention_decode_append", ctypes.c_int, _P, _i32, _P, _P, _P, _i64, _i64, _P, _P, _P, _P, _i32, _P,
     _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32, _i32, _P, _i64, _P)
_sig("paged_attention_decode_append_noalloc", ctypes.c_int, _P, _i32, _P, _P, _P, _i64, _i64, _P, _P, _P, _P, _i32,
     _P, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32, _i32, _P)
_sig("paged_attention_decode_noalloc_max_workspace_bytes", _i64)
for _n in ("paged_attention_decode_partitions", "paged_attention_decode_reduce"):
    _sig(_n, ctypes.c_int, _P, _i32, _P, _P, _P, _P, _i32, _P, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32,
         _i32, _P, _i64, _P)
for _n in ("paged_attention_decode_fp8", "paged_attention_decode_fp8_partitions",
           "paged_attention_decode_fp8_reduce"):
    _sig(_n, ctypes.c_int, _P, _i32, _P, _i32, _P, _P, _f32, _f32, _P, _i32, _P, _i32, _i32, _i32, _i32, _i32, _i64,
         _i32, _f32, _P, _i64, _P)
_sig("paged_attention_verify_workspace_bytes", _i64, _i32, _i32, _i32, _i32)
_sig("paged_attention_verify", ctypes.c_int, _P, _i32, _P, _P, _P, _P, _i32, _P, _P, _i32, _i32, _i32, _i32, _i32,
     _i32, _i32, _i64, _i32, _f32, _i32, _P, _i64, _P)
_sig("paged_attention_verify_fp8", ctypes.c_int, _P, _i32, _P, _i32, _P, _P, _f32, _f32, _P, _i32, _P, _P, _i32, _i32,
     _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32, _P, _i64, _P)
_sig("paged_kv_read_tiles", ctypes.c_int, _P, _P, _P, _i64, _i64, _i64, _i32, _P, _P)
_sig("paged_kv_mfma_rate", ctypes.c_int, _i32, _i32, _i32, _P, _P)
_sig("paged_attention_decode_whole_context", ctypes.c_int32, _i32, _i32, _i32, _i32, _i32, _i32)
_sig("paged_attention_prefill_chunk", ctypes.c_int, _P, _i32, _P, _P, _P, _P, _i32, _P, _P, _i32,
     _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _f32, _i32, _P)


def last_error() -> str:
    return _lib.pkv_last_error().decode()


def _check(rc: int):
    if rc != PKV_OK:
        cls = OutOfBlocks if rc == PKV_ENOMEM_BLOCKS else PagedKVError
        raise cls(rc, last_error())


def dtype_code(dtype) -> int:
    if isinstance(dtype, str):
        return _NAME_CODE[dtype]
    if isinstance(dtype, int):
        return dtype
    return _TORCH_CODE[dtype]


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream, device=None):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise PagedKVError(PKV_EINVAL, f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise PagedKVError(PKV_EINVAL, f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise PagedKVError(PKV_EINVAL, f"{name} must be contiguous")
    return t


# --------------------------------------------------------------------------
# sizing
# --------------------------------------------------------------------------
def paged_kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, dtype) -> int:
    out = _i64()
    _check(_lib.paged_kv_bytes_per_token(n_layers, n_kv_heads, head_dim, dtype_code(dtype), ctypes.byref(out)))
    return out.value


def paged_kv_blocks_for_budget(budget_bytes: int, n_layers: int, n_kv_heads: int, head_dim: int,
                               dtype, block_size: int = BLOCK_SIZE) -> int:
    out = _i64()
    _check(_lib.paged_kv_blocks_for_budget(budget_bytes, n_layers, n_kv_heads, head_dim, block_size,
                                           dtype_code(dtype), ctypes.byref(out)))
    return out.value


def _desc(num_blocks, n_kv_heads, head_dim, dtype, block_size=BLOCK_SIZE, n_layers=1, order=None):
    d = pkv_pool_desc()
    d.num_blocks, d.block_size, d.n_kv_heads, d.head_dim = num_blocks, block_size, n_kv_heads, head_dim
    d.dtype, d.n_layers, d.reserved = dtype_code(dtype), n_layers, 0
    d.initial_free_order = None if order is None else order.ctypes.data
    return d


def paged_kv_pool_bytes(num_blocks, n_kv_heads, head_dim, dtype, block_size=BLOCK_SIZE):
    d = _desc(num_blocks, n_kv_heads, head_dim, dtype, block_size)
    k, v = _i64(), _i64()
    _check(_lib.paged_kv_pool_bytes(ctypes.byref(d), ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


# --------------------------------------------------------------------------
# host block manager
# --------------------------------------------------------------------------
class Pool:
    """Handle of one pool's host block manager (paged_kv_alloc)."""

    def __init__(self, handle, desc):
        self._h = handle
        self.num_blocks = desc.num_blocks
        self.block_size = desc.block_size
        self.n_kv_heads = desc.n_kv_heads
        self.head_dim = desc.head_dim
        self.dtype = desc.dtype

    @property
    def handle(self):
        if self._h is None:
            raise PagedKVError(PKV_ESTATE, "pool destroyed")
        return self._h

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            try:
                _lib.paged_kv_destroy(self._h)
            except Exception:
                pass
            self._h = None


def paged_kv_alloc(num_blocks: int, n_kv_heads: int, head_dim: int, dtype, block_size: int = BLOCK_SIZE,
                   n_layers: int = 1, initial_free_order=None) -> Pool:
    order = None
    if initial_free_order is not None:
        order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
        if order.size != num_blocks:
            raise PagedKVError(PKV_EINVAL, "initial_free_order must have num_blocks entries")
    d = _desc(num_blocks, n_kv_heads, head_dim, dtype, block_size, n_layers, order)
    h = _P()
    _check(_lib.paged_kv_alloc(ctypes.byref(d), ctypes.byref(h)))
    return Pool(h, d)


def paged_kv_destroy(pool: Pool):
    if pool._h is not None:
        _check(_lib.paged_kv_destroy(pool._h))
        pool._h = None


def paged_kv_seq_create(pool: Pool) -> int:
    s = _i64()
    _check(_lib.paged_kv_seq_create(pool.handle, ctypes.byref(s)))
    return s.value


def paged_kv_seq_fork(pool: Pool, parent: int, n_prefix_tokens: int) -> int:
    s = _i64()
    _check(_lib.paged_kv_seq_fork(pool.handle, parent, n_prefix_tokens, ctypes.byref(s)))
    return s.value


def paged_kv_seq_append(pool: Pool, seq: int, n_tokens: int):
    """Returns (slot_mapping int64 [n_tokens], cow pairs list[(src, dst)])."""
    slots = np.empty(max(n_tokens, 0), dtype=np.int64)
    cow = np.empty(2, dtype=np.int32)
    ncow = _i32()
    _check(_lib.paged_kv_seq_append(pool.handle, seq, n_tokens, slots.ctypes.data, cow.ctypes.data, 1,
                                    ctypes.byref(ncow)))
    return slots, [(int(cow[0]), int(cow[1]))] if ncow.value else []


def paged_kv_seqs_append(pool: Pool, seqs, n_tokens=None):
    """A step's appends in one call: n_tokens[i] (default one) new tokens for
    seqs[i], in order.  Returns (slot_mapping int64 [sum of the counts], cow
    pairs list[(src, dst)]).  If a sequence cannot be appended the error
    raised carries n_done, slots and cow for the sequences before it, which
    stay appended."""
    s = np.ascontiguousarray(seqs, dtype=np.int64).reshape(-1)
    if n_tokens is None:
        counts, total = None, s.size
    else:
        counts = np.ascontiguousarray(n_tokens, dtype=np.int64).reshape(-1)
        if counts.size != s.size:
            raise PagedKVError(PKV_EINVAL, "n_tokens must have one count per sequence")
        total = int(np.maximum(counts, 0).sum())
    slots = np.empty(total, dtype=np.int64)
    cow = np.empty(2 * max(s.size, 1), dtype=np.int32)  # at most one pair per sequence
    ncow, ndone = _i32(), _i32()
    rc = _lib.paged_kv_seqs_append(pool.handle, s.ctypes.data if s.size else None, s.size,
                                   counts.ctypes.data if counts is not None else None, slots.ctypes.data,
                                   cow.ctypes.data, s.size, ctypes.byref(ncow), ctypes.byref(ndone))
    pairs = [(int(cow[2 * i]), int(cow[2 * i + 1])) for i in range(ncow.value)]
    if rc != PKV_OK:
        done = ndone.value
        err = (OutOfBlocks if rc == PKV_ENOMEM_BLOCKS else PagedKVError)(rc, last_error())
        err.n_done = done
        err.slots = slots[:done if counts is None else int(counts[:done].sum())]
        err.cow = pairs
        raise err
    return slots, pairs


def paged_kv_prefix_cache_enable(pool: Pool, enable: bool = True):
    _check(_lib.paged_kv_prefix_cache_enable(pool.handle, 1 if enable else 0))


def paged_kv_seq_create_cached(pool: Pool, tokens) -> tuple[int, int]:
    """New sequence for a prompt of token ids; returns (seq, n_cached tokens reused)."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    s, n = _i64(), _i64()
    _check(_lib.paged_kv_seq_create_cached(pool.handle, tok.ctypes.data if tok.size else None, tok.size,
                                           ctypes.byref(s), ctypes.byref(n)))
    return s.value, n.value


def paged_kv_seq_append_tokens(pool: Pool, seq: int, tokens):
    """paged_kv_seq_append with token ids; returns (slot_mapping, cow pairs)."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    slots = np.empty(tok.size, dtype=np.int64)
    cow = np.empty(2, dtype=np.int32)
    ncow = _i32()
    _check(_lib.paged_kv_seq_append_tokens(pool.handle, seq, tok.ctypes.data if tok.size else None, tok.size,
                                           slots.ctypes.data, cow.ctypes.data, 1, ctypes.byref(ncow)))
    return slots, [(int(cow[0]), int(cow[1]))] if ncow.value else []


def paged_kv_prefix_cache_stats(pool: Pool) -> dict:
    c, q, h = _i64(), _i64(), _i64()
    _check(_lib.paged_kv_prefix_cache_stats(pool.handle, ctypes.byref(c), ctypes.byref(q), ctypes.byref(h)))
    return {"cached_blocks": c.value, "queried_blocks": q.value, "hit_blocks": h.value}


def paged_kv_seq_blocks_needed(pool: Pool, seq: int, n_tokens: int) -> int:
    n = _i64()
    _check(_lib.paged_kv_seq_blocks_needed(pool.handle, seq, n_tokens, ctypes.byref(n)))
    return n.value


def paged_kv_seq_free(pool: Pool, seq: int):
    _check(_lib.paged_kv_seq_free(pool.handle, seq))


def paged_kv_seq_len(pool: Pool, seq: int) -> int:
    n = _i64()
    _check(_lib.paged_kv_seq_len(pool.handle, seq, ctypes.byref(n)))
    return n.value


def paged_kv_seq_table(pool: Pool, seq: int) -> np.ndarray:
    n = _i64()
    _check(_lib.paged_kv_seq_table(pool.handle, seq, None, 0, ctypes.byref(n)))
    out = np.empty(n.value, dtype=np.int32)
    _check(_lib.paged_kv_seq_table(pool.handle, seq, out.ctypes.data, out.size, ctypes.byref(n)))
    return out


def paged_kv_block_tables(pool: Pool, seqs, max_blocks: int):
    """Returns (tables int32 [n, max_blocks] padded with -1, lens int32 [n])."""
    s = np.ascontiguousarray(seqs, dtype=np.int64).reshape(-1)
    tab = np.empty((s.size, max_blocks), dtype=np.int32)
    lens = np.empty(s.size, dtype=np.int32)
    _check(_lib.paged_kv_block_tables(pool.handle, s.ctypes.data, s.size, max_blocks, tab.ctypes.data,
                                      lens.ctypes.data))
    return tab, lens


def paged_kv_num_free(pool: Pool) -> int:
    n = _i64()
    _check(_lib.paged_kv_num_free(pool.handle, ctypes.byref(n)))
    return n.value


def paged_kv_block_refcount(pool: Pool, block: int) -> int:
    r = _i32()
    _check(_lib.paged_kv_block_refcount(pool.handle, block, ctypes.byref(r)))
    return r.value


def paged_kv_free_queue(pool: Pool) -> np.ndarray:
    n = _i64()
    _check(_lib.paged_kv_free_queue(pool.handle, None, 0, ctypes.byref(n)))
    out = np.empty(n.value, dtype=np.int32)
    _check(_lib.paged_kv_free_queue(pool.handle, out.ctypes.data, out.size, ctypes.byref(n)))
    return out


def paged_kv_swap_space(pool: Pool, num_cpu_blocks: int):
    _check(_lib.paged_kv_swap_space(pool.handle, num_cpu_blocks))


def _swap(fn, pool: Pool, seq: int) -> np.ndarray:
    n = _i64()
    _check(_lib.paged_kv_seq_table(pool.handle, seq, None, 0, ctypes.byref(n)))
    pairs = np.empty((max(n.value, 1), 2), dtype=np.int32)
    _check(fn(pool.handle, seq, pairs.ctypes.data, pairs.shape[0], ctypes.byref(n)))
    return pairs[:n.value]


def paged_kv_seq_swap_out(pool: Pool, seq: int) -> np.ndarray:
    """Returns the copies to run, int32 [n, 2] of (GPU block, host block)."""
    return _swap(_lib.paged_kv_seq_swap_out, pool, seq)


def paged_kv_seq_swap_in(pool: Pool, seq: int) -> np.ndarray:
    """Returns the copies to run, int32 [n, 2] of (host block, GPU block)."""
    return _swap(_lib.paged_kv_seq_swap_in, pool, seq)


def paged_kv_seq_is_swapped(pool: Pool, seq: int) -> bool:
    r = _i32()
    _check(_lib.paged_kv_seq_is_swapped(pool.handle, seq, ctypes.byref(r)))
    return bool(r.value)


def paged_kv_cpu_free_queue(pool: Pool) -> np.ndarray:
    n = _i64()
    _check(_lib.paged_kv_cpu_free_queue(pool.handle, None, 0, ctypes.byref(n)))
    out = np.empty(n.value, dtype=np.int32)
    _check(_lib.paged_kv_cpu_free_queue(pool.handle, out.ctypes.data, out.size, ctypes.byref(n)))
    return out


# --------------------------------------------------------------------------
# device operations
# --------------------------------------------------------------------------
def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                      slot_mapping: torch.Tensor, num_blocks: int, n_kv_heads: int, head_dim: int,
                      block_size: int = BLOCK_SIZE, stream=None):
    """key/value: device [T, ..., n_kv_heads*head_dim] rows (token stride = stride(0));
    slot_mapping: device int64 [T]."""
    _dev(key, "key", contiguous=False)
    _dev(value, "value", contiguous=False)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    T = slot_mapping.numel()
    if key.shape[0] != T or value.shape[0] != T:
        raise PagedKVError(PKV_EINVAL, "key/value must have one row per slot")
    if key.dtype != k_pool.dtype or value.dtype != v_pool.dtype or key.dtype != value.dtype:
        raise PagedKVError(PKV_EINVAL, "key, value and pools must share a dtype")
    for t, name in ((key, "key"), (value, "value")):
        if t[0].numel() != n_kv_heads * head_dim or (t.dim() > 1 and not t[0].is_contiguous()):
            raise PagedKVError(PKV_EINVAL, f"{name} rows must be contiguous [n_kv_heads*head_dim]")
    need = num_blocks * n_kv_heads * block_size * head_dim
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    _check(_lib.reshape_and_cache(_ptr(key), _ptr(value), key.stride(0), value.stride(0), _ptr(k_pool),
                                  _ptr(v_pool), _ptr(slot_mapping), T, num_blocks, n_kv_heads, head_dim,
                                  block_size, dtype_code(key.dtype), _stream(stream, key.device)))


def _is_codes(t: torch.Tensor) -> bool:
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                          slot_mapping: torch.Tensor, num_blocks: int, n_kv_heads: int, head_dim: int,
                          k_scale: float, v_scale: float, block_size: int = BLOCK_SIZE, stream=None):
    """Quantising cache write: key/value rows (f32, f16 or bf16) -> E4M3 codes
    in 8-bit pools (uint8 or float8_e4m3fn tensors)."""
    _dev(key, "key", contiguous=False)
    _dev(value, "value", key.dtype, contiguous=False)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    if not (_is_codes(k_pool) and _is_codes(v_pool)):
        raise PagedKVError(PKV_EINVAL, "8-bit pools must be uint8 or float8_e4m3fn tensors")
    T = slot_mapping.numel()
    if key.shape[0] != T or value.shape[0] != T:
        raise PagedKVError(PKV_EINVAL, "key/value must have one row per slot")
    for t, name in ((key, "key"), (value, "value")):
        if t[0].numel() != n_kv_heads * head_dim or (t.dim() > 1 and not t[0].is_contiguous()):
            raise PagedKVError(PKV_EINVAL, f"{name} rows must be contiguous [n_kv_heads*head_dim]")
    need = num_blocks * n_kv_heads * block_size * head_dim
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    _check(_lib.reshape_and_cache_fp8(_ptr(key), _ptr(value), dtype_code(key.dtype), key.stride(0), value.stride(0),
                                      _ptr(k_pool), _ptr(v_pool), _ptr(slot_mapping), T, num_blocks, n_kv_heads,
                                      head_dim, block_size, float(k_scale), float(v_scale),
                                      _stream(stream, key.device)))


def paged_kv_copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, pairs: torch.Tensor, num_blocks: int,
                         n_kv_heads: int, head_dim: int, block_size: int = BLOCK_SIZE, stream=None):
    """pairs: device int32 [n, 2] (src, dst)."""
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    _dev(pairs, "pairs", torch.int32)
    n = pairs.numel() // 2
    need = num_blocks * n_kv_heads * block_size * head_dim
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    _check(_lib.paged_kv_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(pairs), n, num_blocks, n_kv_heads,
                                     head_dim, block_size, dtype_code(k_pool.dtype), _stream(stream, k_pool.device)))


def _reachable(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not (t.is_cuda or t.is_pinned()):
        raise PagedKVError(PKV_EINVAL, f"{name} must be a device tensor or pinned host memory")
    if not t.is_contiguous():
        raise PagedKVError(PKV_EINVAL, f"{name} must be contiguous")
    return t


def paged_kv_swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor, dst_v: torch.Tensor,
                         pairs: torch.Tensor, src_num_blocks: int, dst_num_blocks: int, n_kv_heads: int,
                         head_dim: int, block_size: int = BLOCK_SIZE, stream=None):
    """Whole-block copies between pool pairs (device or pinned host tensors);
    pairs int32 [n, 2] (src, dst), device or pinned host."""
    for t, name in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v"), (pairs, "pairs")):
        _reachable(t, name)
    if pairs.dtype != torch.int32:
        raise PagedKVError(PKV_EINVAL, "pairs must be int32")
    dt = {src_k.dtype, src_v.dtype, dst_k.dtype, dst_v.dtype}
    if len(dt) != 1:
        raise PagedKVError(PKV_EINVAL, "pools must share a dtype")
    per = n_kv_heads * block_size * head_dim
    if min(src_k.numel(), src_v.numel()) < src_num_blocks * per or min(dst_k.numel(), dst_v.numel()) < dst_num_blocks * per:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than their block counts")
    dev = src_k.device if src_k.is_cuda else (dst_k.device if dst_k.is_cuda else None)
    _check(_lib.paged_kv_swap_blocks(_ptr(src_k), _ptr(src_v), src_num_blocks, _ptr(dst_k), _ptr(dst_v),
                                     dst_num_blocks, _ptr(pairs), pairs.numel() // 2, n_kv_heads, head_dim,
                                     block_size, dtype_code(src_k.dtype), _stream(stream, dev)))


def paged_attention_decode_partition_size() -> int:
    return int(_lib.paged_attention_decode_partition_size())


def paged_attention_decode_workspace_bytes(num_seqs: int, n_q_heads: int, head_dim: int,
                                           max_context_len: int) -> int:
    return int(_lib.paged_attention_decode_workspace_bytes(num_seqs, n_q_heads, head_dim, max_context_len))


def _decode_call(fn, out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, n_kv_heads,
                 num_blocks, scale, workspace, block_size, stream):
    _dev(out, "out")
    _dev(q, "q", k_pool.dtype)
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool", k_pool.dtype)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [num_seqs, n_q_heads, head_dim]")
    B, Hq, d = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise PagedKVError(PKV_EINVAL, "block_tables/context_lens must have one row per sequence")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(fn(_ptr(out), dtype_code(out.dtype), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
              block_tables.shape[1], _ptr(context_lens), B, Hq, n_kv_heads, d, block_size, num_blocks,
              max_context_len, float(scale), dtype_code(k_pool.dtype), _ptr(workspace), ws_bytes,
              _stream(stream, q.device)))


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                           n_kv_heads: int, num_blocks: int, scale: float, workspace=None,
                           block_size: int = BLOCK_SIZE, stream=None):
    """out [B, Hq, d] (f32 or the KV dtype); q [B, Hq, d] (KV dtype);
    block_tables int32 [B, max_blocks]; context_lens int32 [B]."""
    _decode_call(_lib.paged_attention_decode, out, q, k_pool, v_pool, block_tables, context_lens,
                 max_context_len, n_kv_heads, num_blocks, scale, workspace, block_size, stream)


def paged_attention_decode_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  slot_mapping: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                                  n_kv_heads: int, num_blocks: int, scale: float, workspace=None,
                                  block_size: int = BLOCK_SIZE, stream=None):
    """reshape_and_cache of each sequence's new row, then paged_attention_decode,
    in one call.  k_new / v_new [B, ..., n_kv_heads*head_dim] rows (KV dtype,
    token stride = stride(0)); slot_mapping int64 [B]; the rest as
    paged_attention_decode."""
    _dev(out, "out")
    _dev(q, "q", k_pool.dtype)
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool", k_pool.dtype)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_new, "k_new", k_pool.dtype, contiguous=False)
    _dev(v_new, "v_new", k_pool.dtype, contiguous=False)
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [num_seqs, n_q_heads, head_dim]")
    B, Hq, d = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise PagedKVError(PKV_EINVAL, "block_tables/context_lens must have one row per sequence")
    if slot_mapping.numel() != B or k_new.shape[0] != B or v_new.shape[0] != B:
        raise PagedKVError(PKV_EINVAL, "k_new, v_new and slot_mapping must have one row per sequence")
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if t[0].numel() != n_kv_heads * d or (t.dim() > 1 and not t[0].is_contiguous()):
            raise PagedKVError(PKV_EINVAL, f"{name} rows must be contiguous [n_kv_heads*head_dim]")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.paged_attention_decode_append(
        _ptr(out), dtype_code(out.dtype), _ptr(q), _ptr(k_new), _ptr(v_new), k_new.stride(0), v_new.stride(0),
        _ptr(slot_mapping), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Hq, n_kv_heads, d, block_size, num_blocks, max_context_len, float(scale),
        dtype_code(k_pool.dtype), _ptr(workspace), ws_bytes, _stream(stream, q.device)))

def paged_attention_decode_noalloc_max_workspace_bytes() -> int:
    return int(_lib.paged_attention_decode_noalloc_max_workspace_bytes())


def paged_attention_decode_append_noalloc(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                                          v_new: torch.Tensor, slot_mapping: torch.Tensor, k_pool: torch.Tensor,
                                          v_pool: torch.Tensor, block_tables: torch.Tensor,
                                          context_lens: torch.Tensor, max_context_len: int, n_kv_heads: int,
                                          num_blocks: int, scale: float, block_size: int = BLOCK_SIZE, stream=None):
    """paged_attention_decode_append without a workspace argument: the
    library's own per-GPU scratch holds the split-context partials and nothing
    is allocated (same arguments otherwise)."""
    _dev(out, "out")
    _dev(q, "q", k_pool.dtype)
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool", k_pool.dtype)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_new, "k_new", k_pool.dtype, contiguous=False)
    _dev(v_new, "v_new", k_pool.dtype, contiguous=False)
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [num_seqs, n_q_heads, head_dim]")
    B, Hq, d = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise PagedKVError(PKV_EINVAL, "block_tables/context_lens must have one row per sequence")
    if slot_mapping.numel() != B or k_new.shape[0] != B or v_new.shape[0] != B:
        raise PagedKVError(PKV_EINVAL, "k_new, v_new and slot_mapping must have one row per sequence")
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if t[0].numel() != n_kv_heads * d or (t.dim() > 1 and not t[0].is_contiguous()):
            raise PagedKVError(PKV_EINVAL, f"{name} rows must be contiguous [n_kv_heads*head_dim]")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    _check(_lib.paged_attention_decode_append_noalloc(
        _ptr(out), dtype_code(out.dtype), _ptr(q), _ptr(k_new), _ptr(v_new), k_new.stride(0), v_new.stride(0),
        _ptr(slot_mapping), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Hq, n_kv_heads, d, block_size, num_blocks, max_context_len, float(scale),
        dtype_code(k_pool.dtype), _stream(stream, q.device)))


def paged_attention_decode_partitions(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                                      n_kv_heads, num_blocks, scale, workspace=None,
                                      block_size: int = BLOCK_SIZE, stream=None):
    """Partition pass of paged_attention_decode (same arguments)."""
    _decode_call(_lib.paged_attention_decode_partitions, out, q, k_pool, v_pool, block_tables, context_lens,
                 max_context_len, n_kv_heads, num_blocks, scale, workspace, block_size, stream)


def paged_attention_decode_reduce(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                                  n_kv_heads, num_blocks, scale, workspace=None,
                                  block_size: int = BLOCK_SIZE, stream=None):
    """Split-context merge pass of paged_attention_decode (same arguments)."""
    _decode_call(_lib.paged_attention_decode_reduce, out, q, k_pool, v_pool, block_tables, context_lens,
                 max_context_len, n_kv_heads, num_blocks, scale, workspace, block_size, stream)


def _decode_fp8_call(fn, out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, n_kv_heads,
                     num_blocks, scale, k_scale, v_scale, workspace, block_size, stream):
    _dev(out, "out")
    _dev(q, "q")
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    if not (_is_codes(k_pool) and _is_codes(v_pool)):
        raise PagedKVError(PKV_EINVAL, "8-bit pools must be uint8 or float8_e4m3fn tensors")
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [num_seqs, n_q_heads, head_dim]")
    B, Hq, d = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise PagedKVError(PKV_EINVAL, "block_tables/context_lens must have one row per sequence")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(fn(_ptr(out), dtype_code(out.dtype), _ptr(q), dtype_code(q.dtype), _ptr(k_pool), _ptr(v_pool),
              float(k_scale), float(v_scale), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Hq,
              n_kv_heads, d, block_size, num_blocks, max_context_len, float(scale), _ptr(workspace), ws_bytes,
              _stream(stream, q.device)))


def paged_attention_decode_fp8(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                               block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                               n_kv_heads: int, num_blocks: int, scale: float, k_scale: float, v_scale: float,
                               workspace=None, block_size: int = BLOCK_SIZE, stream=None):
    """Decode over 8-bit pools (uint8 / float8_e4m3fn codes with scales
    k_scale, v_scale): out [B, Hq, d] (f32 or q's dtype); q [B, Hq, d] f16 or bf16."""
    _decode_fp8_call(_lib.paged_attention_decode_fp8, out, q, k_pool, v_pool, block_tables, context_lens,
                     max_context_len, n_kv_heads, num_blocks, scale, k_scale, v_scale, workspace, block_size, stream)



def paged_attention_decode_fp8_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                      slot_mapping: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                      block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                                      n_kv_heads: int, num_blocks: int, scale: float, k_scale: float, v_scale: float,
                                      workspace=None, block_size: int = BLOCK_SIZE, stream=None):
    """reshape_and_cache_fp8 of each sequence's new row (q's dtype), then
    paged_attention_decode_fp8, in one call; arguments as those two."""
    _dev(out, "out")
    _dev(q, "q")
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_new, "k_new", q.dtype, contiguous=False)
    _dev(v_new, "v_new", q.dtype, contiguous=False)
    if not (_is_codes(k_pool) and _is_codes(v_pool)):
        raise PagedKVError(PKV_EINVAL, "8-bit pools must be uint8 or float8_e4m3fn tensors")
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [num_seqs, n_q_heads, head_dim]")
    B, Hq, d = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise PagedKVError(PKV_EINVAL, "block_tables/context_lens must have one row per sequence")
    if slot_mapping.numel() != B or k_new.shape[0] != B or v_new.shape[0] != B:
        raise PagedKVError(PKV_EINVAL, "k_new, v_new and slot_mapping must have one row per sequence")
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if t[0].numel() != n_kv_heads * d or (t.dim() > 1 and not t[0].is_contiguous()):
            raise PagedKVError(PKV_EINVAL, f"{name} rows must be contiguous [n_kv_heads*head_dim]")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.paged_attention_decode_fp8_append(
        _ptr(out), dtype_code(out.dtype), _ptr(q), dtype_code(q.dtype), _ptr(k_new), _ptr(v_new), k_new.stride(0),
        v_new.stride(0), _ptr(slot_mapping), _ptr(k_pool), _ptr(v_pool), float(k_scale), float(v_scale),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Hq, n_kv_heads, d, block_size, num_blocks,
        max_context_len, float(scale), _ptr(workspace), ws_bytes, _stream(stream, q.device)))


def paged_attention_decode_fp8_partitions(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                                          n_kv_heads, num_blocks, scale, k_scale, v_scale, workspace=None,
                                          block_size: int = BLOCK_SIZE, stream=None):
    """Partition pass of paged_attention_decode_fp8 (same arguments)."""
    _decode_fp8_call(_lib.paged_attention_decode_fp8_partitions, out, q, k_pool, v_pool, block_tables,
                     context_lens, max_context_len, n_kv_heads, num_blocks, scale, k_scale, v_scale, workspace,
                     block_size, stream)


def paged_attention_decode_fp8_reduce(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                                      n_kv_heads, num_blocks, scale, k_scale, v_scale, workspace=None,
                                      block_size: int = BLOCK_SIZE, stream=None):
    """Split-context merge pass of paged_attention_decode_fp8 (same arguments)."""
    _decode_fp8_call(_lib.paged_attention_decode_fp8_reduce, out, q, k_pool, v_pool, block_tables, context_lens,
                     max_context_len, n_kv_heads, num_blocks, scale, k_scale, v_scale, workspace, block_size,
                     stream)


def paged_attention_verify_workspace_bytes(total_q: int, n_q_heads: int, head_dim: int, max_context_len: int) -> int:
    return int(_lib.paged_attention_verify_workspace_bytes(total_q, n_q_heads, head_dim, max_context_len))


def paged_attention_verify(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_tables: torch.Tensor, cu_q_lens: torch.Tensor, context_lens: torch.Tensor,
                           max_q_len: int, max_context_len: int, n_kv_heads: int, num_blocks: int, scale: float,
                           workspace=None, block_size: int = BLOCK_SIZE, stream=None):
    """Same arguments as paged_attention_prefill_chunk plus a workspace
    (paged_attention_verify_workspace_bytes); for a few query tokens per sequence."""
    _dev(out, "out")
    _dev(q, "q", k_pool.dtype)
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool", k_pool.dtype)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(cu_q_lens, "cu_q_lens", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [total_q, n_q_heads, head_dim]")
    total_q, Hq, d = q.shape
    n = context_lens.numel()
    if block_tables.dim() != 2 or block_tables.shape[0] != n or cu_q_lens.numel() != n + 1:
        raise PagedKVError(PKV_EINVAL, "block_tables/cu_q_lens must match context_lens")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.paged_attention_verify(
        _ptr(out), dtype_code(out.dtype), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        block_tables.shape[1], _ptr(cu_q_lens), _ptr(context_lens), n, total_q, max_q_len, Hq, n_kv_heads, d,
        block_size, num_blocks, max_context_len, float(scale), dtype_code(k_pool.dtype), _ptr(workspace), ws_bytes,
        _stream(stream, q.device)))


def paged_attention_verify_fp8(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                               block_tables: torch.Tensor, cu_q_lens: torch.Tensor, context_lens: torch.Tensor,
                               max_q_len: int, max_context_len: int, n_kv_heads: int, num_blocks: int, scale: float,
                               k_scale: float, v_scale: float, workspace=None, block_size: int = BLOCK_SIZE,
                               stream=None):
    """paged_attention_verify over 8-bit pools (uint8 / float8_e4m3fn codes
    with scales); q f16 or bf16, out f32 or q's dtype."""
    _dev(out, "out")
    _dev(q, "q")
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool")
    _dev(block_tables, "block_tables", torch.int32)
    _dev(cu_q_lens, "cu_q_lens", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    if not (_is_codes(k_pool) and _is_codes(v_pool)):
        raise PagedKVError(PKV_EINVAL, "8-bit pools must be uint8 or float8_e4m3fn tensors")
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [total_q, n_q_heads, head_dim]")
    total_q, Hq, d = q.shape
    n = context_lens.numel()
    if block_tables.dim() != 2 or block_tables.shape[0] != n or cu_q_lens.numel() != n + 1:
        raise PagedKVError(PKV_EINVAL, "block_tables/cu_q_lens must match context_lens")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.paged_attention_verify_fp8(
        _ptr(out), dtype_code(out.dtype), _ptr(q), dtype_code(q.dtype), _ptr(k_pool), _ptr(v_pool), float(k_scale),
        float(v_scale), _ptr(block_tables), block_tables.shape[1], _ptr(cu_q_lens), _ptr(context_lens), n, total_q,
        max_q_len, Hq, n_kv_heads, d, block_size, num_blocks, max_context_len, float(scale), _ptr(workspace),
        ws_bytes, _stream(stream, q.device)))


def paged_attention_prefill_chunk(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                                  v_pool: torch.Tensor, block_tables: torch.Tensor, cu_q_lens: torch.Tensor,
                                  context_lens: torch.Tensor, max_q_len: int, max_context_len: int,
                                  n_kv_heads: int, num_blocks: int, scale: float,
                                  block_size: int = BLOCK_SIZE, stream=None):
    """out [total_q, Hq, d]; q [total_q, Hq, d]; block_tables int32 [n, max_blocks];
    cu_q_lens int32 [n+1]; context_lens int32 [n] (keys incl. the chunk)."""
    _dev(out, "out")
    _dev(q, "q", k_pool.dtype)
    _dev(k_pool, "k_pool")
    _dev(v_pool, "v_pool", k_pool.dtype)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(cu_q_lens, "cu_q_lens", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    if q.dim() != 3 or out.shape != q.shape:
        raise PagedKVError(PKV_EINVAL, "q and out must be [total_q, n_q_heads, head_dim]")
    total_q, Hq, d = q.shape
    n = context_lens.numel()
    if block_tables.dim() != 2 or block_tables.shape[0] != n or cu_q_lens.numel() != n + 1:
        raise PagedKVError(PKV_EINVAL, "block_tables/cu_q_lens must match context_lens")
    need = num_blocks * n_kv_heads * block_size * d
    if k_pool.numel() < need or v_pool.numel() < need:
        raise PagedKVError(PKV_EINVAL, "pool tensors smaller than num_blocks blocks")
    _check(_lib.paged_attention_prefill_chunk(
        _ptr(out), dtype_code(out.dtype), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        block_tables.shape[1], _ptr(cu_q_lens), _ptr(context_lens), n, total_q, max_q_len, Hq, n_kv_heads,
        d, block_size, num_blocks, max_context_len, float(scale), dtype_code(k_pool.dtype),
        _stream(stream, q.device)))




def paged_kv_read_tiles(k_pool: torch.Tensor, v_pool, tiles, n_k_tiles: int, n_tiles: int, tile_bytes: int,
                        sink: torch.Tensor, stream=None, streaming: bool = True):
    """Read-only pass over pool tiles (a bandwidth ceiling beside the decode
    kernels); tiles: device int64 [n_tiles] or None for a contiguous read;
    streaming: nontemporal loads as the decode kernels use, else plain ones."""
    _dev(k_pool, "k_pool")
    if v_pool is not None:
        _dev(v_pool, "v_pool")
    if tiles is not None:
        _dev(tiles, "tiles", torch.int64)
        if tiles.numel() < n_tiles:
            raise PagedKVError(PKV_EINVAL, "tiles shorter than n_tiles")
    _dev(sink, "sink")
    if tiles is None and n_tiles * tile_bytes > k_pool.numel() * k_pool.element_size():
        raise PagedKVError(PKV_EINVAL, "contiguous read beyond the buffer")
    _check(_lib.paged_kv_read_tiles(_ptr(k_pool), _ptr(v_pool), _ptr(tiles), n_k_tiles, n_tiles, tile_bytes,
                                    1 if streaming else 0, _ptr(sink), _stream(stream, k_pool.device)))


def paged_kv_mfma_rate(mode: int, n_workgroups: int, iters: int, sink: torch.Tensor, stream=None):
    """The matrix-core rate beside the prefill kernel (16x16x32 bf16 MFMAs;
    mode 0: one wave per SIMD, 1: two, 2: one with a softmax-like vector
    wave beside it, 3: that vector wave alone); sink: device float32 [1]."""
    _dev(sink, "sink", torch.float32)
    _check(_lib.paged_kv_mfma_rate(int(mode), int(n_workgroups), int(iters), _ptr(sink),
                                   _stream(stream, sink.device)))


def paged_attention_decode_whole_context(num_seqs: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                         kv_dtype, max_context_len: int) -> bool:
    """Whether paged_attention_decode / _append take the one-launch
    whole-context path for these sizes (short contexts, small batch)."""
    return bool(_lib.paged_attention_decode_whole_context(int(num_seqs), int(n_q_heads), int(n_kv_heads),
                                                          int(head_dim), dtype_code(kv_dtype),
                                                          int(max_context_len)))


__all__ = [n for n in dir() if n.startswith(("paged_", "reshape_", "pkv", "PKV_", "Pool", "PagedKV",
                                                 "OutOfBlocks", "last_error", "dtype_code", "BLOCK_SIZE"))]
