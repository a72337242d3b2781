"""fp64 CPU oracle for the paged KV-cache attention path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.
It shares no code with the HIP path.  The arithmetic lives in ``oracle.c``
(plain loops, fp64, compiled with gcc by :func:`build`); the block-manager
model lives in ``block_manager.py``.  Each function names the passage of the
pages it restates.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_LIB = None

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8_e4m3": 3}
ESIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o", _SO + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.orc_decode.argtypes = [ctypes.c_int, P, i64, P]
        L.orc_slot.argtypes = [P, i64, i32]
        L.orc_slot.restype = i64
        L.orc_gather.argtypes = [ctypes.c_int, P, P, i64, i32, i32, i32, P, i64, i64, P, P]
        L.orc_scatter.argtypes = [ctypes.c_int, P, P, i64, i64, i64, P, P, P, i64, i32, i32, i32]
        L.orc_copy_blocks.argtypes = [ctypes.c_int, P, P, P, i64, i64, i32, i32, i32]
        L.orc_attention.argtypes = [i64, P, P, i64, P, P, i32, i32, i32, dbl, P, P, P, i32]
        L.orc_quantize_e4m3.argtypes = [P, i64, ctypes.c_float, P]
        L.orc_swap_blocks.argtypes = [ctypes.c_int, P, P, i64, P, P, i64, P, i64, i32, i32, i32]
        L.orc_swap_blocks.restype = ctypes.c_int
        for f in (L.orc_decode, L.orc_gather, L.orc_scatter, L.orc_copy_blocks, L.orc_attention,
                  L.orc_quantize_e4m3):
            f.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------------------
# KV-cache sizing ("How big is the KV cache?" and "Worked memory example",
# vLLM Serving deep dive; "The dark side of the cache", Life of a prompt)
# ---------------------------------------------------------------------------
def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, dtype_bytes: int) -> int:
    """Bytes of K plus V for one token across all layers:
    2 (K and V) * layers * KV heads * head dim * bytes per element."""
    return 2 * n_layers * n_kv_heads * d_head * dtype_bytes


def kv_bytes_per_block(n_layers, n_kv_heads, d_head, dtype_bytes, block_size=16) -> int:
    """One block holds ``block_size`` tokens across every layer."""
    return block_size * kv_bytes_per_token(n_layers, n_kv_heads, d_head, dtype_bytes)


def blocks_for_budget(budget_bytes: int, n_layers, n_kv_heads, d_head, dtype_bytes,
                      block_size=16) -> int:
    """Whole blocks that fit in the KV budget (the "# GPU blocks" figure)."""
    return budget_bytes // kv_bytes_per_block(n_layers, n_kv_heads, d_head, dtype_bytes, block_size)


# ---------------------------------------------------------------------------
# value decoding, gather, scatter, block copy
# ---------------------------------------------------------------------------
def decode(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Raw storage bits -> float64, with the oracle's own bit-level decoders."""
    b = np.ascontiguousarray(bits)
    out = np.empty(b.shape, dtype=np.float64)
    rc = _lib().orc_decode(DTYPE_CODE[dtype], _p(b), b.size, _p(out))
    if rc:
        raise ValueError("bad dtype")
    return out


def e4m3_inv_scale(scale: float) -> np.float32:
    """The fp32 reciprocal of an 8-bit pool's scale (IEEE division, rounded
    to nearest)."""
    return np.float32(1.0) / np.float32(scale)


def quantize_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """fp32 values -> E4M3 codes (uint8) for a pool with this scale: the
    nearest E4M3 value of x * (1/scale) in fp32, ties to even, saturating at
    448 (the 8-bit cache of "Quantization", vLLM Serving deep dive; the format
    and the scale rule are readings, see oracle.c)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x32.shape, dtype=np.uint8)
    _lib().orc_quantize_e4m3(_p(x32), x32.size, ctypes.c_float(float(e4m3_inv_scale(scale))), _p(out))
    return out


def dequantize_e4m3(codes: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes -> fp64 values value(code) * scale (exact in fp64)."""
    return decode("fp8_e4m3", np.ascontiguousarray(codes, dtype=np.uint8)) * float(np.float32(scale))


def slot(table, t: int, block_size: int) -> int:
    """Physical slot of logical token ``t``: table[t // bs] * bs + t % bs
    (PagedAttention in depth, Diagram-in-words)."""
    tb = np.ascontiguousarray(table, dtype=np.int32)
    if t < 0 or t // block_size >= tb.size:
        raise IndexError("token outside the table")
    return int(_lib().orc_slot(_p(tb), t, block_size))


def gather(dtype: str, k_pool: np.ndarray, v_pool: np.ndarray, num_blocks: int, block_size: int,
           n_kv_heads: int, head_dim: int, table, n_tokens: int):
    """Logical K/V [n_tokens, Hkv, d] (fp64) of one sequence, read from the
    pools' raw bytes through its block table."""
    tb = np.ascontiguousarray(table, dtype=np.int32).reshape(-1)
    k = np.empty((n_tokens, n_kv_heads, head_dim), np.float64)
    v = np.empty_like(k)
    kp = np.ascontiguousarray(k_pool)
    vp = np.ascontiguousarray(v_pool)
    rc = _lib().orc_gather(DTYPE_CODE[dtype], _p(kp), _p(vp), num_blocks, block_size, n_kv_heads,
                           head_dim, _p(tb), tb.size, n_tokens, _p(k), _p(v))
    if rc:
        raise ValueError(f"gather failed ({rc})")
    return k, v


def scatter(dtype: str, key_bits: np.ndarray, value_bits: np.ndarray, k_pool: np.ndarray,
            v_pool: np.ndarray, slots, num_blocks: int, block_size: int, n_kv_heads: int,
            head_dim: int):
    """Write new tokens' K/V rows (raw bits, [T, Hkv, d]) into their slots of
    the host pool copies, in place.  Slot -1 is skipped."""
    kb = np.ascontiguousarray(key_bits)
    vb = np.ascontiguousarray(value_bits)
    sl = np.ascontiguousarray(slots, dtype=np.int64).reshape(-1)
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    T = sl.size
    stride = n_kv_heads * head_dim
    rc = _lib().orc_scatter(DTYPE_CODE[dtype], _p(kb), _p(vb), T, stride, stride, _p(k_pool),
                            _p(v_pool), _p(sl), num_blocks, block_size, n_kv_heads, head_dim)
    if rc:
        raise ValueError(f"scatter failed ({rc})")


def copy_blocks(dtype: str, k_pool: np.ndarray, v_pool: np.ndarray, pairs, num_blocks: int,
                block_size: int, n_kv_heads: int, head_dim: int):
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    rc = _lib().orc_copy_blocks(DTYPE_CODE[dtype], _p(k_pool), _p(v_pool), _p(pr), pr.shape[0],
                                num_blocks, block_size, n_kv_heads, head_dim)
    if rc:
        raise ValueError(f"copy_blocks failed ({rc})")


def swap_blocks(dtype: str, src_k: np.ndarray, src_v: np.ndarray, src_num_blocks: int, dst_k: np.ndarray,
                dst_v: np.ndarray, dst_num_blocks: int, pairs, block_size: int, n_kv_heads: int, head_dim: int):
    """Copy whole blocks between two pool pairs (GPU pool and host swap pool),
    in place in dst: pairs [n, 2] of (src block, dst block)."""
    pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    assert dst_k.flags.c_contiguous and dst_v.flags.c_contiguous
    sk, sv = np.ascontiguousarray(src_k), np.ascontiguousarray(src_v)
    rc = _lib().orc_swap_blocks(DTYPE_CODE[dtype], _p(sk), _p(sv), src_num_blocks, _p(dst_k), _p(dst_v),
                                dst_num_blocks, _p(pr), pr.shape[0], block_size, n_kv_heads, head_dim)
    if rc:
        raise ValueError(f"swap_blocks failed ({rc})")


def pool_elems(num_blocks: int, block_size: int, n_kv_heads: int, head_dim: int) -> int:
    return num_blocks * n_kv_heads * block_size * head_dim


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def attention(q: np.ndarray, q_pos, k: np.ndarray, v: np.ndarray, scale: float,
              n_threads: int = 1):
    """Causal softmax attention in fp64 over contiguous K/V.

    q [R, Hq, d]; q_pos [R] absolute positions; k, v [N, Hkv, d].
    Returns (out [R, Hq, d], weight_sums [R, Hq])."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    pos = np.ascontiguousarray(q_pos, dtype=np.int64).reshape(-1)
    R, Hq, d = q.shape
    N, Hkv, d2 = k.shape
    assert d2 == d and v.shape == k.shape and pos.size == R
    out = np.empty((R, Hq, d), np.float64)
    ws = np.empty((R, Hq), np.float64)
    nt = max(1, int(n_threads))
    scratch = np.empty(max(N, 1) * nt, np.float64)
    rc = _lib().orc_attention(R, _p(q), _p(pos), N, _p(k), _p(v), Hq, Hkv, d, float(scale),
                              _p(out), _p(ws), _p(scratch), nt)
    if rc:
        raise ValueError("attention: bad shape or position")
    return out, ws
