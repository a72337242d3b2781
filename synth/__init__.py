"""Seeded synthetic inputs for the paged KV-cache attention workloads.

This module draws inputs only: sequence lengths, shared-prefix groups, chunk
contexts, the initial order of the free-block queue, and N(0,1) values for
queries, keys and values.  It contains none of the paging or attention
arithmetic, so both the HIP library's callers and the fp64 oracle can consume
it without sharing anything they are compared on.

Values come from a counter-based generator so that any element can be
regenerated on its own:

* a stream is named by (seed, kind, owner); its 32-bit key is
  ``lowbias32(lowbias32(lowbias32(seed ^ 0x9E3779B9) ^ kind) ^ owner)``;
* element ``e`` of the stream draws ``u = lowbias32((e + key) mod 2**32)``
  (lowbias32 is C. Wellons' two-multiply integer hash);
* the value is the standard normal quantile at the centre of bin ``u >> 16``
  of 65536 equal-probability bins, i.e. ``ndtri((i + 0.5) / 65536)``, rounded
  to fp32 and then to the storage dtype by round-to-nearest-even.  The
  distribution is N(0,1) discretised to 65536 levels, cut at +-4.32.

For a key/value stream ``e = (t * H + h) * d + j`` for token position ``t``,
head ``h`` and dimension ``j``; for a query stream ``H`` is the number of
query heads and ``t`` the query's absolute position.  ``synth/fill.hip``
computes the identical integer function on the device, so multi-GB pools are
filled on the GPU while the host can regenerate any sampled sequence.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "DTYPES", "KIND_K", "KIND_V", "KIND_Q", "lowbias32", "stream_key",
    "normal_table", "values", "Workload", "make_workload", "custom_workload",
    "WORKLOADS",
]

# storage dtypes: name -> (bytes per element, numpy container of the raw bits)
DTYPES = {"f32": (4, np.uint32), "f16": (2, np.uint16), "bf16": (2, np.uint16)}

KIND_K, KIND_V, KIND_Q = 1, 2, 3
GROUP_OWNER_BIT = 0x80000000

_M32 = np.uint32(0xFFFFFFFF)


def lowbias32(x):
    """Wellons' lowbias32 hash on uint32 numpy arrays (or Python ints)."""
    scalar = not isinstance(x, np.ndarray)
    x = np.asarray(x, dtype=np.uint32).copy()
    x ^= x >> np.uint32(16)
    x *= np.uint32(0x7FEB352D)
    x ^= x >> np.uint32(15)
    x *= np.uint32(0x846CA68B)
    x ^= x >> np.uint32(16)
    return int(x) if scalar else x


def stream_key(seed: int, kind: int, owner: int) -> int:
    k = lowbias32((seed ^ 0x9E3779B9) & 0xFFFFFFFF)
    k = lowbias32(k ^ (kind & 0xFFFFFFFF))
    return lowbias32(k ^ (owner & 0xFFFFFFFF))


_TABLES: dict = {}


def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    u = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def normal_table(dtype: str) -> np.ndarray:
    """65536 bin-centre normal quantiles as raw ``dtype`` bits."""
    if dtype not in _TABLES:
        from scipy.special import ndtri
        q = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        x32 = ndtri(q).astype(np.float32)
        if dtype == "f32":
            t = x32.view(np.uint32).copy()
        elif dtype == "f16":
            t = x32.astype(np.float16).view(np.uint16).copy()
        elif dtype == "bf16":
            t = _f32_to_bf16_bits(x32)
        else:
            raise ValueError(dtype)
        t.setflags(write=False)
        _TABLES[dtype] = t
    return _TABLES[dtype]


def values(seed: int, kind: int, owner: int, t0: int, t1: int, heads: int,
           dim: int, dtype: str) -> np.ndarray:
    """Raw bits of stream (seed, kind, owner) for positions [t0, t1):
    an array of shape [t1 - t0, heads, dim]."""
    key = np.uint32(stream_key(seed, kind, owner))
    n = (t1 - t0) * heads * dim
    e = (np.arange(n, dtype=np.uint64) + np.uint64(t0 * heads * dim)) & np.uint64(0xFFFFFFFF)
    e = e.astype(np.uint32) + key  # wraps mod 2**32
    u = lowbias32(e)
    return normal_table(dtype)[u >> np.uint32(16)].reshape(t1 - t0, heads, dim)


@dataclass
class Workload:
    """One batch of paged-attention work.

    ``decode_lens[s]`` counts the keys decode sequence ``s`` attends to,
    including the token appended in this step (so ``decode_lens[s] - 1``
    tokens are already cached).  Its first ``prefix_len[s]`` tokens come from
    the shared prefix of ``prefix_group[s]`` (-1: none).  Prefill chunk ``c``
    has ``chunk_ctx[c]`` cached tokens and appends ``chunk_qlen[c]`` new ones,
    each of which is also a query.  ``free_order`` is the initial order of the
    free-block queue.  Owners: chunk ``c`` is owner ``c``; decode sequence
    ``s`` is owner ``n_chunks + s``; prefix group ``g`` is
    ``GROUP_OWNER_BIT | g``.
    """
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    num_blocks: int
    seed: int
    decode_lens: np.ndarray
    prefix_len: np.ndarray
    prefix_group: np.ndarray
    chunk_ctx: np.ndarray
    chunk_qlen: np.ndarray
    free_order: np.ndarray
    description: str = ""
    scale: float = field(default=0.0)

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / float(np.sqrt(self.head_dim))

    @property
    def n_decode(self) -> int:
        return int(self.decode_lens.shape[0])

    @property
    def n_chunks(self) -> int:
        return int(self.chunk_ctx.shape[0])

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.dtype][0]

    def decode_owner(self, s: int) -> int:
        return self.n_chunks + int(s)

    # -- token-level value access (host) ---------------------------------
    def _kv_segments(self, kind: str, idx: int, t0: int, t1: int):
        """(owner, a, b) segments covering positions [t0, t1)."""
        if kind == "chunk":
            return [(int(idx), t0, t1)]
        if kind == "group":
            return [(GROUP_OWNER_BIT | int(idx), t0, t1)]
        pl = int(self.prefix_len[idx])
        segs = []
        if pl > 0 and t0 < pl:
            segs.append((GROUP_OWNER_BIT | int(self.prefix_group[idx]), t0, min(t1, pl)))
        if t1 > max(t0, pl):
            segs.append((self.decode_owner(idx), max(t0, pl), t1))
        return segs

    def kv(self, kind: str, idx: int, t0: int, t1: int):
        """Raw K and V bits [t1-t0, Hkv, d] of decode sequence (kind="decode"),
        prefill chunk (kind="chunk") or shared prefix group (kind="group")
        ``idx`` for positions [t0, t1)."""
        ks, vs = [], []
        for owner, a, b in self._kv_segments(kind, idx, t0, t1):
            ks.append(values(self.seed, KIND_K, owner, a, b, self.n_kv_heads, self.head_dim, self.dtype))
            vs.append(values(self.seed, KIND_V, owner, a, b, self.n_kv_heads, self.head_dim, self.dtype))
        shape = (0, self.n_kv_heads, self.head_dim)
        cont = DTYPES[self.dtype][1]
        k = np.concatenate(ks) if ks else np.zeros(shape, cont)
        v = np.concatenate(vs) if vs else np.zeros(shape, cont)
        return k, v

    def q(self, kind: str, idx: int, p0: int, p1: int) -> np.ndarray:
        """Raw query bits [p1-p0, Hq, d] for absolute positions [p0, p1)."""
        owner = int(idx) if kind == "chunk" else self.decode_owner(idx)
        return values(self.seed, KIND_Q, owner, p0, p1, self.n_q_heads, self.head_dim, self.dtype)

    def kv_segments(self, kind: str, idx: int, t0: int, t1: int):
        """Public form of the owner segments, with their stream keys:
        a list of (key_k, key_v, a, b)."""
        out = []
        for owner, a, b in self._kv_segments(kind, idx, t0, t1):
            out.append((stream_key(self.seed, KIND_K, owner), stream_key(self.seed, KIND_V, owner), a, b))
        return out


def _rng(seed: int, purpose: int, cfg: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, purpose, cfg])))


_P_LENS, _P_ORDER, _P_CTX = 0x1E45, 0x0DE5, 0xC7C7


def custom_workload(name, n_q_heads, n_kv_heads, head_dim, dtype, num_blocks, seed,
                    decode_lens=(), prefix_len=None, prefix_group=None,
                    chunk_ctx=(), chunk_qlen=(), block_size=16, shuffle=True,
                    description="") -> Workload:
    dl = np.asarray(decode_lens, dtype=np.int64).reshape(-1)
    pl = np.zeros_like(dl) if prefix_len is None else np.asarray(prefix_len, np.int64).reshape(-1)
    pg = np.full_like(dl, -1) if prefix_group is None else np.asarray(prefix_group, np.int64).reshape(-1)
    if shuffle:
        order = _rng(seed, _P_ORDER, num_blocks).permutation(num_blocks).astype(np.int32)
    else:
        order = np.arange(num_blocks, dtype=np.int32)
    return Workload(name=name, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                    dtype=dtype, block_size=block_size, num_blocks=num_blocks, seed=seed,
                    decode_lens=dl, prefix_len=pl, prefix_group=pg,
                    chunk_ctx=np.asarray(chunk_ctx, np.int64).reshape(-1),
                    chunk_qlen=np.asarray(chunk_qlen, np.int64).reshape(-1),
                    free_order=order, description=description)


WORKLOADS = ("toy_f32_decode", "tinyllama_decode", "llama3_8b_decode", "opt13b_decode", "llama3_8b_mixed")
# tag of each workload's length / context streams (fixed, so its inputs never change)
_TAG = {name: i + 1 for i, name in enumerate(WORKLOADS)}


def make_workload(name: str, seed: int = 0) -> Workload:
    """The benchmark's five workloads, by name (see WORKLOADS)."""
    if name not in _TAG:
        raise ValueError(f"unknown workload {name!r}")
    tag = _TAG[name]
    if name == "toy_f32_decode":
        return custom_workload(
            name, 4, 2, 64, "f32", 8, seed, decode_lens=[4, 7, 2],
            description="fp32 decode, 3 sequences of 4/7/2 keys, GQA 4:2, d=64, 8-block pool")
    if name == "tinyllama_decode":
        lens = _rng(seed, _P_LENS, tag).integers(128, 2048 + 1, size=64)
        return custom_workload(
            name, 32, 4, 64, "f16", 16384, seed, decode_lens=lens,
            description="TinyLlama-shaped fp16 decode, B=64, L~U[128,2048], Hq32/Hkv4, d=64")
    if name == "llama3_8b_decode":
        lens = _rng(seed, _P_LENS, tag).integers(512, 4096 + 1, size=256)
        group = np.arange(256) // 8
        plen = np.minimum(lens - 1, 1024)
        return custom_workload(
            name, 32, 8, 128, "bf16", 32768, seed, decode_lens=lens,
            prefix_len=plen, prefix_group=group,
            description="Llama-3-8B-shaped bf16 decode, B=256, L~U[512,4096], groups of 8 "
                        "sharing a 1024-token prefix, Hq32/Hkv8, d=128")
    if name == "opt13b_decode":
        return custom_workload(
            name, 40, 40, 128, "f16", 8192, seed, decode_lens=np.full(32, 2048),
            description="OPT-13B-shaped fp16 MHA decode, B=32, L=2048, Hq=Hkv=40, d=128")
    r = _rng(seed, _P_CTX, tag)
    ctx = r.integers(0, 7680 + 1, size=16)
    lens = _rng(seed, _P_LENS, tag).integers(256, 8192 + 1, size=240)
    return custom_workload(
        name, 32, 8, 128, "bf16", 131072, seed, decode_lens=lens,
        chunk_ctx=ctx, chunk_qlen=np.full(16, 512),
        description="Llama-3-8B-shaped bf16 mixed step: 16 prefill chunks of 512 queries "
                    "over contexts U[0,7680] plus 240 decodes with L~U[256,8192]")


# ---------------------------------------------------------------------------
# device-side fill (same integer function, HIP kernel in synth/fill.hip)
# ---------------------------------------------------------------------------
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "libsynth.so")


def _lib():
    global _LIB
    if _LIB is None:
        import torch  # noqa: F401  (HIP runtime shared with torch)
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(p)
        L.synth_fill.restype = ctypes.c_int
        L.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_uint32, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p]
        _LIB = L
    return _LIB


_DEV_TABLES: dict = {}


def fill_device(dst, t0: int, t1: int, heads: int, dim: int, key: int, dtype: str, stream=None):
    """Write stream values for positions [t0, t1) into the contiguous device
    tensor ``dst`` (at least (t1-t0)*heads*dim elements of ``dtype``)."""
    import torch
    dev = dst.device
    tk = (dtype, dev.index)
    if tk not in _DEV_TABLES:
        tab = normal_table(dtype)
        tt = torch.from_numpy(tab.view(np.int32 if dtype == "f32" else np.int16).copy()).to(dev)
        _DEV_TABLES[tk] = tt
    tab = _DEV_TABLES[tk]
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    n = (t1 - t0) * heads * dim
    if dst.numel() * dst.element_size() < n * DTYPES[dtype][0]:
        raise ValueError("destination too small")
    rc = _lib().synth_fill(ctypes.c_void_p(dst.data_ptr()), t1 - t0, t0, heads, dim,
                           ctypes.c_uint32(key), DTYPES[dtype][0],
                           ctypes.c_void_p(tab.data_ptr()), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill failed ({rc})")


def build_lib(verbose: bool = False) -> str:
    """Compile synth/fill.hip into synth/libsynth.so (hipcc, gfx950)."""
    import subprocess
    src = os.path.join(_HERE, "fill.hip")
    out = lib_path()
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "-O3", "-std=c++17", "-fPIC", "-shared",
           "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           src, "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"synth build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    if verbose:
        print(f"built {out}")
    return out
