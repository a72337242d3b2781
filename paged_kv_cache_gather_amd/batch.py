"""Builds one step's device state for a synthetic workload through the
library's own entry points: the host block manager lays out every sequence
(shared prefixes by fork + copy-on-write), reshape_and_cache writes the cached
context and, each step, the appended tokens; the attention calls read it back
through the block tables.

Values come from ``synth`` (the seeded generator), filled on the device or
uploaded from the host.  With ``kv_cache="fp8_e4m3"`` the pools hold 8-bit
codes: the same rows are quantised on the way in (reshape_and_cache_fp8) and
decode reads them with paged_attention_decode_fp8.  Nothing here computes
attention.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import synth
from . import (paged_kv_alloc, paged_kv_seq_create, paged_kv_seq_fork, paged_kv_seq_append, paged_kv_seqs_append,
               paged_kv_seq_free, paged_kv_block_tables, paged_kv_copy_blocks, reshape_and_cache,
               reshape_and_cache_fp8, paged_attention_decode, paged_attention_decode_fp8,
               paged_attention_decode_fp8_partitions, paged_attention_decode_fp8_reduce,
               paged_attention_decode_workspace_bytes, paged_attention_decode_partitions,
               paged_attention_decode_append, paged_attention_decode_fp8_append,
               paged_attention_decode_reduce, paged_attention_prefill_chunk, paged_attention_verify,
               paged_attention_verify_workspace_bytes, paged_attention_verify_fp8, BLOCK_SIZE)

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_VIEW = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}


def _upload(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    view = bits.view(np.int32 if dtype == "f32" else np.int16)
    return torch.from_numpy(np.ascontiguousarray(view)).to(device).view(TORCH_DTYPE[dtype])


@dataclass
class DecodeState:
    seqs: list
    lens: np.ndarray            # keys attended (incl. appended token)
    slots: torch.Tensor         # int64 [B] slot of the appended token
    k_new: torch.Tensor         # [B, Hkv, d]
    v_new: torch.Tensor
    q: torch.Tensor             # [B, Hq, d]
    tables: torch.Tensor        # int32 [B, max_blocks]
    tables_host: np.ndarray
    lens_dev: torch.Tensor      # int32 [B]
    max_context_len: int
    cow: list = field(default_factory=list)
    workspace: torch.Tensor | None = None


@dataclass
class PrefillState:
    seqs: list
    ctx: np.ndarray             # cached tokens before each chunk
    qlen: np.ndarray
    slots: torch.Tensor         # int64 [total_q]
    k_new: torch.Tensor         # [total_q, Hkv, d]
    v_new: torch.Tensor
    q: torch.Tensor             # [total_q, Hq, d]
    tables: torch.Tensor
    tables_host: np.ndarray
    cu_q_lens: torch.Tensor     # int32 [n+1]
    lens_dev: torch.Tensor      # int32 [n] keys incl. chunk
    max_q_len: int
    max_context_len: int
    cow: list = field(default_factory=list)


class DeviceBatch:
    """Device pools plus the decode and prefill inputs of one step of ``w``."""

    def __init__(self, w: synth.Workload, device="cuda:0", fill: str = "device",
                 out_dtype: str | None = None, stage_tokens: int = 1 << 16, kv_cache: str | None = None,
                 k_scale: float = 1.0, v_scale: float = 1.0):
        self.w = w
        self.device = torch.device(device)
        self.fill = fill
        self.tdt = TORCH_DTYPE[w.dtype]
        self.out_dtype = TORCH_DTYPE[out_dtype or w.dtype]
        self.fp8 = kv_cache == "fp8_e4m3"
        if kv_cache not in (None, w.dtype, "fp8_e4m3"):
            raise ValueError(f"kv_cache {kv_cache!r}: the workload's dtype or fp8_e4m3")
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        H, d = w.n_kv_heads, w.head_dim
        self.pool = paged_kv_alloc(w.num_blocks, H, d, "fp8_e4m3" if self.fp8 else w.dtype,
                                   initial_free_order=w.free_order)
        n = w.num_blocks * H * BLOCK_SIZE * d
        pdt = torch.uint8 if self.fp8 else self.tdt
        self.k_pool = torch.zeros(n, dtype=pdt, device=self.device)
        self.v_pool = torch.zeros(n, dtype=pdt, device=self.device)
        self._stage = max(stage_tokens, 1)
        self.decode = self._build_decode() if w.n_decode else None
        self.prefill = self._build_prefill() if w.n_chunks else None
        torch.cuda.synchronize(self.device)

    # -- value staging ----------------------------------------------------
    def _kv_rows(self, kind: str, idx: int, t0: int, t1: int):
        """Device K and V rows [t1-t0, Hkv, d] of positions [t0, t1)."""
        w = self.w
        H, d = w.n_kv_heads, w.head_dim
        if self.fill == "host":
            k, v = w.kv(kind, idx, t0, t1)
            return _upload(k, w.dtype, self.device), _upload(v, w.dtype, self.device)
        k = torch.empty((t1 - t0, H, d), dtype=self.tdt, device=self.device)
        v = torch.empty_like(k)
        for key_k, key_v, a, b in w.kv_segments(kind, idx, t0, t1):
            synth.fill_device(k[a - t0:b - t0], a, b, H, d, key_k, w.dtype)
            synth.fill_device(v[a - t0:b - t0], a, b, H, d, key_v, w.dtype)
        return k, v

    def _q_rows(self, kind: str, idx: int, p0: int, p1: int):
        w = self.w
        if self.fill == "host":
            return _upload(w.q(kind, idx, p0, p1), w.dtype, self.device)
        qt = torch.empty((p1 - p0, w.n_q_heads, w.head_dim), dtype=self.tdt, device=self.device)
        owner = idx if kind == "chunk" else w.decode_owner(idx)
        synth.fill_device(qt, p0, p1, w.n_q_heads, w.head_dim,
                          synth.stream_key(w.seed, synth.KIND_Q, owner), w.dtype)
        return qt

    def _write(self, kind, idx, t0, t1, slots):
        """Write positions [t0, t1) of a sequence into the given slots."""
        w = self.w
        for a in range(t0, t1, self._stage):
            b = min(t1, a + self._stage)
            k, v = self._kv_rows(kind, idx, a, b)
            sl = torch.from_numpy(np.ascontiguousarray(slots[a - t0:b - t0])).to(self.device)
            self._cache(k.view(b - a, -1), v.view(b - a, -1), sl)

    def _cache(self, k, v, slots, stream=None):
        w = self.w
        if self.fp8:
            reshape_and_cache_fp8(k, v, self.k_pool, self.v_pool, slots, w.num_blocks, w.n_kv_heads, w.head_dim,
                                  self.k_scale, self.v_scale, stream=stream)
        else:
            reshape_and_cache(k, v, self.k_pool, self.v_pool, slots, w.num_blocks, w.n_kv_heads, w.head_dim,
                              stream=stream)

    def _cow(self, pairs):
        if pairs:
            pr = torch.tensor(pairs, dtype=torch.int32, device=self.device)
            w = self.w
            paged_kv_copy_blocks(self.k_pool, self.v_pool, pr, w.num_blocks, w.n_kv_heads, w.head_dim)

    # -- decode sequences -------------------------------------------------
    def _build_decode(self) -> DecodeState:
        w = self.w
        B = w.n_decode
        lens = w.decode_lens.astype(np.int64)
        seqs = [None] * B
        roots = {}
        # shared prefixes: one root per group, holding the longest prefix any member uses
        for g in sorted(set(int(x) for x in w.prefix_group if x >= 0)):
            members = np.flatnonzero(w.prefix_group == g)
            plen = int(w.prefix_len[members].max())
            r = paged_kv_seq_create(self.pool)
            slots, _ = paged_kv_seq_append(self.pool, r, plen)
            self._write("group", g, 0, plen, slots)
            roots[g] = r
        for s in range(B):
            pl = int(w.prefix_len[s]) if w.prefix_group[s] >= 0 else 0
            if pl > 0:
                seq = paged_kv_seq_fork(self.pool, roots[int(w.prefix_group[s])], pl)
            else:
                seq = paged_kv_seq_create(self.pool)
            n_priv = int(lens[s]) - 1 - pl
            if n_priv > 0:
                slots, cow = paged_kv_seq_append(self.pool, seq, n_priv)
                self._cow(cow)
                self._write("decode", s, pl, pl + n_priv, slots)
            seqs[s] = seq
        for r in roots.values():
            paged_kv_seq_free(self.pool, r)
        # this step's appended token, one batched call for the whole batch
        new_slots, cow_all = paged_kv_seqs_append(self.pool, seqs)
        self._cow(cow_all)
        k_new = torch.empty((B, w.n_kv_heads, w.head_dim), dtype=self.tdt, device=self.device)
        v_new = torch.empty_like(k_new)
        q = torch.empty((B, w.n_q_heads, w.head_dim), dtype=self.tdt, device=self.device)
        for s in range(B):
            L = int(lens[s])
            k, v = self._kv_rows("decode", s, L - 1, L)
            k_new[s].copy_(k[0])
            v_new[s].copy_(v[0])
            q[s].copy_(self._q_rows("decode", s, L - 1, L)[0])
        maxb = int(-(-lens.max() // BLOCK_SIZE))
        tab, tl = paged_kv_block_tables(self.pool, seqs, maxb)
        assert np.array_equal(tl.astype(np.int64), lens)
        mcl = int(lens.max())
        ws_bytes = paged_attention_decode_workspace_bytes(B, w.n_q_heads, w.head_dim, mcl)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=self.device) if ws_bytes else None
        return DecodeState(seqs=seqs, lens=lens, slots=torch.from_numpy(new_slots).to(self.device),
                           k_new=k_new, v_new=v_new, q=q, tables=torch.from_numpy(tab).to(self.device),
                           tables_host=tab, lens_dev=torch.from_numpy(tl).to(self.device),
                           max_context_len=mcl, cow=cow_all, workspace=ws)

    # -- prefill chunks ---------------------------------------------------
    def _build_prefill(self) -> PrefillState:
        w = self.w
        n = w.n_chunks
        ctx = w.chunk_ctx.astype(np.int64)
        qlen = w.chunk_qlen.astype(np.int64)
        seqs = []
        for c in range(n):
            seq = paged_kv_seq_create(self.pool)
            if ctx[c] > 0:
                slots, _ = paged_kv_seq_append(self.pool, seq, int(ctx[c]))
                self._write("chunk", c, 0, int(ctx[c]), slots)
            seqs.append(seq)
        total = int(qlen.sum())
        cu = np.zeros(n + 1, dtype=np.int32)
        cu[1:] = np.cumsum(qlen)
        # the chunks' new tokens, one batched call
        slots_all, cow_all = paged_kv_seqs_append(self.pool, seqs, qlen)
        self._cow(cow_all)
        k_new = torch.empty((total, w.n_kv_heads, w.head_dim), dtype=self.tdt, device=self.device)
        v_new = torch.empty_like(k_new)
        q = torch.empty((total, w.n_q_heads, w.head_dim), dtype=self.tdt, device=self.device)
        for c in range(n):
            a, b = int(ctx[c]), int(ctx[c] + qlen[c])
            k, v = self._kv_rows("chunk", c, a, b)
            k_new[cu[c]:cu[c + 1]].copy_(k)
            v_new[cu[c]:cu[c + 1]].copy_(v)
            q[cu[c]:cu[c + 1]].copy_(self._q_rows("chunk", c, a, b))
        keys = ctx + qlen
        maxb = int(-(-keys.max() // BLOCK_SIZE))
        tab, tl = paged_kv_block_tables(self.pool, seqs, maxb)
        return PrefillState(seqs=seqs, ctx=ctx, qlen=qlen, slots=torch.from_numpy(slots_all).to(self.device),
                            k_new=k_new, v_new=v_new, q=q, tables=torch.from_numpy(tab).to(self.device),
                            tables_host=tab, cu_q_lens=torch.from_numpy(cu).to(self.device),
                            lens_dev=torch.from_numpy(tl).to(self.device), max_q_len=int(qlen.max()),
                            max_context_len=int(keys.max()), cow=cow_all)

    # -- one step of the hot path ------------------------------------------
    def append_decode(self, stream=None):
        d = self.decode
        w = self.w
        self._cache(d.k_new.view(w.n_decode, -1), d.v_new.view(w.n_decode, -1), d.slots, stream=stream)

    def attend_decode(self, out: torch.Tensor, stream=None):
        d = self.decode
        w = self.w
        if self.fp8:
            paged_attention_decode_fp8(out, d.q, self.k_pool, self.v_pool, d.tables, d.lens_dev, d.max_context_len,
                                       w.n_kv_heads, w.num_blocks, w.scale, self.k_scale, self.v_scale,
                                       workspace=d.workspace, stream=stream)
        else:
            paged_attention_decode(out, d.q, self.k_pool, self.v_pool, d.tables, d.lens_dev, d.max_context_len,
                                   w.n_kv_heads, w.num_blocks, w.scale, workspace=d.workspace, stream=stream)

    def step_decode(self, out: torch.Tensor, stream=None):
        """The decode step in one call: the new rows' cache write and the
        attention (paged_attention_decode_append, or its 8-bit variant)."""
        d = self.decode
        w = self.w
        if self.fp8:
            paged_attention_decode_fp8_append(out, d.q, d.k_new.view(w.n_decode, -1), d.v_new.view(w.n_decode, -1),
                                              d.slots, self.k_pool, self.v_pool, d.tables, d.lens_dev,
                                              d.max_context_len, w.n_kv_heads, w.num_blocks, w.scale, self.k_scale,
                                              self.v_scale, workspace=d.workspace, stream=stream)
            return
        paged_attention_decode_append(out, d.q, d.k_new.view(w.n_decode, -1), d.v_new.view(w.n_decode, -1), d.slots,
                                      self.k_pool, self.v_pool, d.tables, d.lens_dev, d.max_context_len,
                                      w.n_kv_heads, w.num_blocks, w.scale, workspace=d.workspace, stream=stream)

    def attend_decode_split(self, out: torch.Tensor, between=None, stream=None):
        """The decode attention as its two passes, calling ``between()`` (if
        given) after queueing the partition pass — e.g. to record an event."""
        d = self.decode
        w = self.w
        args = (out, d.q, self.k_pool, self.v_pool, d.tables, d.lens_dev, d.max_context_len, w.n_kv_heads,
                w.num_blocks, w.scale)
        if self.fp8:
            args += (self.k_scale, self.v_scale)
        (paged_attention_decode_fp8_partitions if self.fp8 else paged_attention_decode_partitions)(
            *args, workspace=d.workspace, stream=stream)
        if between is not None:
            between()
        (paged_attention_decode_fp8_reduce if self.fp8 else paged_attention_decode_reduce)(
            *args, workspace=d.workspace, stream=stream)

    def append_prefill(self, stream=None):
        p = self.prefill
        T = p.k_new.shape[0]
        self._cache(p.k_new.view(T, -1), p.v_new.view(T, -1), p.slots, stream=stream)

    def attend_prefill(self, out: torch.Tensor, stream=None):
        if self.fp8:
            raise ValueError("chunked prefill reads 16-bit pools")
        p = self.prefill
        w = self.w
        paged_attention_prefill_chunk(out, p.q, self.k_pool, self.v_pool, p.tables, p.cu_q_lens, p.lens_dev,
                                      p.max_q_len, p.max_context_len, w.n_kv_heads, w.num_blocks, w.scale,
                                      stream=stream)

    def attend_verify(self, out: torch.Tensor, stream=None):
        """The chunks' attention through paged_attention_verify (a few query
        tokens per sequence: checking drafted tokens), or its 8-bit variant."""
        p = self.prefill
        w = self.w
        total = int(p.qlen.sum())
        need = paged_attention_verify_workspace_bytes(total, w.n_q_heads, w.head_dim, p.max_context_len)
        if need and (getattr(self, "_verify_ws", None) is None or self._verify_ws.numel() * 4 < need):
            self._verify_ws = torch.empty(need // 4 + 1, dtype=torch.float32, device=self.device)
        ws = self._verify_ws if need else None
        if self.fp8:
            paged_attention_verify_fp8(out, p.q, self.k_pool, self.v_pool, p.tables, p.cu_q_lens, p.lens_dev,
                                       p.max_q_len, p.max_context_len, w.n_kv_heads, w.num_blocks, w.scale,
                                       self.k_scale, self.v_scale, workspace=ws, stream=stream)
        else:
            paged_attention_verify(out, p.q, self.k_pool, self.v_pool, p.tables, p.cu_q_lens, p.lens_dev,
                                   p.max_q_len, p.max_context_len, w.n_kv_heads, w.num_blocks, w.scale, workspace=ws,
                                   stream=stream)

    def new_decode_out(self):
        w = self.w
        return torch.empty((w.n_decode, w.n_q_heads, w.head_dim), dtype=self.out_dtype, device=self.device)

    def new_prefill_out(self):
        w = self.w
        return torch.empty((int(self.prefill.qlen.sum()), w.n_q_heads, w.head_dim), dtype=self.out_dtype,
                           device=self.device)
