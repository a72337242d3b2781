#!/usr/bin/env python3
"""Benchmark of the paged KV-cache decode step on one MI355X.

Workload (default): the Llama-3-8B-shaped decode batch — one layer, 32 query
heads over 8 KV heads, head_dim 128, bf16 K/V, block size 16, 256 sequences
with context lengths uniform in [512, 4096], in groups of 8 that share the
ref-counted blocks of a 1024-token prefix, the rest of the blocks scattered
over a 32768-block pool.  One step = append each sequence's new token
(reshape_and_cache) + paged decode attention (partition pass + split-K
reduce), inputs resident in HBM.

Timing: before every timed step a 1 GiB device read evicts the L2 caches
and the 256 MB Infinity Cache (outside the timed events), so K/V come from
HBM as they would between the layers of a forward pass; each step is
bracketed by HIP events on the stream it runs on.  Prints one JSON line:
decode tokens/s for one layer (batch / mean step time, the step being one
paged_attention_decode_append call, whose cache write rides in the shared-run
launch), with the partition pass's achieved HBM bandwidth against the
8 TB/s peak (the pass is decode_shared_kernel then decode_partition_kernel,
timed together with events in the three-call form of the step).  Beside it:
the same timings with warm caches, read-only bandwidth ceilings over the
batch's tiles, the fp64 oracle timed on the host cores (gather + attention
from host pools, all sequences on one thread per core and a sample on one
thread), the same step over an 8-bit (E4M3) cache, the toy, TinyLlama- and
OPT-13B-shaped decode batches with their own rooflines, the swap copies of 32
sequences, verify attention of 5 new tokens per sequence, and the mixed
chunked-prefill + decode step with the prefill kernel's MFMA fraction.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-fp8] [--no-mixed] ...
  python bench.py --copy-calibration     # plain device copy of a known size
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(b):
    """Algorithmic bytes of one partition-pass launch, and the logical KV bytes.

    Unit = one context token of one KV head: 2 * head_dim * esize bytes of K
    and V (esize 1 for an 8-bit cache).  Physical blocks shared by several sequences count once, with the
    most tokens any sequence reads from them.  Plus q, block-table entries and
    lengths read, and the outputs it writes for single-partition sequences."""
    import numpy as np
    from paged_kv_cache_gather_amd import paged_attention_decode_partition_size
    w, d = b.w, b.decode
    eb = w.elem_bytes
    unit = 2 * w.head_dim * (1 if b.fp8 else eb)
    lens = d.lens.astype(np.int64)
    nb = -(-lens // 16)
    rows = np.repeat(np.arange(w.n_decode), nb)
    idx = np.concatenate([np.arange(n) for n in nb])
    blk = d.tables_host[rows, idx].astype(np.int64)
    valid = np.minimum(16, lens[rows] - 16 * idx)
    best = np.zeros(w.num_blocks, np.int64)
    np.maximum.at(best, blk, valid)
    unique_tokens = int(best.sum())
    logical_tokens = int(lens.sum())
    out_bytes = b.out_dtype.itemsize
    single = int((lens <= paged_attention_decode_partition_size()).sum())
    extra = (w.n_decode * w.n_q_heads * w.head_dim * eb + int(nb.sum()) * 4 + 4 * w.n_decode
             + single * w.n_q_heads * w.head_dim * out_bytes)
    return {
        "unit_bytes": unit * w.n_kv_heads,
        "unique_units": unique_tokens,
        "unique_kv_bytes": unique_tokens * unit * w.n_kv_heads,
        "logical_kv_bytes": logical_tokens * unit * w.n_kv_heads,
        "other_bytes": extra,
        "algorithmic_bytes": unique_tokens * unit * w.n_kv_heads + extra,
    }


def profiled_traffic(profile, sources):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE + WRITE_SIZE
    (scaled by a plain-copy calibration) and recorded in profiles/<profile>.md,
    or None when the kernel sources changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile + ".md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_sources_sha256_16"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    m = hashlib.sha256()
    for src in sources:
        m.update(open(os.path.join(ROOT, "paged_kv_cache_gather_amd", "csrc", src), "rb").read())
    if rec.get("kernel_sources_sha256_16") != m.hexdigest()[:16] or "traffic_bytes_per_launch" not in rec:
        return None
    return int(rec["traffic_bytes_per_launch"])


def prefill_flops(w):
    """Algorithmic FLOPs of one prefill launch: 4 * d * Hq per unmasked
    (query, key) pair (two multiply-adds per dim, for Q K^T and for P V);
    query i of a chunk with c cached tokens sees c + i + 1 keys."""
    import numpy as np
    pairs = 0
    for c, ql in zip(w.chunk_ctx.astype(np.int64), w.chunk_qlen.astype(np.int64)):
        pairs += int(ql * c + ql * (ql + 1) // 2)
    return 4 * w.head_dim * w.n_q_heads * pairs, pairs


WARM_MS = 200.0  # minimum wall time of untimed work before a leg's timed steps


def warm(fn, count, flush=None):
    """`count` untimed calls of fn, then more until they have kept the GPU
    busy for at least WARM_MS of wall time: after host-side work the GPU's
    clocks take tens of milliseconds of load to settle (the first ~20 mixed
    steps after building a batch run ~12 % slower than the rest).  With
    `flush`, each call follows a cache flush as the timed ones do, so every
    launch of the leg sees the same cache state (and a kernel trace's
    averages agree with the timed steps); without it, or with the
    write-flush variant (diagnostic timings that follow a read-flushed leg),
    only the `count` calls run."""
    import torch

    def one():
        if flush is not None:
            flush()
        fn()

    for _ in range(count):
        one()
    torch.cuda.synchronize()
    if flush is None or getattr(flush, "mode", "read") != "read":
        return  # unflushed and write-flushed timings follow a read-flushed leg: the clocks are up already
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < WARM_MS:
        for _ in range(4):
            one()
        torch.cuda.synchronize()


def mixed_step(steps, warmup, seed, flush):
    """The mixed chunked-prefill + decode step (16 chunks of 512 queries and
    240 decodes): append both, then prefill attention and decode attention,
    each timed step after a cache flush."""
    import numpy as np
    import torch
    import synth
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.make_workload("llama3_8b_mixed", seed=seed)
    log(f"building {w.name}: {w.description}")
    b = DeviceBatch(w, "cuda:0", fill="device")
    outp, outd = b.new_prefill_out(), b.new_decode_out()
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]

    def step(e=None):
        rec = (lambda i: e[i].record(st)) if e is not None else (lambda i: None)
        rec(0)
        b.append_prefill()
        b.append_decode()
        rec(1)
        b.attend_prefill(outp)
        rec(2)
        b.attend_decode_split(outd, between=lambda: rec(3))
        rec(4)

    warm(step, warmup, flush)
    for i in range(steps):
        flush()
        step(ev[i])
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[4]) for e in ev]))
    pre = np.array([e[1].elapsed_time(e[2]) for e in ev])
    dpart = np.array([e[2].elapsed_time(e[3]) for e in ev])
    flops, pairs = prefill_flops(w)
    by = decode_bytes(b)
    tf = flops / (pre.mean() * 1e-3) / 1e12
    toks = int(w.chunk_qlen.sum()) + w.n_decode
    log(f"mixed step {ms * 1e3:.1f} us | prefill {pre.mean() * 1e3:.1f} us = {tf:.0f} TFLOP/s "
        f"({tf / MFMA_BF16_PEAK_TFLOPS:.1%} of MFMA peak) | decode partitions {dpart.mean() * 1e3:.1f} us = "
        f"{by['algorithmic_bytes'] / (dpart.mean() * 1e-3) / 1e9:.0f} GB/s")
    return {
        "workload": w.name, "description": w.description, "ms_per_step": ms,
        "tokens_per_step": toks, "tokens_per_s": toks / (ms * 1e-3),
        "prefill": {"kernel": "prefill_chunk_kernel", "bound": "mfma", "us": float(pre.mean()) * 1e3,
                    "algorithmic_flops": flops, "causal_pairs": pairs, "achieved": tf,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": (profiled_traffic("prefill_chunk_llama3_8b_mixed", ["prefill.hip", "pkv_device.h"])
                                if seed == 0 else None)},
        "decode": {"kernel": "decode partition pass (decode_partition_kernel + decode_shared_kernel)",
                   "bound": "hbm", "us": float(dpart.mean()) * 1e3,
                   "algorithmic_bytes": by["algorithmic_bytes"],
                   "achieved": by["algorithmic_bytes"] / (dpart.mean() * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                   "unit": "GB/s",
                   "frac": by["algorithmic_bytes"] / (dpart.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }


def mfma_ceiling_leg(prefill_tflops, iters=2000, reps=5):
    """The matrix-core rate beside the prefill kernel (paged_kv_mfma_rate):
    16x16x32 bf16 MFMAs from one and from two waves per SIMD, one wave per
    SIMD with the softmax's vector mix running on the other, and that vector
    mix alone; one workgroup per CU, best of `reps` launches."""
    import numpy as np
    import torch
    import paged_kv_cache_gather_amd as pkv
    n_wg = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream()
    res = {"kernel": "mfma_rate_kernel", "workgroups": n_wg, "iters": iters}
    names = {0: "one_wave_per_simd", 1: "two_waves_per_simd", 2: "with_softmax_mix_beside", 3: "softmax_mix_alone"}
    for mode, name in names.items():
        pkv.paged_kv_mfma_rate(mode, n_wg, iters, sink)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(st)
            pkv.paged_kv_mfma_rate(mode, n_wg, iters, sink)
            e1.record(st)
        torch.cuda.synchronize()
        us = float(np.min([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
        waves = {0: 4, 1: 8, 2: 4, 3: 0}[mode]
        flops = n_wg * waves * iters * 8 * 16384
        r = {"us": us}
        if flops:
            r["tflops"] = flops / (us * 1e-6) / 1e12
            r["frac_of_peak"] = r["tflops"] / MFMA_BF16_PEAK_TFLOPS
            r["prefill_frac"] = prefill_tflops / r["tflops"]
        res[name] = r
    log("matrix-core rate: " + ", ".join(f"{n} {res[n]['tflops']:.0f} TFLOP/s" for n in names.values()
                                         if "tflops" in res[n])
        + f" | vector mix alone {res['softmax_mix_alone']['us']:.1f} us | prefill {prefill_tflops:.0f} TFLOP/s")
    return res


def sweep_decode(K, W, seed, flush):
    """Decode attention (paged_attention_decode, one call) across batch sizes
    and uniform context lengths: Llama-3-8B heads (Hq 32 / Hkv 8, d 128, bf16),
    no shared prefixes, random block placement, each timed call after a cache
    flush.  The batches at and below 2048 keys with at most 256 (sequence, KV
    head) pairs take the whole-context path."""
    import numpy as np
    import torch
    import synth
    import paged_kv_cache_gather_amd as pkv
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    rows = []
    for B in (32, 64, 128, 256):
        for L in (512, 1024, 2048, 4096, 8192):
            w = synth.custom_workload(f"sweep_b{B}_l{L}", 32, 8, 128, "bf16", B * (L // 16) + 64, seed,
                                      decode_lens=[L] * B)
            b = DeviceBatch(w, "cuda:0", fill="device")
            b.append_decode()
            out = b.new_decode_out()
            us = _stats_us(time_attend(b, out, K, W, flush))["mean"]
            by = decode_bytes(b)["algorithmic_bytes"]
            path = "whole" if pkv.paged_attention_decode_whole_context(B, 32, 8, 128, "bf16", L) else "split"
            rows.append({"B": B, "L": L, "us": us, "bytes": by, "gbs": by / (us * 1e-6) / 1e9, "path": path})
            log(f"decode sweep B={B:4d} L={L:5d}: {us:8.1f} us  {rows[-1]['gbs']:6.0f} GB/s  ({path})")
            del b, out
            torch.cuda.empty_cache()
    return rows


def sweep_prefill(K, W, seed, flush):
    """The chunked-prefill kernel across head shapes: 16 chunks of 512 queries
    over cached contexts U[0, 7680] (numpy's default generator, seed `seed`),
    Hq 32, each timed launch after a cache flush."""
    import numpy as np
    import torch
    import synth
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    ctx = np.random.default_rng(seed).integers(0, 7680 + 1, size=16)
    rows = []
    for name, hkv, d, dt in (("GQA 4 (Hkv 8), d 128, bf16", 8, 128, "bf16"), ("MHA (Hkv 32), d 128, f16", 32, 128, "f16"),
                             ("GQA 2 (Hkv 16), d 128, bf16", 16, 128, "bf16"),
                             ("GQA 16 (Hkv 2), d 128, bf16", 2, 128, "bf16"),
                             ("GQA 8 (Hkv 4), d 64, f16", 4, 64, "f16"), ("GQA 4 (Hkv 8), d 64, bf16", 8, 64, "bf16")):
        nb = int(((ctx + 512 + 15) // 16).sum()) + 64
        w = synth.custom_workload("sweep_prefill", 32, hkv, d, dt, nb, seed, chunk_ctx=ctx, chunk_qlen=[512] * 16)
        b = DeviceBatch(w, "cuda:0", fill="device")
        b.append_prefill()
        out = b.new_prefill_out()
        st = torch.cuda.current_stream()
        warm(lambda: b.attend_prefill(out), W, flush)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for e0, e1 in ev:
            flush()
            e0.record(st)
            b.attend_prefill(out)
            e1.record(st)
        torch.cuda.synchronize()
        us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3
        flops, _ = prefill_flops(w)
        tf = flops / (us * 1e-6) / 1e12
        rows.append({"shape": name, "us": us, "tflops": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS})
        log(f"prefill sweep {name:30s}: {us:8.1f} us  {tf:5.0f} TFLOP/s  {tf / MFMA_BF16_PEAK_TFLOPS:.1%}")
        del b, out
        torch.cuda.empty_cache()
    return rows


def host_allocator_us(b, reps=5):
    """Per-step cost of the host block manager on this batch: append one token
    to every sequence (one batched call, which also returns the slot
    mapping) and export the block tables (median of reps).  Run after the
    timed steps: it advances the host state of b's pool."""
    import numpy as np
    import paged_kv_cache_gather_amd as pkv
    seqs = np.asarray(b.decode.seqs, dtype=np.int64)
    maxb = int(-(-(b.decode.lens.max() + reps) // 16))
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        pkv.paged_kv_seqs_append(b.pool, seqs)
        pkv.paged_kv_block_tables(b.pool, seqs, maxb)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)) * 1e6


def prefix_cache_host(n_req=256, group=8, prefix=1024, lens=(512, 4096), seed=0):
    """Host cost of automatic prefix caching in the block manager: n_req
    requests in groups of `group` whose prompts share a `prefix`-token start
    (the decode batch's sharing structure, prompts of lengths U[lens]); each
    request looks its prompt up, appends the uncached rest with token ids
    (labelling the blocks it fills) and is freed.  The reference model runs
    the same operations beside it."""
    import numpy as np
    import paged_kv_cache_gather_amd as pkv
    from oracle import block_manager as bm
    rng = np.random.default_rng(seed)
    prompts = []
    for g in range(n_req // group):
        base = rng.integers(0, 32000, size=prefix).tolist()
        for _ in range(group):
            L = int(rng.integers(lens[0], lens[1] + 1))
            prompts.append(base[:min(prefix, L - 1)] + rng.integers(0, 32000, size=max(0, L - prefix)).tolist()
                           if L > prefix else base[:L])
    nblocks = sum(-(-len(t) // 16) for t in prompts) + 64
    total_blocks = sum(len(t) // 16 for t in prompts)

    def run_lib():
        pool = pkv.paged_kv_alloc(nblocks, 8, 128, "bf16")
        pkv.paged_kv_prefix_cache_enable(pool)
        t0 = time.perf_counter()
        reused = 0
        for t in prompts:
            sq, n = pkv.paged_kv_seq_create_cached(pool, t)
            pkv.paged_kv_seq_append_tokens(pool, sq, t[n:])
            reused += n
            pkv.paged_kv_seq_free(pool, sq)
        return time.perf_counter() - t0, reused, pkv.paged_kv_prefix_cache_stats(pool)

    def run_model():
        m = bm.BlockManagerModel(nblocks, 16)
        m.enable_caching(True)
        t0 = time.perf_counter()
        reused = 0
        for t in prompts:
            sq, n = m.create_cached(t)
            m.append_tokens(sq, t[n:])
            reused += n
            m.release(sq)
        return time.perf_counter() - t0, reused, m.cache_stats()

    dt, reused, stats = run_lib()
    dtm, reused_m, stats_m = run_model()
    assert reused == reused_m and stats == stats_m
    toks = sum(len(t) for t in prompts)
    return {"requests": len(prompts), "prompt_tokens": toks, "reused_tokens": reused,
            "full_prompt_blocks": total_blocks, "stats": stats,
            "us_per_request": dt / len(prompts) * 1e6, "prompt_tokens_per_s": toks / dt,
            "model_us_per_request": dtm / len(prompts) * 1e6}


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction


def swap_leg(b, n_seqs=32, reps=10):
    """Swap copies (paged_kv_swap_blocks) of the first n_seqs sequences'
    blocks between the HBM pools and pinned host pools, one launch each way,
    timed with HIP events; beside them a plain copy of the same number of
    bytes between a contiguous device buffer and pinned host memory (torch's
    copy_, the runtime's DMA path) as the host link's practical ceiling.
    Swapping in writes the same bytes back into the same blocks, so the batch
    is unchanged."""
    import numpy as np
    import torch
    import paged_kv_cache_gather_amd as pkv
    w, d = b.w, b.decode
    rows = d.tables_host[:n_seqs]
    blocks = np.unique(rows[rows >= 0]).astype(np.int32)
    n = int(blocks.size)
    per = w.n_kv_heads * 16 * w.head_dim
    cpu_k = torch.empty(n * per, dtype=b.k_pool.dtype, pin_memory=True)
    cpu_v = torch.empty(n * per, dtype=b.k_pool.dtype, pin_memory=True)
    idx = np.arange(n, dtype=np.int32)
    p_out = torch.from_numpy(np.stack([blocks, idx], 1)).to("cuda:0")
    p_in = torch.from_numpy(np.stack([idx, blocks], 1)).to("cuda:0")
    nbytes = 2 * n * per * b.k_pool.element_size()
    st = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_out = timed(lambda: pkv.paged_kv_swap_blocks(b.k_pool, b.v_pool, cpu_k, cpu_v, p_out, w.num_blocks, n,
                                                   w.n_kv_heads, w.head_dim))
    t_in = timed(lambda: pkv.paged_kv_swap_blocks(cpu_k, cpu_v, b.k_pool, b.v_pool, p_in, n, w.num_blocks,
                                                  w.n_kv_heads, w.head_dim))
    dev_buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    host_buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    t_d2h = timed(lambda: host_buf.copy_(dev_buf, non_blocking=True))
    t_h2d = timed(lambda: dev_buf.copy_(host_buf, non_blocking=True))
    gb = lambda t: nbytes / t / 1e9
    log(f"swap {n} blocks ({nbytes / 1e6:.0f} MB): out {t_out * 1e3:.2f} ms = {gb(t_out):.1f} GB/s, in "
        f"{t_in * 1e3:.2f} ms = {gb(t_in):.1f} GB/s | contiguous copy d2h {gb(t_d2h):.1f}, h2d {gb(t_h2d):.1f} GB/s")
    return {"kernel": "swap_blocks_kernel", "sequences": n_seqs, "blocks": n, "bytes": nbytes,
            "out_ms": t_out * 1e3, "in_ms": t_in * 1e3, "out_gbs": gb(t_out), "in_gbs": gb(t_in),
            "copy_d2h_gbs": gb(t_d2h), "copy_h2d_gbs": gb(t_h2d), "link_peak_gbs": HOST_LINK_PEAK_GBS,
            "out_frac_of_copy": t_d2h / t_out, "in_frac_of_copy": t_h2d / t_in}


def verify_bytes(b, kv_elem_bytes=None):
    """Algorithmic bytes of one verify launch: every sequence's keys and
    values (its context plus the new tokens) once per KV head (kv_elem_bytes
    per element: 1 for 8-bit pools), the queries, block-table entries, lengths
    and the outputs."""
    import numpy as np
    w, p = b.w, b.prefill
    keys = (p.ctx + p.qlen).astype(np.int64)
    eb = w.elem_bytes
    kb = eb if kv_elem_bytes is None else kv_elem_bytes
    total_q = int(p.qlen.sum())
    kv = int(keys.sum()) * 2 * w.head_dim * kb * w.n_kv_heads
    other = (2 * total_q * w.n_q_heads * w.head_dim * eb + int((-(-keys // 16)).sum()) * 4 + 8 * len(keys))
    return {"unit_bytes": 2 * w.head_dim * kb * w.n_kv_heads, "kv_bytes": kv, "other_bytes": other,
            "algorithmic_bytes": kv + other}


def verify_leg(steps, warmup, seed, flush, k=5):
    """Checking k drafted tokens per sequence (k + 1 - 1 = k new query tokens
    each) on the Llama-3-8B-shaped batch: 256 sequences with the decode
    batch's context lengths; one step = append the new tokens + verify
    attention (paged_attention_verify), timed with HIP events; beside it the
    chunked-prefill kernel on the same batch."""
    import numpy as np
    import torch
    import synth
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    lens = synth.make_workload("llama3_8b_decode", seed).decode_lens
    w = synth.custom_workload("llama3_8b_verify", 32, 8, 128, "bf16", 70000, seed, chunk_ctx=lens - 1,
                              chunk_qlen=np.full(lens.size, k),
                              description=f"Llama-3-8B-shaped verify step: 256 sequences, {k} new tokens each over "
                                          "contexts L-1 with L~U[512,4096], Hq32/Hkv8, d=128, bf16")
    b = DeviceBatch(w, "cuda:0", fill="device")
    out = b.new_prefill_out()
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(e=None):
        rec = (lambda i: e[i].record(st)) if e is not None else (lambda i: None)
        rec(0)
        b.append_prefill()
        rec(1)
        b.attend_verify(out)
        rec(2)
        b.attend_prefill(out)
        rec(3)

    warm(step, warmup, flush)
    for i in range(steps):
        flush()
        step(ev[i])
    torch.cuda.synchronize()
    app = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    ver = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    pre = np.array([e[2].elapsed_time(e[3]) for e in ev]) * 1e3
    by = verify_bytes(b)
    ach = by["algorithmic_bytes"] / (ver.mean() * 1e-6) / 1e9
    toks = int(w.chunk_qlen.sum())
    log(f"verify ({k} tokens x {w.n_chunks} seqs): append {app.mean():.1f} us | verify {ver.mean():.1f} us = "
        f"{ach:.0f} GB/s ({ach / HBM_PEAK_GBS:.1%}) | same batch through the prefill kernel {pre.mean():.1f} us")
    res = {"workload": w.name, "description": w.description, "new_tokens_per_seq": k,
           "step_us": float(app.mean() + ver.mean()), "tokens_per_s": toks / ((app.mean() + ver.mean()) * 1e-6),
           "breakdown_us": {"append": float(app.mean()), "verify": float(ver.mean()),
                            "prefill_kernel_same_batch": float(pre.mean())},
           "roofline": {"bound": "hbm", "kernel": "verify_partition_kernel + decode_reduce_kernel",
                        "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                        "traffic": (profiled_traffic("verify_llama3_8b_verify", ["decode.hip", "pkv_device.h"])
                                    if seed == 0 else None),
                        "algorithmic_bytes": by["algorithmic_bytes"]},
           "bytes": by}
    del b, out
    torch.cuda.empty_cache()
    res["fp8"] = verify_fp8(w, steps, warmup, flush)
    return res


def verify_fp8(w, steps, warmup, flush):
    """The same verify step over 8-bit (E4M3) pools: the new rows quantised
    by reshape_and_cache_fp8, then paged_attention_verify_fp8."""
    import numpy as np
    import torch
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(w, "cuda:0", fill="device", kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    out = b.new_prefill_out()
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

    def step(e=None):
        rec = (lambda i: e[i].record(st)) if e is not None else (lambda i: None)
        rec(0)
        b.append_prefill()
        rec(1)
        b.attend_verify(out)
        rec(2)

    warm(step, warmup, flush)
    for i in range(steps):
        flush()
        step(ev[i])
    torch.cuda.synchronize()
    app = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    ver = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    by = verify_bytes(b, kv_elem_bytes=1)
    ach = by["algorithmic_bytes"] / (ver.mean() * 1e-6) / 1e9
    toks = int(w.chunk_qlen.sum())
    log(f"verify over 8-bit pools: append {app.mean():.1f} us | verify {ver.mean():.1f} us = {ach:.0f} GB/s "
        f"({ach / HBM_PEAK_GBS:.1%})")
    res = {"kv_cache": "fp8_e4m3", "step_us": float(app.mean() + ver.mean()),
           "tokens_per_s": toks / ((app.mean() + ver.mean()) * 1e-6),
           "breakdown_us": {"append": float(app.mean()), "verify": float(ver.mean())},
           "roofline": {"bound": "hbm", "kernel": "verify_partition_kernel<FP8, ...> + decode_reduce_kernel",
                        "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                        "traffic": (profiled_traffic("verify_fp8_llama3_8b_verify", ["decode.hip", "pkv_device.h"])
                                    if w.seed == 0 else None),
                        "algorithmic_bytes": by["algorithmic_bytes"]},
           "bytes": by}
    del b, out
    torch.cuda.empty_cache()
    return res


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, tables, sample_1thread=32):
    """The fp64 oracle as it stands, timed on the host: for each decode
    sequence, gather its K/V from host copies of the pools through its block
    table (oracle.gather) and run the attention (oracle.attention).  The host
    pools are written by the oracle's own scatter from the seeded generator's
    rows (not timed).  Timed twice: every sequence with one worker thread per
    host core (at most 16: the host cores one GPU of the node is allotted), and a
    sample on one thread."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    threads = max(1, min(os.cpu_count() or 1, 16))
    H, d, bs = w.n_kv_heads, w.head_dim, 16
    pool_elems = w.num_blocks * H * bs * d
    cont = np.uint32 if w.dtype == "f32" else np.uint16
    kp, vp = np.zeros(pool_elems, cont), np.zeros(pool_elems, cont)
    lens = w.decode_lens.astype(np.int64)

    def fill(s):
        L = int(lens[s])
        k, v = w.kv("decode", s, 0, L)
        t = np.arange(L)
        slots = tables[s, t // bs].astype(np.int64) * bs + t % bs
        oracle.scatter(w.dtype, k, v, kp, vp, slots, w.num_blocks, bs, H, d)
        return oracle.decode(w.dtype, w.q("decode", s, L - 1, L))

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        qs = list(ex.map(fill, range(w.n_decode)))  # shared prefix blocks get the same bytes from every member
    t_fill = time.perf_counter() - t0

    def one(s):
        L = int(lens[s])
        k, v = oracle.gather(w.dtype, kp, vp, w.num_blocks, bs, H, d, tables[s, :-(-L // bs)], L)
        out, _ = oracle.attention(qs[s], [L - 1], k, v, w.scale)
        return out

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(w.n_decode)))
    t_all = time.perf_counter() - t0
    stride = max(1, w.n_decode // sample_1thread)
    sample = list(range(0, w.n_decode, stride))[:sample_1thread]
    t0 = time.perf_counter()
    for s in sample:
        one(s)
    t_one = time.perf_counter() - t0
    toks = int(lens.sum())
    log(f"oracle: {w.n_decode} sequences on {threads} threads in {t_all:.2f} s "
        f"({w.n_decode / t_all:.1f} tokens/s); {len(sample)} on 1 thread in {t_one:.2f} s "
        f"({len(sample) / t_one:.2f} tokens/s); host cores {os.cpu_count()} ({_cpu_model()})")
    return {"value": w.n_decode / t_all, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"all {w.n_decode} decode sequences of {w.name} ({toks} context tokens): fp64 gather "
                      f"from host pools through the block tables + attention, one worker thread per core, "
                      f"{t_all:.2f} s",
            "host_cpu_count": os.cpu_count(), "cpu_model": _cpu_model(),
            "one_thread": {"value": len(sample) / t_one, "unit": "tokens/s", "cores": 1,
                           "sample": f"{len(sample)} sequences (every {stride}th), {t_one:.2f} s"},
            "host_pool_fill_s": t_fill}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes x5")


class CacheFlush:
    """Evicts L2 (8 x 4 MB) and the 256 MB Infinity Cache before a timed
    step, outside the timed events, so the step reads its K/V from HBM as it
    would between the layers of a forward pass.  The default reads a 1 GiB
    device buffer (paged_kv_read_tiles, contiguous, plain loads): the caches
    end up full of clean lines of unrelated data.  mode="write" writes the buffer instead,
    which also evicts but leaves up to ~290 MB of dirty lines that are
    written back while the timed step runs (reported beside the headline,
    not as it)."""

    def __init__(self, device="cuda:0", nbytes=1 << 30, mode="read"):
        import torch
        self.buf = torch.ones(nbytes, dtype=torch.uint8, device=device)
        self.sink = torch.zeros(1, dtype=torch.int32, device=device)
        self.mode = mode
        self.i = 0

    def __call__(self):
        import paged_kv_cache_gather_amd as pkv
        if self.mode == "write":
            self.i ^= 1
            self.buf.fill_(self.i)
        else:
            n = self.buf.numel() // 4096
            pkv.paged_kv_read_tiles(self.buf, None, None, n, n, 4096, self.sink, streaming=False)


def _stats_us(ms):
    import numpy as np
    us = np.asarray(ms) * 1e3
    return {"mean": float(us.mean()), "median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90))}


def time_decode(b, out, K, W, flush=None):
    """W untimed then K timed decode steps of batch b as three calls: append
    the new tokens, then the partition pass and the reduce, with HIP events
    between them on the stream they run on.  With flush, the caches are
    flushed before every step (outside the events)."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        b.append_decode()
        if e is not None:
            e[1].record(stream)
        b.attend_decode_split(out, between=(lambda: e[2].record(stream)) if e is not None else None)
        if e is not None:
            e[3].record(stream)

    warm(step, W, flush)
    t0 = time.perf_counter()
    for i in range(K):
        if flush is not None:
            flush()
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return {"wall_ms_step": (t1 - t0) * 1e3 / K,
            "step_ms": np.array([ev[i][0].elapsed_time(ev[i][3]) for i in range(K)]),
            "part_ms": np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]),
            "append_ms": np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]),
            "reduce_ms": np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)])}


def time_attend(b, out, K, W, flush=None):
    """K timed one-call decode attentions (paged_attention_decode, no cache
    write), each after a cache flush when given: the whole-context path's
    single launch."""
    import numpy as np
    import torch
    st = torch.cuda.current_stream()
    warm(lambda: b.attend_decode(out), W, flush)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for e0, e1 in ev:
        if flush is not None:
            flush()
        e0.record(st)
        b.attend_decode(out)
        e1.record(st)
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) for e0, e1 in ev])


def fused_step(b, out, K, W, flush):
    """The step in one call (paged_attention_decode_append or its 8-bit
    variant: the new rows' cache write rides in the shared-run launch, then
    the per-sequence pass and the merge).  Timed three ways: K eager steps,
    each after a cache flush, with HIP events around each step (the
    headline); K eager steps back to back, wall clock between two
    synchronisations (caches warm from the previous step); and the step
    captured once in a HIP graph, replayed K times after flushes (events)."""
    import numpy as np
    import torch
    st = torch.cuda.current_stream()
    warm(lambda: b.step_decode(out), W, flush)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        flush()
        ev[i][0].record(st)
        b.step_decode(out)
        ev[i][1].record(st)
    torch.cuda.synchronize()
    flushed = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    t0 = time.perf_counter()
    for _ in range(K):
        b.step_decode(out)
    torch.cuda.synchronize()
    warm_us = (time.perf_counter() - t0) * 1e6 / K
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.step_decode(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.step_decode(out)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    for i in range(K):
        flush()
        ev[i][0].record(st)
        graph.replay()
        ev[i][1].record(st)
    torch.cuda.synchronize()
    graph_flushed = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    return {"flushed_us": _stats_us(flushed), "back_to_back_wall_us": warm_us,
            "graph_flushed_us": _stats_us(graph_flushed)}


# scales of the 8-bit leg: the synthetic values are standard normal quantiles
# (|x| < 4.4), which these map inside E4M3's +-448
FP8_K_SCALE, FP8_V_SCALE = 0.0125, 0.0103


def decode_leg(w, K, W, out_dtype, seed, flush, fp8=False, modes=True, profile=None):
    """One decode workload: build the batch on the device, then time the
    step.  The step is one paged_attention_decode_append call (or its 8-bit
    variant), K times after a cache flush each, with HIP events around each
    step: tokens/s = B / mean step time.  The three-call form (append,
    partition pass, merge, events between them) gives the breakdown and the
    partition pass's roofline, flushed as well; the same without flushes and
    the one call back to back (wall clock) and from a HIP graph are reported
    beside it."""
    import torch
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    kw = dict(kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE) if fp8 else {}
    log(f"building {w.name}{' (8-bit cache)' if fp8 else ''}: {w.description}")
    b = DeviceBatch(w, "cuda:0", fill="device", out_dtype=out_dtype, **kw)
    out = b.new_decode_out()
    import paged_kv_cache_gather_amd as pkv
    whole = pkv.paged_attention_decode_whole_context(
        w.n_decode, w.n_q_heads, w.n_kv_heads, w.head_dim, "fp8_e4m3" if fp8 else w.dtype, b.decode.max_context_len)
    t = time_decode(b, out, K, W, flush)
    warm3 = time_decode(b, out, K, 2)
    by = decode_bytes(b)
    split_part = _stats_us(t["part_ms"])
    if whole:
        # the one-call forms take the whole-context path: its single launch
        # is the pass; the split path's partition pass is reported beside it
        part_ms = time_attend(b, out, K, W, flush)
        warm_ms = time_attend(b, out, K, 2)
        wflush_ms = time_attend(b, out, K, 2, CacheFlush(mode="write") if flush is not None else None)
    else:
        part_ms = t["part_ms"]
        warm_ms = warm3["part_ms"]
        wflush_ms = time_decode(b, out, K, 2, CacheFlush(mode="write") if flush is not None else None)["part_ms"]
    part = _stats_us(part_ms)
    achieved = by["algorithmic_bytes"] / (part["mean"] * 1e-6) / 1e9
    warm_part = _stats_us(warm_ms)
    g = fused_step(b, out, K, W, flush) if modes else None
    step_us = g["flushed_us"]["mean"] if g else _stats_us(t["step_ms"])["mean"]
    tok_s = w.n_decode / (step_us * 1e-6)
    log(f"{w.name}{' fp8' if fp8 else ''}: step {step_us:.1f} us ({tok_s / 1e6:.3f} M tokens/s, flushed) | "
        f"{'whole-context launch' if whole else 'partitions'} {part['mean']:.1f} us = {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBS:.1%}; caches warm: "
        f"{warm_part['mean']:.1f} us) | append {t['append_ms'].mean() * 1e3:.1f} | reduce "
        f"{t['reduce_ms'].mean() * 1e3:.1f} us" + (f" | back to back {g['back_to_back_wall_us']:.1f} us, graph "
                                                   f"{g['graph_flushed_us']['mean']:.1f} us" if g else "")
        + (f" | split path's partitions {split_part['mean']:.1f} us" if whole else ""))
    kernel = ("decode_whole_kernel (whole-context path: one launch)" if whole else
              "decode partition pass (decode_shared_kernel + " +
              ("decode_fp8_partition_kernel)" if fp8 else "decode_partition_kernel)"))
    res = {
        "workload": w.name, "description": w.description, "batch": w.n_decode,
        "kv_cache": "fp8_e4m3 (OCP E4M3, one fp32 scale per pool)" if fp8 else w.dtype,
        "out_dtype": str(b.out_dtype).replace("torch.", ""),
        "step": ((("paged_attention_decode_fp8_append" if fp8 else "paged_attention_decode_append") +
                  (" (cache write, then the whole-context launch)" if whole else
                   " (cache write + partition pass + split-K reduce in one call)")) if g else
                 "cache write, partition pass, reduce (three calls)"),
        "path": "whole-context" if whole else "split-context",
        "us_per_step": step_us, "tokens_per_s": tok_s,
        "timing": {"caches": "1 GiB read through the caches before every timed step (outside the events)",
                   "one_call_flushed_us": g["flushed_us"] if g else None,
                   "one_call_back_to_back_wall_us": g["back_to_back_wall_us"] if g else None,
                   "one_call_graph_flushed_us": g["graph_flushed_us"] if g else None,
                   "three_calls_flushed_us": _stats_us(t["step_ms"]),
                   "three_calls_warm_us": _stats_us(warm3["step_ms"])},
        "breakdown_us": {"append": float(t["append_ms"].mean()) * 1e3, "partitions": split_part["mean"],
                         "reduce": float(t["reduce_ms"].mean()) * 1e3,
                         **({"whole_context_launch": part["mean"]} if whole else {})},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (profiled_traffic(profile, ["decode.hip", "pkv_device.h"])
                                 if profile and seed == 0 else None),
                     "algorithmic_bytes": by["algorithmic_bytes"], "launch_us": part,
                     "caches_warm": {"launch_us": warm_part,
                                     "achieved": by["algorithmic_bytes"] / (warm_part["mean"] * 1e-6) / 1e9},
                     "after_write_flush": {"launch_us": _stats_us(wflush_ms),
                                           "achieved": by["algorithmic_bytes"] /
                                           (float(wflush_ms.mean()) * 1e-3) / 1e9}},
        "bytes": by,
        "logical_gbs": (by["logical_kv_bytes"] + by["other_bytes"]) / (part["mean"] * 1e-6) / 1e9,
    }
    if fp8:
        res["k_scale"], res["v_scale"] = FP8_K_SCALE, FP8_V_SCALE
    return b, out, res


def ceiling_leg(b, K, flush, part_achieved):
    """Read-only passes beside the decode pass (paged_kv_read_tiles): every
    (block, KV head) tile the batch's tables name, read once (K tiles, then V
    tiles), in table order and in a random order, and the same number of
    tiles from the start of each pool (contiguous bytes); each timed K times
    after a cache flush.  They give
    what the chip delivers for this access pattern with no arithmetic."""
    import numpy as np
    import torch
    import paged_kv_cache_gather_amd as pkv
    w, d = b.w, b.decode
    nb = -(-d.lens.astype(np.int64) // 16)
    blocks = np.concatenate([d.tables_host[s, :nb[s]] for s in range(w.n_decode)]).astype(np.int64)
    _, first = np.unique(blocks, return_index=True)
    uniq = blocks[np.sort(first)]
    tiles = (uniq[:, None] * w.n_kv_heads + np.arange(w.n_kv_heads)).reshape(-1)
    n_k = tiles.size
    tile_bytes = 16 * w.head_dim * b.k_pool.element_size()
    nbytes = 2 * n_k * tile_bytes
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    perm = np.random.default_rng(1).permutation(n_k)
    lists = {"table_order": np.concatenate([tiles, tiles]),
             "random_order": np.concatenate([tiles[perm], tiles[perm]])}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for e0, e1 in ev:
            flush()
            e0.record(st)
            fn()
            e1.record(st)
        torch.cuda.synchronize()
        return _stats_us([e0.elapsed_time(e1) for e0, e1 in ev])

    res = {"kernel": "read_tiles_kernel", "loads": "streaming (nontemporal), as the decode kernels read K/V",
           "tiles": int(2 * n_k), "tile_bytes": tile_bytes, "bytes": nbytes}
    for name, lst in lists.items():
        dev = torch.from_numpy(lst).to("cuda:0")
        t = timed(lambda: pkv.paged_kv_read_tiles(b.k_pool, b.v_pool, dev, n_k, 2 * n_k, tile_bytes, sink))
        res[name] = {"us": t, "gbs": nbytes / (t["mean"] * 1e-6) / 1e9}
        if name == "table_order":  # the same pass with plain loads
            t = timed(lambda: pkv.paged_kv_read_tiles(b.k_pool, b.v_pool, dev, n_k, 2 * n_k, tile_bytes, sink,
                                                      streaming=False))
            res["table_order_plain_loads"] = {"us": t, "gbs": nbytes / (t["mean"] * 1e-6) / 1e9}
    # the same number of tiles from the start of each pool: contiguous bytes
    ident = torch.arange(n_k, dtype=torch.int64, device="cuda:0").repeat(2)
    t = timed(lambda: pkv.paged_kv_read_tiles(b.k_pool, b.v_pool, ident, n_k, 2 * n_k, tile_bytes, sink))
    res["contiguous"] = {"us": t, "gbs": nbytes / (t["mean"] * 1e-6) / 1e9}
    for name in ("table_order", "random_order", "contiguous"):
        if name in res:
            res[name]["decode_pass_frac"] = part_achieved / res[name]["gbs"]
    log("read ceilings: " + ", ".join(f"{n} {res[n]['gbs']:.0f} GB/s" for n in ("table_order", "random_order",
                                                                                 "contiguous", "table_order_plain_loads")
                                        if n in res)
        + f" ({nbytes / 1e9:.3f} GB) | decode pass {part_achieved:.0f} GB/s")
    return res


def main():
    global WARM_MS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-ms", type=float, default=WARM_MS,
                    help="after the W warmup steps, keep warming each leg until this much wall time has passed")
    ap.add_argument("--workload", default="llama3_8b_decode",
                    choices=["tinyllama_decode", "llama3_8b_decode", "opt13b_decode"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out-dtype", default="kv", choices=["kv", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed prefill+decode step")
    ap.add_argument("--only-mixed", action="store_true", help="run only the mixed prefill+decode step")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit-cache decode leg")
    ap.add_argument("--no-swap", action="store_true", help="skip the swap-copy leg")
    ap.add_argument("--no-verify", action="store_true", help="skip the verify-attention leg")
    ap.add_argument("--only-verify", action="store_true", help="run only the verify-attention leg")
    ap.add_argument("--sweep", choices=("decode", "prefill"),
                    help="time decode across batch sizes and context lengths, or prefill across head shapes, "
                         "and print one JSON line of rows (not the benchmark line)")
    ap.add_argument("--only-fp8", action="store_true", help="run only the 8-bit-cache decode leg")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the toy, TinyLlama- and OPT-13B-shaped decode legs")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the read-only bandwidth ceilings")
    ap.add_argument("--no-step-modes", action="store_true",
                    help="time only the three-call step (no one-call or graph runs; for kernel profiles)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: this library has no multi-GPU path "
                                   "(decode would shard by sequence or by KV head with no exchange)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import synth

    if args.copy_calibration:
        copy_calibration()
        return
    flush = CacheFlush()
    WARM_MS = args.warm_ms
    K, W = args.steps, args.warmup
    out_dtype = None if args.out_dtype == "kv" else "f32"
    if args.only_mixed:
        r = mixed_step(args.steps, args.warmup, args.seed, flush)
        if not args.no_ceilings:
            r["mfma_ceiling"] = mfma_ceiling_leg(r["prefill"]["achieved"])
        print(json.dumps(r), flush=True)
        return
    if args.sweep:
        fn = sweep_decode if args.sweep == "decode" else sweep_prefill
        print(json.dumps({"sweep": args.sweep, "rows": fn(K, W, args.seed, flush)}), flush=True)
        return
    if args.only_verify:
        print(json.dumps(verify_leg(args.steps, args.warmup, args.seed, flush)), flush=True)
        return
    w = synth.make_workload(args.workload, seed=args.seed)
    profile = {n: "decode_partition_" + n for n in ("llama3_8b_decode", "opt13b_decode")}
    profile["tinyllama_decode"] = "decode_whole_tinyllama_decode"  # the whole-context path
    if args.only_fp8:
        b, _, r = decode_leg(w, K, W, out_dtype, args.seed, flush, fp8=True, modes=not args.no_step_modes,
                             profile="decode_fp8_partition_llama3_8b_decode" if args.workload == "llama3_8b_decode" else None)
        print(json.dumps(r), flush=True)
        return

    t_build = time.perf_counter()
    b, out, head = decode_leg(w, K, W, out_dtype, args.seed, flush, modes=not args.no_step_modes,
                              profile=profile[args.workload])
    log(f"built and timed in {time.perf_counter() - t_build:.1f} s")
    by = head["bytes"]
    res = {
        "metric": "paged-attn decode tokens/sec and achieved HBM GB/s (% of peak), 1 GPU",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "warmup_min_ms": WARM_MS,
        "ms_per_step": head["us_per_step"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "layers": 1,
                   "batch": w.n_decode, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "out_dtype": head["out_dtype"], "seed": args.seed, "step": head["step"],
                   "timing": "each timed step follows a 1 GiB device read that evicts L2 and the Infinity "
                             "Cache; HIP events around each step; value = batch / mean step time"},
        "roofline": head["roofline"],
        "breakdown_us": dict(head["breakdown_us"], host_allocator_step=host_allocator_us(b)),
        "timing": head["timing"],
        "bytes": by,
        "logical_gbs": head["logical_gbs"],
        "prefix_cache_host": prefix_cache_host(),
    }
    if not args.no_ceilings:
        res["read_ceilings"] = ceiling_leg(b, K, flush, head["roofline"]["achieved"])
    if not args.no_swap:
        res["swap"] = swap_leg(b)
    tables = b.decode.tables_host
    del b, out
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, tables)
    if not args.no_fp8:
        b, _, r = decode_leg(w, K, W, out_dtype, args.seed, flush, fp8=True, modes=not args.no_step_modes,
                             profile="decode_fp8_partition_llama3_8b_decode" if args.workload == "llama3_8b_decode" else None)
        if not args.no_ceilings:  # the same read-only passes over the 8-bit tiles (2 KiB at head_dim 128)
            r["read_ceilings"] = ceiling_leg(b, K, flush, r["roofline"]["achieved"])
        res["fp8_kv_decode"] = r
        del b
        torch.cuda.empty_cache()
    if not args.no_other_workloads:
        res["other_workloads"] = {}
        for name in ("toy_f32_decode", "tinyllama_decode", "llama3_8b_decode", "opt13b_decode"):
            if name == args.workload:
                continue
            wo = synth.make_workload(name, seed=args.seed)
            b, _, r = decode_leg(wo, K, W, out_dtype, args.seed, flush, modes=not args.no_step_modes,
                                 profile=profile.get(name))
            if not args.no_ceilings and wo.dtype != "f32":
                r["read_ceilings"] = ceiling_leg(b, K, flush, r["roofline"]["achieved"])
            tables = b.decode.tables_host
            del b
            torch.cuda.empty_cache()
            if not args.no_cpu_baseline:
                r["cpu_baseline"] = cpu_baseline(wo, tables)
            res["other_workloads"][wo.name] = r
    if not args.no_verify:
        res["verify"] = verify_leg(max(5, K // 2), max(2, W // 2), args.seed, flush)
    if not args.no_mixed:
        res["mixed_step"] = mixed_step(max(5, K // 2), max(2, W // 2), args.seed, flush)
        if not args.no_ceilings:
            res["mixed_step"]["mfma_ceiling"] = mfma_ceiling_leg(res["mixed_step"]["prefill"]["achieved"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
