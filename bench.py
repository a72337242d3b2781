#!/usr/bin/env python3
"""Benchmark of the paged KV-cache decode step on one MI355X.

Workload (default): the Llama-3-8B-shaped decode batch — one layer, 32 query
heads over 8 KV heads, head_dim 128, bf16 K/V, block size 16, 256 sequences
with context lengths uniform in [512, 4096], in groups of 8 that share the
ref-counted blocks of a 1024-token prefix, the rest of the blocks scattered
over a 32768-block pool.  One step = append each sequence's new token
(reshape_and_cache) + paged decode attention (partition pass + split-K
reduce), inputs resident in HBM.

Prints one JSON line: decode tokens/s (one layer; the step as one
paged_attention_decode_append call, whose cache write rides in the
shared-run launch — the three separate calls and the one call replayed from
a HIP graph are reported beside it) with the partition pass's achieved HBM bandwidth
against the 8 TB/s peak, and the fp64 oracle timed on a bounded sample of the
same batch on the host cores.  The partition pass is
two kernels queued back to back on the caller's stream: decode_shared_kernel
(partitions whose blocks neighbouring sequences share, read once for all of
them) and decode_partition_kernel (every other partition); it is timed with
HIP events around the whole pass.  The JSON also carries the same step over
an 8-bit (E4M3) cache (fp8_kv_decode: rows quantised on the way in, half the
bytes per step), the swap copies of 32 sequences between HBM and pinned host
blocks (swap), verify attention of 5 new tokens per sequence (verify), and
the mixed chunked-prefill + decode step.

  python bench.py [--steps K] [--warmup W] [--workload 2|3|4] [--no-cpu-baseline] [--no-fp8] [--no-mixed]
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


def mixed_step(steps, warmup, seed):
    """The mixed chunked-prefill + decode step (16 chunks of 512 queries and
    240 decodes): append both, then prefill attention and decode attention."""
    import numpy as np
    import torch
    import synth
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.make_workload(5, seed=seed)
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
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


def verify_leg(steps, warmup, seed, k=5):
    """Checking k drafted tokens per sequence (k + 1 - 1 = k new query tokens
    each) on the Llama-3-8B-shaped batch: 256 sequences with the decode
    batch's context lengths; one step = append the new tokens + verify
    attention (paged_attention_verify), timed with HIP events; beside it the
    chunked-prefill kernel on the same batch."""
    import numpy as np
    import torch
    import synth
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    lens = synth.make_workload(3, seed).decode_lens
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    for i in range(steps):
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
    res["fp8"] = verify_fp8(w, steps, warmup)
    return res


def verify_fp8(w, steps, warmup):
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    for i in range(steps):
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
                        "traffic": None, "algorithmic_bytes": by["algorithmic_bytes"]},
           "bytes": by}
    del b, out
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, n_seqs):
    """The fp64 oracle (as it stands) on every k-th sequence of the batch."""
    import numpy as np
    import oracle
    threads = max(1, min(os.cpu_count() or 1, 16))
    stride = max(1, w.n_decode // n_seqs)
    sample = list(range(0, w.n_decode, stride))[:n_seqs]
    inputs = []
    for s in sample:
        L = int(w.decode_lens[s])
        k, v = w.kv("decode", s, 0, L)
        inputs.append((w.q("decode", s, L - 1, L), k, v, L))
    t0 = time.perf_counter()
    for q, k, v, L in inputs:
        oracle.attention(oracle.decode(w.dtype, q), [L - 1], oracle.decode(w.dtype, k), oracle.decode(w.dtype, v),
                         w.scale, n_threads=threads)
    dt = time.perf_counter() - t0
    toks = int(sum(x[3] for x in inputs))
    return {"value": len(sample) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(sample)} of {w.n_decode} decode sequences (every {stride}th, {toks} context "
                      f"tokens), fp64 decode+attention from contiguous K/V, {dt:.2f} s"}


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes x5")


def time_decode(b, out, K, W):
    """W untimed then K timed decode steps of batch b: append the new tokens,
    then the partition pass and the reduce, with HIP events between them on
    the stream they run on."""
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

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return {"ms_step": (t1 - t0) * 1e3 / K,
            "part_ms": np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]),
            "append_ms": np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]),
            "reduce_ms": np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)])}


def fused_step(b, out, K, W):
    """The step in one call (paged_attention_decode_append: the new rows'
    cache write rides in the shared-run launch, then the per-sequence pass and
    the merge): W untimed and K timed eager steps, then the same step captured
    once in a HIP graph and replayed K times back to back, each timed as wall
    clock between two synchronisations (HIP events around the replays too)."""
    import torch
    for _ in range(W):
        b.step_decode(out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        b.step_decode(out)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) * 1e6 / K
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / K
    return {"us_per_step": us, "event_us_per_step": e0.elapsed_time(e1) * 1e3 / K,
            "tokens_per_s": b.w.n_decode / (us * 1e-6), "steps": K, "eager_us_per_step": eager_us}


# scales of the 8-bit leg: the synthetic values are standard normal quantiles
# (|x| < 4.4), which these map inside E4M3's +-448
FP8_K_SCALE, FP8_V_SCALE = 0.0125, 0.0103


def fp8_decode_leg(w, K, W, out_dtype, seed, modes=True):
    """The same decode step over an 8-bit (E4M3) cache: the new rows are
    quantised on the way in, the partition pass reads half the bytes
    (decode_shared_kernel + decode_fp8_partition_kernel).  The step is one
    paged_attention_decode_fp8_append call (the quantising write rides in the
    shared-run launch); the three-call run (reshape_and_cache_fp8, partition
    pass, merge, with events between them) gives the breakdown and the
    roofline."""
    import torch
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(w, "cuda:0", fill="device", out_dtype=out_dtype, kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE,
                    v_scale=FP8_V_SCALE)
    out = b.new_decode_out()
    t = time_decode(b, out, K, W)
    by = decode_bytes(b)
    part_us = float(t["part_ms"].mean()) * 1e3
    achieved = by["algorithmic_bytes"] / (part_us * 1e-6) / 1e9
    ms_step = t["ms_step"]
    g = fused_step(b, out, K, W) if modes else None
    if g:
        ms_step = g["eager_us_per_step"] * 1e-3
    log(f"fp8 cache: step {ms_step * 1e3:.1f} us | three calls {t['ms_step'] * 1e3:.1f} us: append "
        f"{t['append_ms'].mean() * 1e3:.1f} us | partitions {part_us:.1f} us = {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBS:.1%}) | reduce {t['reduce_ms'].mean() * 1e3:.1f} us")
    res = {"kv_cache": "fp8_e4m3 (OCP E4M3, one fp32 scale per pool)", "k_scale": FP8_K_SCALE,
           "v_scale": FP8_V_SCALE, "ms_per_step": ms_step, "tokens_per_s": w.n_decode / (ms_step * 1e-3),
           "step": ("paged_attention_decode_fp8_append" if g else
                    "reshape_and_cache_fp8, then paged_attention_decode_fp8 (three calls)"),
           "step_modes": ({"one_call_ms": ms_step, "one_call_graph_replay_ms": g["us_per_step"] * 1e-3,
                           "three_calls_ms": t["ms_step"]} if g else {"three_calls_ms": t["ms_step"]}),
           "breakdown_us": {"append": float(t["append_ms"].mean()) * 1e3, "partitions": part_us,
                            "reduce": float(t["reduce_ms"].mean()) * 1e3},
           "roofline": {"bound": "hbm", "kernel": "decode partition pass, 8-bit cache "
                                                  "(decode_fp8_partition_kernel + decode_shared_kernel)",
                        "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                        "traffic": (profiled_traffic("decode_fp8_partition_llama3_8b_decode",
                                                     ["decode.hip", "pkv_device.h"])
                                    if w.name == "llama3_8b_decode" and seed == 0 else None),
                        "algorithmic_bytes": by["algorithmic_bytes"]},
           "bytes": by}
    del b
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out-dtype", default="kv", choices=["kv", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=256)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed prefill+decode step")
    ap.add_argument("--only-mixed", action="store_true", help="run only the mixed prefill+decode step")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit-cache decode leg")
    ap.add_argument("--no-swap", action="store_true", help="skip the swap-copy leg")
    ap.add_argument("--no-verify", action="store_true", help="skip the verify-attention leg")
    ap.add_argument("--only-verify", action="store_true", help="run only the verify-attention leg")
    ap.add_argument("--only-fp8", action="store_true", help="run only the 8-bit-cache decode leg")
    ap.add_argument("--no-step-modes", action="store_true",
                    help="time only the three-call step (no one-call or graph runs; for kernel profiles)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: this library has no multi-GPU path "
                                   "(decode shards by sequence or KV head with no exchange; see DESIGN.md)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from paged_kv_cache_gather_amd.batch import DeviceBatch

    if args.copy_calibration:
        copy_calibration()
        return

    if args.only_mixed:
        print(json.dumps(mixed_step(args.steps, args.warmup, args.seed)), flush=True)
        return
    if args.only_verify:
        print(json.dumps(verify_leg(args.steps, args.warmup, args.seed)), flush=True)
        return

    w = synth.make_workload(args.workload, seed=args.seed)
    if args.only_fp8:
        print(json.dumps(fp8_decode_leg(w, args.steps, args.warmup, None if args.out_dtype == "kv" else "f32",
                                        args.seed, not args.no_step_modes)), flush=True)
        return
    log(f"building {w.name}: {w.description}")
    t_build = time.perf_counter()
    b = DeviceBatch(w, "cuda:0", fill="device", out_dtype=None if args.out_dtype == "kv" else "f32")
    log(f"built in {time.perf_counter() - t_build:.1f} s")
    out = b.new_decode_out()
    K, W = args.steps, args.warmup
    t = time_decode(b, out, K, W)
    ms_step, part_ms, append_ms, reduce_ms = t["ms_step"], t["part_ms"], t["append_ms"], t["reduce_ms"]
    by = decode_bytes(b)
    part_s = float(part_ms.mean()) * 1e-3
    achieved = by["algorithmic_bytes"] / part_s / 1e9
    logical = (by["logical_kv_bytes"] + by["other_bytes"]) / part_s / 1e9
    # the headline: the step in one call (K steps between two
    # synchronisations); the eager run above, three calls with events between
    # them, gives the breakdown and the partition pass's roofline; the one
    # call replayed from a HIP graph is reported beside it
    eager_ms_step = ms_step
    g = None
    if not args.no_step_modes:
        g = fused_step(b, out, K, W)
        ms_step = g["eager_us_per_step"] * 1e-3
    tok_s = w.n_decode / (ms_step * 1e-3)
    if g:
        log(f"step in one call {g['eager_us_per_step']:.1f} us ({tok_s / 1e6:.3f} M tokens/s) | replayed from a "
            f"HIP graph {g['us_per_step']:.1f} us | three calls {eager_ms_step * 1e3:.1f} us")
    log(f"eager three-call step {eager_ms_step * 1e3:.1f} us | append {append_ms.mean() * 1e3:.1f} us | partitions "
        f"{part_ms.mean() * 1e3:.1f} us (p10 {np.percentile(part_ms, 10) * 1e3:.1f}, p90 "
        f"{np.percentile(part_ms, 90) * 1e3:.1f}) | reduce {reduce_ms.mean() * 1e3:.1f} us")
    log(f"unique {by['unique_kv_bytes'] / 1e9:.3f} GB, logical {by['logical_kv_bytes'] / 1e9:.3f} GB -> "
        f"{achieved:.0f} GB/s unique ({achieved / HBM_PEAK_GBS:.1%}), {logical:.0f} GB/s logical")

    res = {
        "metric": "paged-attn decode tokens/sec and achieved HBM GB/s (% of peak), 1 GPU",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "layers": 1,
                   "batch": w.n_decode, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "out_dtype": str(b.out_dtype).replace("torch.", ""), "seed": args.seed,
                   "step": ("paged_attention_decode_append (cache write + decode partition pass + split-K "
                            "reduce)" if g else "reshape_and_cache, then paged_attention_decode (three calls)")},
        "roofline": {"bound": "hbm",
                     "kernel": "decode partition pass (decode_partition_kernel + decode_shared_kernel)",
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (profiled_traffic("decode_partition_llama3_8b_decode", ["decode.hip", "pkv_device.h"])
                                 if w.name == "llama3_8b_decode" and args.seed == 0 else None),
                     "algorithmic_bytes": by["algorithmic_bytes"]},
        "breakdown_us": {"append": float(append_ms.mean()) * 1e3, "partitions": float(part_ms.mean()) * 1e3,
                         "reduce": float(reduce_ms.mean()) * 1e3,
                         "host_allocator_step": host_allocator_us(b)},
        "bytes": by,
        "logical_gbs": logical,
        "step_modes": ({"one_call_ms": ms_step, "one_call_graph_replay_ms": g["us_per_step"] * 1e-3,
                        "three_calls_ms": eager_ms_step,
                        "three_calls_tokens_per_s": w.n_decode / (eager_ms_step * 1e-3)} if g else
                       {"three_calls_ms": eager_ms_step, "note": "--no-step-modes: value is the three-call step"}),
        "prefix_cache_host": prefix_cache_host(),
    }
    if not args.no_swap:
        res["swap"] = swap_leg(b)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    del b, out
    torch.cuda.empty_cache()
    if not args.no_fp8:
        res["fp8_kv_decode"] = fp8_decode_leg(w, K, W, None if args.out_dtype == "kv" else "f32", args.seed,
                                              not args.no_step_modes)
    if not args.no_verify:
        res["verify"] = verify_leg(max(5, K // 2), max(2, W // 2), args.seed)
    if not args.no_mixed:
        res["mixed_step"] = mixed_step(max(5, K // 2), max(2, W // 2), args.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
