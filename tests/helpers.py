"""Shared pieces of the GPU parity tests: oracle references for a workload's
sequences, and the tolerance rule.

Tolerance (per element, |got - ref| <= atol + rtol * |ref|):
  * fp32 K/V: rtol 1e-5, atol 1e-6;
  * fp16 / bf16 K/V with fp32 accumulation: rtol = atol = 2e-3.
When the output itself is stored in fp16 / bf16, its final rounding adds up
to u * |ref| (u = 2^-11 for fp16, 2^-8 for bf16, round to nearest), so that
term is added to rtol: the fp32 result must be within the bound above and
the stored value within one more rounding of it.
"""
import numpy as np

import oracle

U_OUT = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def tolerance(kv_dtype: str, out_dtype: str):
    if kv_dtype == "f32":
        atol, rtol = 1e-6, 1e-5
    else:
        atol, rtol = 2e-3, 2e-3
    return atol, rtol + U_OUT[out_dtype]


def assert_close(name, got, ref, atol, rtol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - ref)
    lim = atol + rtol * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {i}: "
                             f"got {got[i]:.6g} ref {ref[i]:.6g} (max abs err {err.max():.3e})")


def decode_reference(w, s):
    """Oracle output [Hq, d] for decode sequence s of workload w."""
    L = int(w.decode_lens[s])
    k, v = w.kv("decode", s, 0, L)
    q = w.q("decode", s, L - 1, L)
    out, ws = oracle.attention(oracle.decode(w.dtype, q), [L - 1], oracle.decode(w.dtype, k),
                               oracle.decode(w.dtype, v), w.scale)
    assert np.all(np.abs(ws - 1) < 1e-9)
    return out[0]


def prefill_reference(w, c, rows=None, n_threads=8):
    """Oracle output [len(rows), Hq, d] for prefill chunk c of workload w
    (rows: chunk-local query indices, default all)."""
    ctx, ql = int(w.chunk_ctx[c]), int(w.chunk_qlen[c])
    rows = np.arange(ql) if rows is None else np.asarray(rows)
    last = int(rows.max()) + 1
    k, v = w.kv("chunk", c, 0, ctx + last)
    qb = w.q("chunk", c, ctx, ctx + ql)[rows]
    out, _ = oracle.attention(oracle.decode(w.dtype, qb), ctx + rows, oracle.decode(w.dtype, k),
                              oracle.decode(w.dtype, v), w.scale, n_threads=n_threads)
    return out


# scales of the 8-bit cache in the tests: the synthetic values are standard
# normal quantiles (|x| < 4.4), so these map them to at most ~350 / ~430,
# inside E4M3's 448 (not powers of two, so the reciprocal rounds)
FP8_K_SCALE, FP8_V_SCALE = 0.0125, 0.0103


_QTABLES = {}


def _quantise(dtype, bits, scale):
    """The oracle's E4M3 quantiser applied to raw 16-bit (or fp32) rows.  A
    16-bit element has at most 65536 bit patterns, so the quantiser runs once
    on every pattern and the rows are looked up in that table (the same
    function values; the oracle's exhaustive search is slow per element)."""
    if dtype == "f32":
        return oracle.quantize_e4m3(oracle.decode(dtype, bits).astype(np.float32), scale)
    key = (dtype, float(scale))
    if key not in _QTABLES:
        pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        _QTABLES[key] = oracle.quantize_e4m3(oracle.decode(dtype, pats).astype(np.float32), scale)
    return _QTABLES[key][np.ascontiguousarray(bits).view(np.uint16)]


def quantised_kv(w, kind, idx, t0, t1, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE):
    """Dequantised fp64 K/V of positions [t0, t1): the workload's rows put
    through the oracle's E4M3 quantiser and read back with the scales."""
    k, v = w.kv(kind, idx, t0, t1)
    kq = _quantise(w.dtype, k, k_scale)
    vq = _quantise(w.dtype, v, v_scale)
    return oracle.dequantize_e4m3(kq, k_scale), oracle.dequantize_e4m3(vq, v_scale)


def decode_reference_fp8(w, s, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE):
    """Oracle output [Hq, d] for decode sequence s over an 8-bit cache."""
    L = int(w.decode_lens[s])
    k, v = quantised_kv(w, "decode", s, 0, L, k_scale, v_scale)
    q = w.q("decode", s, L - 1, L)
    out, ws = oracle.attention(oracle.decode(w.dtype, q), [L - 1], k, v, w.scale)
    assert np.all(np.abs(ws - 1) < 1e-9)
    return out[0]


def prefill_reference_fp8(w, c, rows=None, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE, n_threads=8):
    """Oracle output [len(rows), Hq, d] for chunk c over an 8-bit cache."""
    ctx, ql = int(w.chunk_ctx[c]), int(w.chunk_qlen[c])
    rows = np.arange(ql) if rows is None else np.asarray(rows)
    last = int(rows.max()) + 1
    k, v = quantised_kv(w, "chunk", c, 0, ctx + last, k_scale, v_scale)
    qb = w.q("chunk", c, ctx, ctx + ql)[rows]
    out, _ = oracle.attention(oracle.decode(w.dtype, qb), ctx + rows, k, v, w.scale, n_threads=n_threads)
    return out


def oracle_workers() -> int:
    """Host threads for the oracle in the GPU tests: the machine's CPU share is
    16 threads, whatever os.cpu_count() reports."""
    import os
    return max(1, min(os.cpu_count() or 1, 16))


def decode_references(w, seqs, fp8=False):
    """Oracle outputs {s: [Hq, d]} for many decode sequences of w: each
    sequence's K/V are regenerated on the host and its oracle run in a worker
    thread (the oracle's C loops and numpy's large-array work release the
    interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    ref = decode_reference_fp8 if fp8 else decode_reference
    seqs = list(seqs)
    if fp8 and w.dtype != "f32":  # fill the quantiser's tables before the threads start
        _quantise(w.dtype, np.zeros(1, np.uint16), FP8_K_SCALE)
        _quantise(w.dtype, np.zeros(1, np.uint16), FP8_V_SCALE)
    with ThreadPoolExecutor(oracle_workers()) as ex:
        return dict(zip(seqs, ex.map(lambda s: ref(w, s), seqs)))


def prefill_references(w, chunks, fp8=False):
    """Oracle outputs {c: [q_len, Hq, d]} for every row of the given chunks
    (the oracle's own threads split each chunk's rows and heads)."""
    ref = prefill_reference_fp8 if fp8 else prefill_reference
    return {c: ref(w, c, n_threads=oracle_workers()) for c in chunks}
