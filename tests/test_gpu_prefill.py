"""GPU parity of chunked-prefill attention (MFMA) against the fp64 oracle:
ragged chunks over existing contexts (including empty ones and partial
blocks), every GQA ratio the kernel builds, both output dtypes, sampled rows
of the full-size mixed step, and the invariants that chunking does not change
the rows and that a decode step equals the last prefill row."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, decode_reference, prefill_reference, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _run_prefill(w, out_dtype=None, fill="host"):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(w, DEV, fill=fill, out_dtype=out_dtype)
    b.append_prefill()
    out = b.new_prefill_out()
    b.attend_prefill(out)
    torch.cuda.synchronize()
    return b, out


def _check_chunks(w, out, out_dtype, rows_per_chunk=None, seed=0):
    atol, rtol = tolerance(w.dtype, out_dtype)
    got = out.double().cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    rng = np.random.default_rng(seed)
    for c in range(w.n_chunks):
        ql = int(w.chunk_qlen[c])
        if rows_per_chunk is None or rows_per_chunk >= ql:
            rows = np.arange(ql)
        else:
            rows = np.unique(np.concatenate([[0, ql - 1], rng.choice(ql, rows_per_chunk, replace=False)]))
        ref = prefill_reference(w, c, rows)
        assert_close(f"{w.name} chunk {c} ctx={int(w.chunk_ctx[c])} q={ql}", got[cu[c] + rows], ref, atol, rtol)


CASES = [
    # name, Hq, Hkv, d, dtype, contexts, q_lens
    ("llama3_edges", 32, 8, 128, "bf16", [0, 1, 15, 16, 17, 100, 1000, 0], [1, 5, 16, 17, 64, 100, 130, 200]),
    ("opt13b_mha", 40, 40, 128, "f16", [0, 300], [70, 33]),
    ("gqa2_d64", 8, 4, 64, "f16", [0, 31, 200], [130, 7, 64]),
    ("tinyllama_gqa8", 32, 4, 64, "bf16", [0, 513], [65, 40]),
    ("gqa16", 32, 2, 128, "f16", [10, 0], [50, 16]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,ctx,ql", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("out_kind", ["f32", "kv"])
def test_prefill_small(name, Hq, Hkv, d, dtype, ctx, ql, out_kind):
    out_dtype = "f32" if out_kind == "f32" else dtype
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 1024, seed=7, chunk_ctx=ctx, chunk_qlen=ql)
    print(f"prefill {name} out={out_dtype}", flush=True)
    _, out = _run_prefill(w, out_dtype)
    _check_chunks(w, out, out_dtype)


def test_config5_prefill_sampled_rows():
    w = synth.make_workload("llama3_8b_mixed", seed=0)
    print("prefill full llama3_8b_mixed", flush=True)
    b, out = _run_prefill(w, None, fill="device")
    assert torch.isfinite(out.float()).all()
    sub = synth.make_workload("llama3_8b_mixed", seed=0)
    keep = [int(np.argmin(w.chunk_ctx)), int(np.argmax(w.chunk_ctx)), 3, 9]
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    atol, rtol = tolerance(w.dtype, w.dtype)
    got = out.double().cpu().numpy()
    rng = np.random.default_rng(5)
    for c in keep:
        rows = np.unique(np.concatenate([[0, 511], rng.choice(512, 24, replace=False)]))
        assert_close(f"mixed-step chunk {c} ctx={int(w.chunk_ctx[c])}", got[cu[c] + rows], prefill_reference(sub, c, rows),
                     atol, rtol)


def test_chunking_does_not_change_rows():
    # one 300-token prompt prefilled whole vs in chunks of 100 + 120 + 80
    full = synth.custom_workload("whole", 32, 8, 128, "bf16", 256, seed=9, chunk_ctx=[0], chunk_qlen=[300])
    _, out_full = _run_prefill(full, "f32")
    parts = []
    for ctx, ql in [(0, 100), (100, 120), (220, 80)]:
        w = synth.custom_workload("whole", 32, 8, 128, "bf16", 256, seed=9, chunk_ctx=[ctx], chunk_qlen=[ql])
        _, o = _run_prefill(w, "f32")
        parts.append(o.cpu().numpy())
    got = np.concatenate(parts)
    np.testing.assert_allclose(got, out_full.cpu().numpy(), rtol=2e-3, atol=2e-3)


def test_decode_equals_last_prefill_row():
    # the decode step's output is the last row of the causal prefill over the same keys
    L = 777
    wp = synth.custom_workload("dp", 32, 8, 128, "bf16", 256, seed=11, chunk_ctx=[L - 1], chunk_qlen=[1])
    _, op = _run_prefill(wp, "f32")
    ref = prefill_reference(wp, 0)[0]
    atol, rtol = tolerance("bf16", "f32")
    assert_close("prefill last row", op.cpu().numpy()[0], ref, atol, rtol)
    wd = synth.custom_workload("dp", 32, 8, 128, "bf16", 256, seed=11, decode_lens=[L])
    # same owner numbering: decode sequence 0 is owner n_chunks + 0 = 0 here
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(wd, DEV, fill="host", out_dtype="f32")
    b.append_decode()
    od = b.new_decode_out()
    b.attend_decode(od)
    torch.cuda.synchronize()
    np.testing.assert_allclose(od.cpu().numpy()[0], op.cpu().numpy()[0], rtol=2e-3, atol=2e-3)
    assert_close("decode vs oracle", od.cpu().numpy()[0], decode_reference(wd, 0), atol, rtol)


def test_dispatch_order_ties_and_ranked_chunks():
    # chunks are dispatched in decreasing context length; equal lengths (ties,
    # ranked by index) with different context/query splits, and one shorter
    ctx = [100, 50, 0, 140, 100, 120, 0, 30, 150, 149]
    ql = [60, 110, 160, 20, 60, 40, 1, 130, 10, 11]
    w = synth.custom_workload("ties", 16, 4, 128, "bf16", 512, seed=13, chunk_ctx=ctx, chunk_qlen=ql)
    print("prefill ties", flush=True)
    _, out = _run_prefill(w, "f32")
    _check_chunks(w, out, "f32")


def test_more_chunks_than_the_ranking_covers():
    # beyond 512 chunks the workgroups keep index order
    rng = np.random.default_rng(17)
    n = 600
    ctx = rng.integers(0, 120, size=n).tolist()
    ql = rng.integers(1, 5, size=n).tolist()
    nb = sum(-(-(c + q) // 16) + 1 for c, q in zip(ctx, ql)) + 16
    w = synth.custom_workload("many_chunks", 8, 2, 64, "f16", nb, seed=17, chunk_ctx=ctx, chunk_qlen=ql)
    print(f"prefill {n} chunks", flush=True)
    _, out = _run_prefill(w, "f32")
    _check_chunks(w, out, "f32")
