"""GPU parity of verify attention (a few new query tokens per sequence, each
attending causally to the cached keys and the new ones before it: checking
drafted tokens, "Speculative decoding" in the vLLM Serving deep dive) against
the fp64 oracle: new tokens placed at and across the 512-token partition
edges, every GQA ratio (one and several 32-row token groups), both output
dtypes, sampled sequences of a Llama-3-8B-shaped batch of 256 sequences, the
agreement with chunked prefill on the same batch, and bad arguments."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, prefill_reference, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _run_verify(w, out_dtype=None, fill="host"):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(w, DEV, fill=fill, out_dtype=out_dtype)
    b.append_prefill()
    out = b.new_prefill_out()
    b.attend_verify(out)
    torch.cuda.synchronize()
    return b, out


def _check(w, out, out_dtype, chunks=None):
    atol, rtol = tolerance(w.dtype, out_dtype)
    got = out.double().cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    for c in (range(w.n_chunks) if chunks is None else chunks):
        ql = int(w.chunk_qlen[c])
        rows = np.arange(ql)
        assert_close(f"{w.name} seq {c} ctx={int(w.chunk_ctx[c])} q={ql}", got[cu[c]:cu[c + 1]],
                     prefill_reference(w, c, rows), atol, rtol)


CASES = [
    # name, Hq, Hkv, d, dtype, cached contexts, new tokens
    ("llama3_edges", 32, 8, 128, "bf16", [0, 1, 15, 16, 17, 300, 507, 508, 511, 512, 1020, 2043, 4000],
     [5, 5, 1, 2, 8, 5, 5, 5, 1, 5, 8, 5, 3]),
    ("mha_two_groups", 8, 8, 128, "f16", [100, 600, 200], [33, 40, 64]),
    ("gqa2_d64", 8, 4, 64, "f16", [0, 700, 1023], [16, 17, 2]),
    ("gqa8_d64", 32, 4, 64, "bf16", [513, 3, 1500], [4, 9, 5]),
    ("gqa16_d128", 32, 2, 128, "f16", [1000, 10, 509], [5, 2, 7]),
    # rows over 8 to 18 partitions (the merge takes partials in batches of 8)
    ("long_contexts", 32, 8, 128, "bf16", [4090, 8190, 9000], [8, 5, 3]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,ctx,ql", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("out_kind", ["f32", "kv"])
def test_verify_small(name, Hq, Hkv, d, dtype, ctx, ql, out_kind):
    out_dtype = "f32" if out_kind == "f32" else dtype
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 2048, seed=31, chunk_ctx=ctx, chunk_qlen=ql)
    print(f"verify {name} out={out_dtype}", flush=True)
    _, out = _run_verify(w, out_dtype)
    _check(w, out, out_dtype)


def _llama3_verify_batch(seed=0, k=5):
    lens = synth.make_workload("llama3_8b_decode", seed).decode_lens  # the decode batch's context lengths
    return synth.custom_workload("llama3_8b_verify", 32, 8, 128, "bf16", 70000, seed, chunk_ctx=lens - 1,
                                 chunk_qlen=np.full(lens.size, k))


def test_verify_full_size_sampled_and_equal_to_prefill():
    w = _llama3_verify_batch()
    print("verify full llama3_8b_verify", flush=True)
    b, out = _run_verify(w, "bf16", fill="device")
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(2)
    sample = sorted(set(rng.choice(w.n_chunks, 5, replace=False).tolist()
                        + [int(np.argmax(w.chunk_ctx)), int(np.argmin(w.chunk_ctx))]))
    _check(w, out, "bf16", sample)
    # the chunked-prefill kernel on the same batch agrees within the tolerance
    ref = b.new_prefill_out()
    b.attend_prefill(ref)
    torch.cuda.synchronize()
    atol, rtol = tolerance("bf16", "bf16")
    assert_close("verify vs prefill", out.double().cpu().numpy(), ref.double().cpu().numpy(), 2 * atol, 2 * rtol)


def test_verify_rejects_long_chunks_and_bad_workspace():
    import paged_kv_cache_gather_amd as pkv
    w = synth.custom_workload("verify_args", 8, 2, 64, "f16", 256, seed=3, chunk_ctx=[600], chunk_qlen=[70])
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(w, DEV, fill="host")
    p = b.prefill
    out = b.new_prefill_out()
    with pytest.raises(pkv.PagedKVError) as e:  # 70 > 64 new tokens: the prefill kernel's job
        pkv.paged_attention_verify(out, p.q, b.k_pool, b.v_pool, p.tables, p.cu_q_lens, p.lens_dev, 70,
                                   p.max_context_len, 2, w.num_blocks, w.scale)
    assert e.value.code == pkv.PKV_EUNSUPPORTED
    with pytest.raises(pkv.PagedKVError) as e:  # two partitions need a workspace
        pkv.paged_attention_verify(out, p.q, b.k_pool, b.v_pool, p.tables, p.cu_q_lens, p.lens_dev, 64,
                                   p.max_context_len, 2, w.num_blocks, w.scale)
    assert e.value.code == pkv.PKV_EINVAL


FP8_CASES = [
    ("llama3_fp8", 32, 8, 128, "bf16", [0, 17, 507, 508, 1020, 3000], [5, 8, 5, 5, 8, 3]),
    ("gqa16_fp8_f16", 32, 2, 64, "f16", [600, 5], [5, 2]),
    ("mha_fp8", 8, 8, 128, "f16", [300], [40]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,ctx,ql", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_verify_over_an_8bit_cache(name, Hq, Hkv, d, dtype, ctx, ql):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    from tests.helpers import FP8_K_SCALE, FP8_V_SCALE, prefill_reference_fp8
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 2048, seed=37, chunk_ctx=ctx, chunk_qlen=ql)
    print(f"verify fp8 {name}", flush=True)
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32", kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE,
                    v_scale=FP8_V_SCALE)
    b.append_prefill()
    out = b.new_prefill_out()
    b.attend_verify(out)
    torch.cuda.synchronize()
    atol, rtol = tolerance(dtype, "f32")
    got = out.double().cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    for c in range(w.n_chunks):
        assert_close(f"{name} seq {c}", got[cu[c]:cu[c + 1]], prefill_reference_fp8(w, c), atol, rtol)


def test_long_chunks_over_an_8bit_cache_in_pieces():
    # chunked prefill over an 8-bit cache: the chunk's rows are appended
    # once, then its queries go through paged_attention_verify_fp8 in pieces
    # of at most 64 tokens, each piece seeing the cache up to its last query
    import paged_kv_cache_gather_amd as pkv
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    from tests.helpers import FP8_K_SCALE, FP8_V_SCALE, prefill_reference_fp8
    w = synth.custom_workload("fp8_long_chunks", 32, 8, 128, "bf16", 2048, seed=39, chunk_ctx=[300, 0, 1500],
                              chunk_qlen=[200, 130, 64])
    print("fp8 chunks in pieces of 64", flush=True)
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32", kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE,
                    v_scale=FP8_V_SCALE)
    b.append_prefill()
    p = b.prefill
    out = b.new_prefill_out()
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    for c in range(w.n_chunks):
        ctx, ql = int(w.chunk_ctx[c]), int(w.chunk_qlen[c])
        for a in range(0, ql, 64):
            e = min(a + 64, ql)
            r0, r1 = int(cu[c]) + a, int(cu[c]) + e
            cu_piece = torch.tensor([0, e - a], dtype=torch.int32, device=DEV)
            lens = torch.tensor([ctx + e], dtype=torch.int32, device=DEV)
            need = pkv.paged_attention_verify_workspace_bytes(e - a, w.n_q_heads, w.head_dim, ctx + e)
            ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device=DEV) if need else None
            pkv.paged_attention_verify_fp8(out[r0:r1], p.q[r0:r1], b.k_pool, b.v_pool, p.tables[c:c + 1], cu_piece,
                                           lens, e - a, ctx + e, w.n_kv_heads, w.num_blocks, w.scale, b.k_scale,
                                           b.v_scale, workspace=ws)
    torch.cuda.synchronize()
    atol, rtol = tolerance("bf16", "f32")
    got = out.double().cpu().numpy()
    for c in range(w.n_chunks):
        assert_close(f"chunk {c}", got[cu[c]:cu[c + 1]], prefill_reference_fp8(w, c), atol, rtol)
