"""The whole-context decode path (short contexts, small batch: one launch,
one workgroup per (sequence, KV head), no split partitions and no merge)
against the fp64 oracle and against the split-context path on the same
batch (paged_attention_decode_partitions + _reduce always split): every GQA
ratio and head dim the path takes, all three K/V dtypes, contexts at and
around block and partition edges up to the 2048-token span, sequences
forked from a shared prefix, the one-call step bit for bit against its two
calls, and the step captured in a HIP graph."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, decode_references, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"
LENS = [1, 15, 16, 17, 100, 511, 512, 513, 1024, 1500, 2047, 2048]
LONG = [2049, 3071, 4095, 4096]  # past the vector routine's span, within the MFMA routine's


def _lens(n_kv_heads, long=True):
    """LENS (and LONG) repeated to 128 (sequence, KV head) pairs: contexts up
    to the span take the whole-context path from 128 pairs on."""
    base = LENS + LONG if long else LENS
    n = -(-128 // n_kv_heads)
    return [base[i % len(base)] for i in range(max(n, len(base)))]

CASES = [
    # name, Hq, Hkv, d, dtype
    ("tinyllama_gqa8_d64_f16", 32, 4, 64, "f16"),
    ("gqa8_d64_bf16", 16, 2, 64, "bf16"),
    ("gqa4_d128_bf16", 16, 4, 128, "bf16"),
    ("gqa2_d128_f16", 8, 4, 128, "f16"),
    ("mha_d128_bf16", 4, 4, 128, "bf16"),
    ("gqa8_d128_bf16", 32, 4, 128, "bf16"),
    ("gqa16_d128_f16", 32, 2, 128, "f16"),
    ("gqa4_d64_f32", 8, 2, 64, "f32"),
    ("gqa2_d128_f32", 4, 2, 128, "f32"),
]


def _whole(w, max_len):
    import paged_kv_cache_gather_amd as pkv
    return pkv.paged_attention_decode_whole_context(w.n_decode, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype,
                                                    max_len)


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("out_kind", ["f32", "kv"])
def test_whole_context_matches_oracle_and_split_path(name, Hq, Hkv, d, dtype, out_kind):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 8192, seed=71, decode_lens=_lens(Hkv, dtype != "f32"))
    out_dtype = "f32" if out_kind == "f32" else dtype
    b = DeviceBatch(w, DEV, fill="host", out_dtype=out_dtype)
    assert _whole(w, b.decode.max_context_len)
    print(f"whole context {name} out {out_dtype}", flush=True)
    b.append_decode()
    whole, split = b.new_decode_out(), b.new_decode_out()
    b.attend_decode(whole)
    b.attend_decode_split(split)
    torch.cuda.synchronize()
    atol, rtol = tolerance(dtype, out_dtype)
    refs = decode_references(w, range(w.n_decode))
    gw, gs = whole.double().cpu().numpy(), split.double().cpu().numpy()
    for s in range(w.n_decode):
        L = int(w.decode_lens[s])
        assert_close(f"whole L={L}", gw[s], refs[s], atol, rtol)
        assert_close(f"split L={L}", gs[s], refs[s], atol, rtol)
    # one partition on both paths: the same kernel code over the same tokens,
    # but dealt to 16 waves instead of 4, so only the tolerance holds
    assert_close("whole vs split", gw, gs, atol, rtol)


def test_whole_context_with_shared_prefixes_and_forks():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    # groups forked from shared prefixes (the split path would read them once
    # per run; this path reads them per sequence)
    lens = [1500, 1500, 1536, 1200, 700, 700, 520, 33]
    w = synth.custom_workload("whole_shared", 32, 8, 128, "bf16", 2048, seed=72, decode_lens=lens,
                              prefix_len=[1100, 1100, 1100, 1100, 600, 600, 0, 0],
                              prefix_group=[0, 0, 0, 0, 1, 1, -1, -1])
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    assert _whole(w, b.decode.max_context_len)
    print("whole context with shared prefixes", flush=True)
    b.append_decode()
    out = b.new_decode_out()
    b.attend_decode(out)
    torch.cuda.synchronize()
    atol, rtol = tolerance("bf16", "f32")
    refs = decode_references(w, range(w.n_decode))
    got = out.double().cpu().numpy()
    for s in range(w.n_decode):
        assert_close(f"seq {s}", got[s], refs[s], atol, rtol)


def test_whole_context_one_call_step_equals_two_calls():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload("whole_append", 32, 4, 64, "f16", 4096, seed=73, decode_lens=_lens(4))
    sep = DeviceBatch(w, DEV, fill="host", out_dtype="f16")
    one = DeviceBatch(w, DEV, fill="host", out_dtype="f16")
    assert _whole(w, sep.decode.max_context_len)
    print("whole context one-call step", flush=True)
    sep.decode.slots[3] = -1  # a padding row: not written by either form
    one.decode.slots[3] = -1
    out_sep, out_one = sep.new_decode_out(), one.new_decode_out()
    sep.append_decode()
    sep.attend_decode(out_sep)
    one.step_decode(out_one)
    torch.cuda.synchronize()
    assert torch.equal(out_sep.view(torch.int16), out_one.view(torch.int16))
    assert torch.equal(sep.k_pool.view(torch.uint8), one.k_pool.view(torch.uint8))
    assert torch.equal(sep.v_pool.view(torch.uint8), one.v_pool.view(torch.uint8))


def test_whole_context_step_replays_from_a_graph():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    from tests.test_gpu_graph import _replays_match
    w = synth.custom_workload("whole_graph", 32, 4, 64, "f16", 4096, seed=74, decode_lens=_lens(4))
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    assert _whole(w, b.decode.max_context_len)
    print("whole context graph", flush=True)
    out = b.new_decode_out()
    _replays_match(lambda: b.step_decode(out), [out])


def test_whole_context_limits():
    import paged_kv_cache_gather_amd as pkv
    f = pkv.paged_attention_decode_whole_context
    assert f(64, 32, 4, 64, "f16", 2048)        # TinyLlama-shaped batch: 256 pairs
    assert f(64, 32, 4, 64, "f16", 4096)        # the MFMA routine's span
    assert not f(64, 32, 4, 64, "f16", 4097)    # a context past the span
    assert not f(64, 8, 4, 64, "f32", 2049)     # past the vector routine's span (fp32 pools)
    assert f(32, 32, 4, 64, "f16", 2048)        # 128 pairs
    assert not f(31, 32, 4, 64, "f16", 2048)    # 124 pairs, contexts past 1536
    assert f(31, 32, 4, 64, "f16", 1536)        # 124 pairs, contexts up to 1536
    # a second round of workgroups: 384 to 512 pairs at any length (16-bit and 8-bit pools)
    assert f(128, 32, 4, 64, "f16", 1535)       # 512 pairs
    assert f(48, 32, 8, 128, "bf16", 2048)      # 384 pairs
    assert not f(48, 32, 8, 128, "bf16", 2049)  # a second round only up to 2048 tokens
    assert not f(47, 32, 8, 128, "bf16", 2048)  # 376 pairs
    assert not f(40, 32, 8, 128, "bf16", 1024)  # 320 pairs
    assert f(56, 32, 8, 128, "bf16", 512)       # 448 pairs
    assert not f(129, 32, 4, 64, "f16", 2048)   # 516 pairs
    # fp32 pools (the vector routine): 448 to 512 pairs, 384 KiB or more per pair
    assert f(256, 4, 2, 128, "f32", 384)        # 512 pairs, 384 KiB
    assert not f(256, 4, 2, 128, "f32", 383)
    assert not f(192, 4, 2, 128, "f32", 2048)   # 384 pairs
    assert f(64, 16, 4, 128, "bf16", 1000)      # G 4 at head_dim 128
    assert f(64, 32, 4, 128, "bf16", 1000)      # G 8 at head_dim 128 (16-bit: MFMA)
    assert f(64, 64, 4, 128, "f16", 1000)       # G 16
    assert f(64, 16, 4, 64, "f32", 1000)        # fp32 pools: G x d x 4 <= 1024
    assert not f(64, 32, 4, 64, "f32", 1000)    # fp32, G 8 at head_dim 64: registers
    assert f(8, 32, 8, 128, "fp8_e4m3", 1000)  # 8-bit pools: the same rule
    assert not f(8, 32, 8, 128, "fp8_e4m3", 2000)  # 64 pairs, contexts past 1536
    assert f(64, 32, 8, 128, "fp8_e4m3", 100)   # 512 pairs
    assert not f(40, 32, 8, 128, "fp8_e4m3", 1000)  # 320 pairs
    assert not f(0, 32, 4, 64, "f16", 100)
    assert not f(8, 30, 4, 64, "f16", 100)      # n_q_heads not a multiple
    # the split path just past the span still matches the oracle
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload("whole_edge", 32, 4, 64, "f16", 8192, seed=75, decode_lens=[4097, 7, 4096] * 11)
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    assert not _whole(w, b.decode.max_context_len)
    b.append_decode()
    out = b.new_decode_out()
    b.attend_decode(out)
    torch.cuda.synchronize()
    atol, rtol = tolerance("f16", "f32")
    refs = decode_references(w, range(w.n_decode))
    got = out.double().cpu().numpy()
    for s in range(w.n_decode):
        assert_close(f"seq {s}", got[s], refs[s], atol, rtol)
