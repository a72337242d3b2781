"""Prefix caching end to end on the GPU: request A is prefilled and finished;
request B, whose prompt starts with A's first 64 tokens, reuses A's cached
full blocks (only its other tokens are appended and written), and chunked
prefill over B's block table — reused blocks included — matches the fp64
oracle over B's logical keys and values.  A decode of B's next token reads
the same blocks."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"
HQ, HKV, D, DT = 32, 8, 128, "bf16"
TD = torch.bfloat16


def _rows(kind, owner, t0, t1, heads):
    bits = synth.values(7, kind, owner, t0, t1, heads, D, DT)
    return torch.from_numpy(bits.view(np.int16)).view(TD)


def _write(pkv, pool_k, pool_v, slots, owner, t0, t1, nblocks):
    k = _rows(synth.KIND_K, owner, t0, t1, HKV).to(DEV)
    v = _rows(synth.KIND_V, owner, t0, t1, HKV).to(DEV)
    pkv.reshape_and_cache(k, v, pool_k, pool_v, torch.from_numpy(np.asarray(slots, np.int64)).to(DEV),
                          nblocks, HKV, D)


def test_prefill_over_reused_prefix_blocks():
    import paged_kv_cache_gather_amd as pkv
    nblocks = 64
    pool = pkv.paged_kv_alloc(nblocks, HKV, D, DT, initial_free_order=np.random.default_rng(3).permutation(nblocks))
    pkv.paged_kv_prefix_cache_enable(pool)
    elems = nblocks * HKV * 16 * D
    pool_k = torch.zeros(elems, dtype=TD, device=DEV)
    pool_v = torch.zeros(elems, dtype=TD, device=DEV)
    rng = np.random.default_rng(11)
    tok_a = rng.integers(0, 30000, size=100).tolist()
    tok_b = tok_a[:64] + rng.integers(0, 30000, size=40).tolist()

    # request A: nothing cached yet; its K/V rows belong to the shared text (owner 1)
    a, n = pkv.paged_kv_seq_create_cached(pool, tok_a)
    assert n == 0
    slots, _ = pkv.paged_kv_seq_append_tokens(pool, a, tok_a)
    _write(pkv, pool_k, pool_v, slots, 1, 0, 100, nblocks)
    pkv.paged_kv_seq_free(pool, a)

    # request B reuses A's first four full blocks; its own tokens are owner 2
    b, n = pkv.paged_kv_seq_create_cached(pool, tok_b)
    assert n == 64
    slots, cow = pkv.paged_kv_seq_append_tokens(pool, b, tok_b[n:])
    assert cow == []
    _write(pkv, pool_k, pool_v, slots, 2, 64, 104, nblocks)
    torch.cuda.synchronize()

    L, ql = 104, 40
    table = pkv.paged_kv_seq_table(pool, b)
    tables = torch.from_numpy(table.reshape(1, -1).astype(np.int32)).to(DEV)
    q = _rows(synth.KIND_Q, 2, 64, 104, HQ).to(DEV)
    out = torch.empty((ql, HQ, D), dtype=torch.float32, device=DEV)
    scale = 1.0 / np.sqrt(D)
    pkv.paged_attention_prefill_chunk(out, q, pool_k, pool_v, tables,
                                      torch.tensor([0, ql], dtype=torch.int32, device=DEV),
                                      torch.tensor([L], dtype=torch.int32, device=DEV), ql, L, HKV, nblocks, scale)
    torch.cuda.synchronize()

    k_log = np.concatenate([synth.values(7, synth.KIND_K, 1, 0, 64, HKV, D, DT),
                            synth.values(7, synth.KIND_K, 2, 64, 104, HKV, D, DT)])
    v_log = np.concatenate([synth.values(7, synth.KIND_V, 1, 0, 64, HKV, D, DT),
                            synth.values(7, synth.KIND_V, 2, 64, 104, HKV, D, DT)])
    q_bits = synth.values(7, synth.KIND_Q, 2, 64, 104, HQ, D, DT)
    ref, _ = oracle.attention(oracle.decode(DT, q_bits), np.arange(64, 104), oracle.decode(DT, k_log),
                              oracle.decode(DT, v_log), scale)
    atol, rtol = tolerance(DT, "f32")
    assert_close("prefill over reused blocks", out.double().cpu().numpy(), ref, atol, rtol)

    # the next decode step of B over the same blocks
    slots, _ = pkv.paged_kv_seq_append_tokens(pool, b, [123])
    _write(pkv, pool_k, pool_v, slots, 2, 104, 105, nblocks)
    table = pkv.paged_kv_seq_table(pool, b)
    tables = torch.from_numpy(table.reshape(1, -1).astype(np.int32)).to(DEV)
    qd = _rows(synth.KIND_Q, 2, 104, 105, HQ).to(DEV)
    outd = torch.empty((1, HQ, D), dtype=torch.float32, device=DEV)
    pkv.paged_attention_decode(outd, qd, pool_k, pool_v, tables, torch.tensor([105], dtype=torch.int32, device=DEV),
                               105, HKV, nblocks, scale)
    torch.cuda.synchronize()
    k_log = np.concatenate([k_log, synth.values(7, synth.KIND_K, 2, 104, 105, HKV, D, DT)])
    v_log = np.concatenate([v_log, synth.values(7, synth.KIND_V, 2, 104, 105, HKV, D, DT)])
    refd, _ = oracle.attention(oracle.decode(DT, synth.values(7, synth.KIND_Q, 2, 104, 105, HQ, D, DT)), [104],
                               oracle.decode(DT, k_log), oracle.decode(DT, v_log), scale)
    assert_close("decode over reused blocks", outd.double().cpu().numpy(), refd, atol, rtol)
