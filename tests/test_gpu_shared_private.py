"""Paging changes where K/V live, not what attention computes ("Sharing and
copy-on-write", vLLM Serving deep dive; the PagedAttention section of The
hands-on guide to LLM Inference with vLLM): a batch whose sequences share
ref-counted prefix blocks and the same batch with every block a private copy
of the same bytes give the same attention, up to rounding.  On the GPU the
two layouts take different kernels — partitions that sequences of one run
window share are scored once for all of them on the matrix cores, private ones on the vector
units — so they agree within the tolerance, not bit for bit; both are
checked against the oracle, including shared runs that cross the run window.

Also here: bf16 values of any finite size.  The MFMA paths take bf16 V
unconverted (the probabilities as a bf16 pair), so V entries far beyond
fp16's range — up to about 4e6 — are exact operands in decode shared runs
and verify attention; scaling one dim of every V row by 2^e scales that
output dim by exactly 2^e.  Chunked prefill converts V to fp16 and clamps
entries beyond +-65504 (its documented limit), checked against the oracle
over the clamped values."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, decode_references, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _shared_batch(name, seed):
    # window of 8 sequences at G = 4: group 0 fills it (3 shared partitions),
    # group 1 straddles windows 1 and 2 with a prefix ending inside a block,
    # group 2 shares exactly one partition; singles between them
    lens = [1600, 1700, 2000, 2100, 2500, 3000, 1537, 1536,
            1100, 1200, 1300, 1030, 700, 2049, 1500, 1110, 1031, 1040,
            520, 600, 513, 1000]
    # (a member's prefix is at most L - 1 tokens: the step appends the L-th;
    # sequence 7's prefix ends one token short of its third partition)
    plen = [1536] * 7 + [1535] + [0, 0, 1029, 1029, 699, 1029, 1029, 1029, 1029, 1029] + [512, 512, 512, 0]
    grp = [0] * 8 + [-1, -1, 1, 1, 1, 1, 1, 1, 1, 1] + [2, 2, 2, -1]
    return synth.custom_workload(name, 32, 8, 128, "bf16", 4096, seed=seed, decode_lens=lens, prefix_len=plen,
                                 prefix_group=grp)


def _attend(b, tables, out):
    import paged_kv_cache_gather_amd as pkv
    d, w = b.decode, b.w
    pkv.paged_attention_decode(out, d.q, b.k_pool, b.v_pool, tables, d.lens_dev, d.max_context_len, w.n_kv_heads,
                               w.num_blocks, w.scale, workspace=d.workspace)


def _private_tables(b):
    """Copy every block of every sequence to a block no table names, on the
    device (paged_kv_copy_blocks), and return the tables of the copies."""
    import paged_kv_cache_gather_amd as pkv
    w = b.w
    tab = b.decode.tables_host
    used = set(tab[tab >= 0].tolist())
    free = iter(x for x in range(w.num_blocks) if x not in used)
    new = tab.copy()
    pairs = []
    for s in range(tab.shape[0]):
        for j in range(-(-int(b.decode.lens[s]) // 16)):
            nb = next(free)
            pairs.append((int(tab[s, j]), nb))
            new[s, j] = nb
    pkv.paged_kv_copy_blocks(b.k_pool, b.v_pool, torch.tensor(pairs, dtype=torch.int32, device=DEV), w.num_blocks,
                             w.n_kv_heads, w.head_dim)
    assert len(set(new[new >= 0].tolist())) == int((new >= 0).sum())  # every block private
    return torch.from_numpy(new).to(DEV)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_shared_blocks_equal_private_copies(out_dtype):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = _shared_batch("shared_vs_private", 41)
    print(f"shared vs private, out {out_dtype}", flush=True)
    b = DeviceBatch(w, DEV, fill="host", out_dtype=out_dtype)
    b.append_decode()
    out_shared, out_private = b.new_decode_out(), b.new_decode_out()
    _attend(b, b.decode.tables, out_shared)
    _attend(b, _private_tables(b), out_private)
    torch.cuda.synchronize()
    atol, rtol = tolerance("bf16", out_dtype)
    refs = decode_references(w, range(w.n_decode))
    gs, gp = out_shared.double().cpu().numpy(), out_private.double().cpu().numpy()
    for s in range(w.n_decode):
        assert_close(f"shared layout seq {s}", gs[s], refs[s], atol, rtol)
        assert_close(f"private layout seq {s}", gp[s], refs[s], atol, rtol)
        assert_close(f"shared vs private seq {s}", gs[s], gp[s], atol, rtol)
    # sequences with no shared partition take the same kernel either way: bitwise
    for s in (8, 9, 21):
        assert np.array_equal(gs[s], gp[s]), s


def _dim_scales(d, top=20):
    e = (np.arange(d) * 7) % (top + 1)  # 2^0 .. 2^top, every value used
    return e, np.ldexp(1.0, e)


def _scale_v_pool(b, sc):
    w = b.w
    f = torch.tensor(sc, dtype=torch.float32, device=DEV).to(b.v_pool.dtype)
    b.v_pool.view(w.num_blocks, w.n_kv_heads, w.head_dim, 16).mul_(f.view(1, 1, -1, 1))


def test_bf16_values_beyond_fp16_range_in_shared_decode():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = _shared_batch("large_v", 43)
    e, sc = _dim_scales(w.head_dim)
    print(f"decode with V up to {4.4 * sc.max():.3g}", flush=True)
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    b.append_decode()
    base = b.new_decode_out()
    b.attend_decode(base)
    _scale_v_pool(b, sc)
    big = b.new_decode_out()
    b.attend_decode(big)
    torch.cuda.synchronize()
    scale_t = torch.tensor(sc, dtype=torch.float32, device=DEV)
    # power-of-two scaling of a V dim scales that output dim exactly
    assert torch.equal(big, base * scale_t), "scaled V does not scale the output exactly"
    got = big.double().cpu().numpy()
    atol, rtol = tolerance("bf16", "f32")
    for s in range(w.n_decode):
        L = int(w.decode_lens[s])
        k, v = w.kv("decode", s, 0, L)
        q = w.q("decode", s, L - 1, L)
        vbig = oracle.decode("bf16", v) * sc  # exact in fp64: |v| up to ~4.5e6
        assert np.abs(vbig).max() > 65504 or L < 2
        ref, _ = oracle.attention(oracle.decode("bf16", q), [L - 1], oracle.decode("bf16", k), vbig, w.scale)
        # the tolerance scales with the dim's scale: compare in the unscaled units
        assert_close(f"large-V seq {s}", got[s] / sc, ref[0] / sc, atol, rtol)


def test_bf16_values_beyond_fp16_range_in_verify_and_prefill():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload("large_v_verify", 32, 8, 128, "bf16", 1024, seed=47, chunk_ctx=[0, 40, 600, 1400],
                              chunk_qlen=[5, 8, 5, 3])
    e, sc = _dim_scales(w.head_dim)
    print("verify and prefill with V up to 4.5e6", flush=True)
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    b.append_prefill()
    base = b.new_prefill_out()
    b.attend_verify(base)
    _scale_v_pool(b, sc)
    big, pre = b.new_prefill_out(), b.new_prefill_out()
    b.attend_verify(big)
    b.attend_prefill(pre)
    torch.cuda.synchronize()
    scale_t = torch.tensor(sc, dtype=torch.float32, device=DEV)
    assert torch.equal(big, base * scale_t), "verify: scaled V does not scale the output exactly"
    got, gotp = big.double().cpu().numpy(), pre.double().cpu().numpy()
    atol, rtol = tolerance("bf16", "f32")
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    for c in range(w.n_chunks):
        ctx, ql = int(w.chunk_ctx[c]), int(w.chunk_qlen[c])
        k, v = w.kv("chunk", c, 0, ctx + ql)
        q = oracle.decode("bf16", w.q("chunk", c, ctx, ctx + ql))
        kk, vbig = oracle.decode("bf16", k), oracle.decode("bf16", v) * sc
        ref, _ = oracle.attention(q, ctx + np.arange(ql), kk, vbig, w.scale)
        assert_close(f"verify large-V seq {c}", got[cu[c]:cu[c + 1]] / sc, ref / sc, atol, rtol)
        # chunked prefill: V entries beyond fp16's range are clamped to +-65504
        refc, _ = oracle.attention(q, ctx + np.arange(ql), kk, np.clip(vbig, -65504.0, 65504.0), w.scale)
        assert_close(f"prefill clamped-V chunk {c}", gotp[cu[c]:cu[c + 1]] / sc, refc / sc, atol, rtol)
