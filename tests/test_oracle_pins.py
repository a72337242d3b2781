"""Pins of the fp64 oracle to facts fixed outside it: figures printed on the
pages (tests/golden/*.json, each with its citation), closed forms, a textbook
matrix form of softmax attention, invariants the pages state, and brute force
on tiny inputs.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
from oracle import block_manager as bm

GIB = 1 << 30


@pytest.fixture(scope="module")
def sizing(golden_dir):
    with open(os.path.join(golden_dir, "kv_sizing.json")) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def tables(golden_dir):
    with open(os.path.join(golden_dir, "block_tables.json")) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# sizing
# --------------------------------------------------------------------------
def test_kv_bytes_per_token_printed(sizing):
    for e in sizing["per_token"]:
        got = oracle.kv_bytes_per_token(e["n_layers"], e["n_kv_heads"], e["d_head"], e["dtype_bytes"])
        assert got == e["bytes_per_token"], e["cite"]


def test_kv_bytes_per_sequence_printed(sizing):
    for e in sizing["per_sequence"]:
        b = oracle.kv_bytes_per_token(e["n_layers"], e["n_kv_heads"], e["d_head"], e["dtype_bytes"]) * e["tokens"]
        if "exact_gib" in e:
            assert b == e["exact_gib"] * GIB, e["cite"]
            if "times_64_gib" in e:
                assert 64 * b == e["times_64_gib"] * GIB
        else:
            assert e["lo"] <= b <= e["hi"], e["cite"]


def test_pool_sizing_worked_example(sizing):
    p = sizing["pool"]
    bb = oracle.kv_bytes_per_block(p["n_layers"], p["n_kv_heads"], p["d_head"], p["dtype_bytes"], p["block_size"])
    assert bb == p["block_bytes"]
    nb = oracle.blocks_for_budget(p["kv_budget_gib"] * GIB, p["n_layers"], p["n_kv_heads"], p["d_head"],
                                  p["dtype_bytes"], p["block_size"])
    assert nb == p["gpu_blocks"]
    assert nb * p["block_size"] == p["kv_tokens"]
    assert round(nb * p["block_size"] / p["max_len"], 1) == p["concurrency"]


# --------------------------------------------------------------------------
# value decoders against library conversions, over every 16-bit pattern
# --------------------------------------------------------------------------
def _cmp_nan(a, b):
    both_nan = np.isnan(a) & np.isnan(b)
    return np.all(both_nan | (a == b))


def test_f16_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    assert _cmp_nan(oracle.decode("f16", bits), ref)


def test_bf16_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert _cmp_nan(oracle.decode("bf16", bits), ref)


def test_f32_decoder_sample():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1e-45, 3.4e38, np.inf, -np.inf], np.float32)])
    assert np.array_equal(oracle.decode("f32", x.view(np.uint32)), x.astype(np.float64))


# --------------------------------------------------------------------------
# block table / slot mapping
# --------------------------------------------------------------------------
def test_slot_diagram_in_words(tables):
    ex = tables["diagram_in_words"]
    bs, table = ex["block_size"], ex["table"]
    for lb, (a, b) in enumerate(ex["logical_blocks"]):
        for t in range(a, b + 1):
            s = oracle.slot(table, t, bs)
            assert s // bs == table[lb] and s % bs == t % bs
    assert [oracle.slot(table, t, bs) for t in (0, 17, 32)] == [112, 49, 176]


def test_slot_notepad_pages(tables):
    table = tables["notepad_pages"]["table"]
    assert oracle.slot(table, 0, 16) // 16 == 7
    assert oracle.slot(table, 16, 16) // 16 == 2


# --------------------------------------------------------------------------
# attention against the textbook matrix form (brute force, tiny inputs)
# --------------------------------------------------------------------------
def _matrix_form(q, pos, k, v, scale):
    """softmax(Q K^T * scale + causal mask) V, per head, with each query head
    reading KV head h // (Hq / Hkv)."""
    R, Hq, d = q.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=1)  # [N, Hq, d]
    vv = np.repeat(v, G, axis=1)
    out = np.empty_like(q)
    mask = np.where(np.arange(N)[None, :] <= np.asarray(pos)[:, None], 0.0, -np.inf)
    for h in range(Hq):
        S = q[:, h, :] @ kk[:, h, :].T * scale + mask
        out[:, h, :] = softmax(S, axis=1) @ vv[:, h, :]
    return out


@pytest.mark.parametrize("Hq,Hkv,d,N", [(4, 2, 8, 7), (2, 2, 16, 19), (8, 1, 4, 33), (3, 3, 5, 1)])
def test_attention_matches_matrix_form(Hq, Hkv, d, N):
    rng = np.random.default_rng(Hq * 100 + N)
    q = rng.standard_normal((N, Hq, d))
    k = rng.standard_normal((N, Hkv, d))
    v = rng.standard_normal((N, Hkv, d))
    pos = np.arange(N)
    scale = 1 / math.sqrt(d)
    out, ws = oracle.attention(q, pos, k, v, scale)
    ref = _matrix_form(q, pos, k, v, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    assert np.all(np.abs(ws - 1.0) <= 4 * N * np.finfo(np.float64).eps)


def test_attention_closed_form_two_keys():
    # d = 1, one head: s_j = q * k_j / sqrt(1); out = sum_j e^{s_j} v_j / sum_j e^{s_j}
    q = np.array([[[0.5]]])
    k = np.array([[[2.0]], [[-1.0]]])
    v = np.array([[[3.0]], [[7.0]]])
    out, _ = oracle.attention(q, [1], k, v, 1.0)
    e0, e1 = math.exp(1.0), math.exp(-0.5)
    assert out[0, 0, 0] == pytest.approx((e0 * 3 + e1 * 7) / (e0 + e1), rel=1e-15)
    # the causal rule: at position 0 only the first key is visible
    out0, _ = oracle.attention(q, [0], k, v, 1.0)
    assert out0[0, 0, 0] == 3.0


def test_single_key_returns_that_value_exactly():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((1, 2, 16))
    out, _ = oracle.attention(rng.standard_normal((1, 4, 16)), [0], rng.standard_normal((1, 2, 16)), v, 0.25)
    assert np.array_equal(out[0], np.repeat(v[0], 2, axis=0))


def test_equal_scores_average_the_values():
    rng = np.random.default_rng(4)
    N, d = 13, 8
    v = rng.standard_normal((N, 1, d))
    k = np.tile(rng.standard_normal((1, 1, d)), (N, 1, 1))
    out, _ = oracle.attention(rng.standard_normal((1, 1, d)), [N - 1], k, v, 0.3)
    np.testing.assert_allclose(out[0, 0], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)
    out, _ = oracle.attention(np.zeros((1, 1, d)), [N - 1], rng.standard_normal((N, 1, d)), v, 0.3)
    np.testing.assert_allclose(out[0, 0], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_long_context_two_level_scores_closed_form(dtype):
    # 16500 tokens (33 partitions of 512) of 16-bit K/V written through a
    # shuffled block table and read back by the paged gather.  Keys take two
    # values per KV head, +u_g for the first n_a tokens and -u_g after, and
    # query head h holds c_h u_g / |u_g|^2, so every score is +-scale c_h and
    # the softmax average is a closed form of two plain sums:
    #   out = (e^{a} S_A + e^{-a} S_B) / (n_A e^{a} + n_B e^{-a}),  a = scale c_h
    # (c_h = 0: equal scores, the mean of V).  Queries at the last position
    # and at an interior one (causal: keys 0..pos).
    rng = np.random.default_rng(21)
    L, Hkv, G, d, bs, n_a = 16500, 2, 4, 64, 16, 6100
    Hq, scale = Hkv * G, 1.0 / 8.0

    def to_bits(x):
        if dtype == "f16":
            return x.astype(np.float16).view(np.uint16)
        return (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
                .view(np.uint16))

    u_bits = to_bits(rng.standard_normal((Hkv, d)))
    u = oracle.decode(dtype, u_bits)
    kbits = np.empty((L, Hkv, d), np.uint16)
    neg = to_bits(-u)
    kbits[:n_a] = u_bits
    kbits[n_a:] = neg
    vbits = to_bits(rng.standard_normal((L, Hkv, d)))
    nblk = -(-L // bs)
    nb = nblk + 9
    table = rng.permutation(nb)[:nblk].astype(np.int32)
    slots = [oracle.slot(table, t, bs) for t in range(L)]
    kp = np.zeros(oracle.pool_elems(nb, bs, Hkv, d), np.uint16)
    vp = np.zeros_like(kp)
    oracle.scatter(dtype, kbits, vbits, kp, vp, slots, nb, bs, Hkv, d)
    k, v = oracle.gather(dtype, kp, vp, nb, bs, Hkv, d, table, L)
    c = np.array([0.0, 3.0, 12.0, -16.0] * Hkv)
    q = np.empty((2, Hq, d))
    for h in range(Hq):
        ug = u[h // G]
        q[:, h] = c[h] * ug / np.dot(ug, ug)
    positions = [L - 1, 9000]
    out, _ = oracle.attention(q, positions, k, v, scale, n_threads=4)
    vv = oracle.decode(dtype, vbits)
    for r, pos in enumerate(positions):
        na, nbk = min(n_a, pos + 1), max(0, pos + 1 - n_a)
        for h in range(Hq):
            g, a = h // G, scale * c[h]
            sa = vv[:na, g].sum(axis=0)
            sb = vv[n_a:pos + 1, g].sum(axis=0)
            exp = (math.exp(a) * sa + math.exp(-a) * sb) / (na * math.exp(a) + nbk * math.exp(-a))
            np.testing.assert_allclose(out[r, h], exp, rtol=1e-11, atol=1e-13,
                                       err_msg=f"{dtype} row {r} head {h}")


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(5)
    N, d = 9, 4
    k = rng.standard_normal((N, 1, d)) * 0.01
    q = np.ones((1, 1, d))
    k[4, 0, :] = 100.0
    v = rng.standard_normal((N, 1, d))
    out, _ = oracle.attention(q, [N - 1], k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[4, 0], rtol=0, atol=1e-12)


def test_decode_is_last_row_of_prefill():
    # Life of a prompt: the next token needs only the last row of the context matrix
    rng = np.random.default_rng(6)
    N, Hq, Hkv, d = 21, 4, 2, 8
    q = rng.standard_normal((N, Hq, d))
    k = rng.standard_normal((N, Hkv, d))
    v = rng.standard_normal((N, Hkv, d))
    full, _ = oracle.attention(q, np.arange(N), k, v, 0.35)
    last, _ = oracle.attention(q[-1:], [N - 1], k, v, 0.35)
    assert np.array_equal(full[-1], last[0])


def test_chunked_rows_equal_monolithic():
    # chunking changes when rows are computed, not what they are
    rng = np.random.default_rng(7)
    N, Hq, Hkv, d = 40, 2, 1, 8
    q = rng.standard_normal((N, Hq, d))
    k = rng.standard_normal((N, Hkv, d))
    v = rng.standard_normal((N, Hkv, d))
    full, _ = oracle.attention(q, np.arange(N), k, v, 0.3)
    for a, b in [(0, 13), (13, 29), (29, 40)]:
        part, _ = oracle.attention(q[a:b], np.arange(a, b), k[:b], v[:b], 0.3)
        assert np.array_equal(part, full[a:b])


def test_bad_position_rejected():
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 1, 4)), [3], np.zeros((3, 1, 4)), np.zeros((3, 1, 4)), 1.0)


# --------------------------------------------------------------------------
# pool layout, scatter / gather, block copies
# --------------------------------------------------------------------------
def test_layout_hand_computed_offsets():
    # bf16 (x = 8), 2 blocks, H = 2, d = 16, bs = 16; token lands in block 1, offset 3
    nb, H, d, bs = 2, 2, 16, 16
    kp = np.zeros(nb * H * bs * d, np.uint16)
    vp = np.zeros_like(kp)
    key = np.zeros((1, H, d), np.uint16)
    val = np.zeros_like(key)
    key[0, 1, 10] = 0xABCD
    val[0, 1, 10] = 0x1234
    oracle.scatter("bf16", key, val, kp, vp, [1 * bs + 3], nb, bs, H, d)
    # K: ((((1*2+1)*(16/8) + 10//8)*16 + 3)*8 + 10%8) = 922 ; V: ((1*2+1)*16 + 10)*16 + 3 = 931
    assert np.flatnonzero(kp).tolist() == [922] and kp[922] == 0xABCD
    assert np.flatnonzero(vp).tolist() == [931] and vp[931] == 0x1234


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_scatter_gather_roundtrip_bitwise(dtype):
    rng = np.random.default_rng(8)
    nb, H, d, bs, L = 12, 3, 16 if dtype != "f32" else 8, 16, 37
    cont = np.uint32 if dtype == "f32" else np.uint16
    kbits = rng.integers(0, 0x7000, size=(L, H, d)).astype(cont)
    vbits = rng.integers(0, 0x7000, size=(L, H, d)).astype(cont)
    table = rng.permutation(nb)[: -(-L // bs)].astype(np.int32)
    slots = [oracle.slot(table, t, bs) for t in range(L)]
    kp = np.zeros(oracle.pool_elems(nb, bs, H, d), cont)
    vp = np.zeros_like(kp)
    oracle.scatter(dtype, kbits, vbits, kp, vp, slots, nb, bs, H, d)
    k, v = oracle.gather(dtype, kp, vp, nb, bs, H, d, table, L)
    assert np.array_equal(k, oracle.decode(dtype, kbits))
    assert np.array_equal(v, oracle.decode(dtype, vbits))


def test_scatter_skips_padding_slots():
    nb, H, d, bs = 2, 1, 8, 16
    kp = np.zeros(oracle.pool_elems(nb, bs, H, d), np.uint16)
    vp = np.zeros_like(kp)
    ones = np.ones((2, H, d), np.uint16)
    oracle.scatter("f16", ones, ones, kp, vp, [-1, 5], nb, bs, H, d)
    assert kp.sum() == d and vp.sum() == d


def test_gather_rejects_out_of_pool_block():
    kp = np.zeros(oracle.pool_elems(2, 16, 1, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.gather("f16", kp, kp, 2, 16, 1, 8, [5], 3)


def _place_and_attend(dtype, kbits, vbits, qbits, table, nb, bs, H, d, Hq, scale):
    L = kbits.shape[0]
    cont = kbits.dtype
    kp = np.zeros(oracle.pool_elems(nb, bs, H, d), cont)
    vp = np.zeros_like(kp)
    oracle.scatter(dtype, kbits, vbits, kp, vp, [oracle.slot(table, t, bs) for t in range(L)], nb, bs, H, d)
    k, v = oracle.gather(dtype, kp, vp, nb, bs, H, d, table, L)
    return oracle.attention(oracle.decode(dtype, qbits), [L - 1], k, v, scale)[0]


def test_output_invariant_under_block_placement():
    # same logical K/V, different physical placement: bit-for-bit the same output
    rng = np.random.default_rng(9)
    nb, H, d, bs, L, Hq = 16, 2, 16, 16, 70, 4
    kbits = rng.integers(0x3000, 0x3C00, size=(L, H, d)).astype(np.uint16)
    vbits = rng.integers(0x3000, 0x3C00, size=(L, H, d)).astype(np.uint16)
    qbits = rng.integers(0x3000, 0x3C00, size=(1, Hq, d)).astype(np.uint16)
    outs = []
    for seed in range(4):
        table = np.random.default_rng(seed).permutation(nb)[: -(-L // bs)].astype(np.int32)
        outs.append(_place_and_attend("f16", kbits, vbits, qbits, table, nb, bs, H, d, Hq, 0.25))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_shared_prefix_equals_private_copy():
    # two sequences pointing at the same prefix blocks read the same numbers as
    # with private copies of those bytes
    rng = np.random.default_rng(10)
    nb, H, d, bs, Hq = 16, 1, 8, 16, 2
    prefix = rng.integers(0, 0x7000, size=(32, H, d)).astype(np.uint16)
    tails = [rng.integers(0, 0x7000, size=(9, H, d)).astype(np.uint16) for _ in range(2)]
    q = rng.integers(0x3000, 0x3C00, size=(1, Hq, d)).astype(np.uint16)
    kp = np.zeros(oracle.pool_elems(nb, bs, H, d), np.uint16)
    vp = np.zeros_like(kp)
    shared = [3, 7]
    tables_shared = [shared + [10], shared + [12]]
    tables_private = [[0, 1, 2], [4, 5, 6]]
    for tabs in (tables_shared, tables_private):
        for tab, tail in zip(tabs, tails):
            seq = np.concatenate([prefix, tail])
            oracle.scatter("bf16", seq, seq, kp, vp, [oracle.slot(tab, t, bs) for t in range(41)], nb, bs, H, d)
    for i in range(2):
        a = oracle.attention(oracle.decode("bf16", q), [40], *oracle.gather("bf16", kp, vp, nb, bs, H, d,
                                                                            tables_shared[i], 41), 0.3)[0]
        b = oracle.attention(oracle.decode("bf16", q), [40], *oracle.gather("bf16", kp, vp, nb, bs, H, d,
                                                                            tables_private[i], 41), 0.3)[0]
        assert np.array_equal(a, b)


def test_copy_blocks_copies_whole_block():
    nb, H, d, bs = 4, 2, 8, 16
    rng = np.random.default_rng(11)
    kp = rng.integers(0, 65535, size=oracle.pool_elems(nb, bs, H, d)).astype(np.uint16)
    vp = rng.integers(0, 65535, size=kp.size).astype(np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    oracle.copy_blocks("f16", kp, vp, [[1, 3]], nb, bs, H, d)
    blk = H * bs * d
    assert np.array_equal(kp[3 * blk:4 * blk], k0[blk:2 * blk])
    assert np.array_equal(vp[3 * blk:4 * blk], v0[blk:2 * blk])
    assert np.array_equal(kp[:3 * blk], k0[:3 * blk]) and np.array_equal(vp[:3 * blk], v0[:3 * blk])


# --------------------------------------------------------------------------
# block manager model against the pages' worked examples
# --------------------------------------------------------------------------
def test_three_prompts_take_blocks_from_queue_head(tables):
    ex = tables["three_prompts"]
    m = bm.BlockManagerModel(8, ex["block_size"])
    got = []
    for n in ex["prompt_tokens"]:
        s = m.create()
        m.append(s, n)
        got.append(m.table(s))
    assert [len(t) for t in got] == ex["blocks_each"]
    assert got == [[0], [1], [2]]


def test_diagram_table_from_free_queue(tables):
    ex = tables["diagram_in_words"]
    order = ex["table"] + [b for b in range(16) if b not in ex["table"]]
    m = bm.BlockManagerModel(16, 16, order)
    s = m.create()
    slots, cow = m.append(s, 40)
    assert m.table(s) == ex["table"] and cow == []
    assert slots[0] == 112 and slots[17] == 49 and slots[32] == 176


def test_thirty_tokens_two_blocks(tables):
    ex = tables["thirty_tokens"]
    m = bm.BlockManagerModel(8, 16)
    s = m.create()
    m.append(s, ex["tokens"])
    assert len(m.table(s)) == ex["blocks"]
    waste = ex["blocks"] * 16 - ex["tokens"]
    assert ex["slots"] == ex["blocks"] * 16 and 0 <= waste <= ex["max_waste"]


def test_one_block_per_sixteen_tokens():
    m = bm.BlockManagerModel(64, 16)
    s = m.create()
    for L in range(1, 200):
        m.append(s, 1)
        assert len(m.table(s)) == -(-L // 16)
        assert m.num_free() == 64 - len(m.table(s))


def test_finished_blocks_return_immediately():
    m = bm.BlockManagerModel(4, 16)
    a, b = m.create(), m.create()
    m.append(a, 20)  # blocks 0, 1
    m.append(b, 5)   # block 2
    m.release(a)
    assert m.free_queue() == [3, 0, 1]
    c = m.create()
    m.append(c, 17)
    assert m.table(c) == [3, 0]


def test_copy_on_write_touches_one_block():
    m = bm.BlockManagerModel(16, 16)
    root = m.create()
    m.append(root, 40)           # blocks 0, 1, 2 (last one partial)
    kids = [m.fork(root, 40) for _ in range(3)]
    assert all(m.ref[b] == 4 for b in (0, 1, 2))
    slots, cow = m.append(kids[0], 1)
    assert cow == [(2, 3)] and m.table(kids[0]) == [0, 1, 3]
    assert m.table(kids[1]) == [0, 1, 2] and m.table(root) == [0, 1, 2]
    assert m.ref[2] == 3 and m.ref[3] == 1 and slots == [3 * 16 + 8]


def test_full_shared_block_needs_no_copy():
    m = bm.BlockManagerModel(8, 16)
    root = m.create()
    m.append(root, 32)
    kid = m.fork(root, 32)
    slots, cow = m.append(kid, 1)
    assert cow == [] and m.table(kid) == [0, 1, 2] and slots == [32]


def test_out_of_blocks_changes_nothing():
    m = bm.BlockManagerModel(3, 16)
    s = m.create()
    m.append(s, 30)
    before = (m.free_queue(), m.table(s), m.lens[s])
    with pytest.raises(bm.OutOfBlocks):
        m.append(s, 40)
    assert (m.free_queue(), m.table(s), m.lens[s]) == before


# --------------------------------------------------------------------------
# swapping: CPU blocks, the block copy between pools, the model's rules
# --------------------------------------------------------------------------
def test_cpu_blocks_from_the_swap_space(sizing):
    c = sizing["cpu_pool"]
    nb = oracle.blocks_for_budget(c["swap_gib"] * GIB, c["n_layers"], c["n_kv_heads"], c["d_head"],
                                  c["dtype_bytes"], c["block_size"])
    assert nb == c["cpu_blocks"], c["cite"]


def test_swap_blocks_is_a_whole_block_copy():
    rng = np.random.default_rng(7)
    H, d, nb_src, nb_dst = 2, 64, 6, 4
    per = H * 16 * d
    sk = rng.integers(0, 2**16, size=nb_src * per, dtype=np.uint16)
    sv = rng.integers(0, 2**16, size=nb_src * per, dtype=np.uint16)
    dk = np.zeros(nb_dst * per, np.uint16)
    dv = np.zeros_like(dk)
    pairs = [(5, 0), (2, 3), (0, 1)]
    oracle.swap_blocks("bf16", sk, sv, nb_src, dk, dv, nb_dst, pairs, 16, H, d)
    for s, t in pairs:
        assert np.array_equal(dk.reshape(nb_dst, per)[t], sk.reshape(nb_src, per)[s])
        assert np.array_equal(dv.reshape(nb_dst, per)[t], sv.reshape(nb_src, per)[s])
    assert not dk.reshape(nb_dst, per)[2].any()  # untouched block
    with pytest.raises(ValueError):
        oracle.swap_blocks("bf16", sk, sv, nb_src, dk, dv, nb_dst, [(6, 0)], 16, H, d)


def test_swap_out_and_in_restores_the_sequence():
    # a preempted sequence parks its blocks in CPU blocks; its GPU blocks are
    # reused by another sequence meanwhile; swapping in restores every value
    rng = np.random.default_rng(8)
    H, d, nb, ncpu = 2, 64, 8, 6
    m = bm.BlockManagerModel(nb, 16, rng.permutation(nb))
    m.set_swap_space(ncpu)
    kp = np.zeros(nb * H * 16 * d, np.uint16)
    vp = np.zeros_like(kp)
    ck, cv = np.zeros(ncpu * H * 16 * d, np.uint16), np.zeros(ncpu * H * 16 * d, np.uint16)
    a = m.create()
    slots, _ = m.append(a, 70)
    kb = rng.integers(0, 2**16, size=(70, H, d), dtype=np.uint16)
    vb = rng.integers(0, 2**16, size=(70, H, d), dtype=np.uint16)
    oracle.scatter("bf16", kb, vb, kp, vp, slots, nb, 16, H, d)
    out_pairs = m.swap_out(a)
    assert [g for g, _ in out_pairs] == m.free_queue()[-5:]  # released to the tail in logical order
    oracle.swap_blocks("bf16", kp, vp, nb, ck, cv, ncpu, out_pairs, 16, H, d)
    other = m.create()
    s2, _ = m.append(other, 16 * 6)  # takes the freed blocks too
    junk = np.full((96, H, d), 0x7FC0, np.uint16)
    oracle.scatter("bf16", junk, junk, kp, vp, s2, nb, 16, H, d)
    m.release(other)
    in_pairs = m.swap_in(a)
    oracle.swap_blocks("bf16", ck, cv, ncpu, kp, vp, nb, in_pairs, 16, H, d)
    k, v = oracle.gather("bf16", kp, vp, nb, 16, H, d, m.table(a), 70)
    assert np.array_equal(k, oracle.decode("bf16", kb), equal_nan=True)
    assert np.array_equal(v, oracle.decode("bf16", vb), equal_nan=True)


def test_swap_rules():
    m = bm.BlockManagerModel(10, 16, list(range(10)))
    m.set_swap_space(4)
    root = m.create()
    m.append(root, 40)                      # blocks 0, 1, 2
    child = m.fork(root, 40)                # shares them
    assert m.swap_out(root) == [(0, 0), (1, 1), (2, 2)]
    assert [m.ref[b] for b in (0, 1, 2)] == [1, 1, 1] and m.table(child) == [0, 1, 2]
    for op in (lambda: m.append(root, 1), lambda: m.fork(root, 1), lambda: m.swap_out(root),
               lambda: m.blocks_needed(root, 1), lambda: m.padded_tables([root], 4),
               lambda: m.set_swap_space(8)):
        with pytest.raises(bm.StateError):
            op()
    big = m.create()
    m.append(big, 33)                       # three blocks; one CPU block is left
    with pytest.raises(bm.OutOfBlocks):
        m.swap_out(big)
    assert m.cpu_free_queue() == [3] and m.table(big) == [3, 4, 5]
    m.append(big, 16 * 4)                   # the GPU pool is now exhausted
    with pytest.raises(bm.OutOfBlocks):
        m.swap_in(root)
    assert root in m.swapped and m.cpu_free_queue() == [3]
    m.release(root)                         # a swapped-out sequence frees its CPU blocks
    assert m.cpu_free_queue() == [3, 0, 1, 2]
    with pytest.raises(bm.StateError):
        m.swap_in(child)
