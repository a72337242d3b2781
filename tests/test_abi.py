"""The C-ABI library on the host: it loads, exports every entry point the
header declares, sizes pools like the oracle, and its block manager matches
the reference model table for table and slot for slot.  No GPU calls."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import paged_kv_cache_gather_amd as pkv
from oracle import block_manager as bm
from tests.conftest import ROOT


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pagedkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_entry_points():
    names = _declared_functions()
    for n in ("paged_kv_alloc", "reshape_and_cache", "paged_attention_decode", "paged_attention_prefill_chunk"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pkv.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_sizing_matches_oracle():
    for L, H, d, dt, b in [(32, 8, 128, "bf16", 2), (40, 40, 128, "f16", 2), (22, 4, 64, "f16", 2), (1, 2, 64, "f32", 4)]:
        assert pkv.paged_kv_bytes_per_token(L, H, d, dt) == oracle.kv_bytes_per_token(L, H, d, b)
        budget = 54 << 30
        assert pkv.paged_kv_blocks_for_budget(budget, L, H, d, dt) == oracle.blocks_for_budget(budget, L, H, d, b)
    kb, vb = pkv.paged_kv_pool_bytes(32768, 8, 128, "bf16")
    assert kb == vb == 32768 * 8 * 16 * 128 * 2


def test_pool_descriptor_validation():
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_kv_alloc(16, 2, 96, "f16")
    assert e.value.code == pkv.PKV_EUNSUPPORTED
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_kv_alloc(16, 2, 64, "f16", block_size=32)
    assert e.value.code == pkv.PKV_EUNSUPPORTED
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_kv_alloc(4, 2, 64, "f16", initial_free_order=[0, 1, 1, 2])
    assert e.value.code == pkv.PKV_EINVAL
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_kv_alloc(0, 2, 64, "f16")


def test_unknown_sequence_and_bad_fork():
    p = pkv.paged_kv_alloc(8, 1, 64, "f16")
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_kv_seq_append(p, 99, 1)
    assert e.value.code == pkv.PKV_ESTATE
    s = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, s, 5)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_kv_seq_fork(p, s, 6)
    assert e.value.code == pkv.PKV_EINVAL
    pkv.paged_kv_seq_free(p, s)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_kv_seq_free(p, s)
    assert e.value.code == pkv.PKV_ESTATE


def test_out_of_blocks_is_all_or_nothing():
    p = pkv.paged_kv_alloc(3, 1, 64, "f16")
    s = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, s, 30)
    before = (pkv.paged_kv_free_queue(p).tolist(), pkv.paged_kv_seq_table(p, s).tolist(), pkv.paged_kv_seq_len(p, s))
    with pytest.raises(pkv.OutOfBlocks):
        pkv.paged_kv_seq_append(p, s, 40)
    after = (pkv.paged_kv_free_queue(p).tolist(), pkv.paged_kv_seq_table(p, s).tolist(), pkv.paged_kv_seq_len(p, s))
    assert before == after


def test_diagram_example_through_the_abi():
    order = [7, 3, 11] + [b for b in range(16) if b not in (7, 3, 11)]
    p = pkv.paged_kv_alloc(16, 1, 64, "f16", initial_free_order=order)
    s = pkv.paged_kv_seq_create(p)
    slots, cow = pkv.paged_kv_seq_append(p, s, 40)
    assert pkv.paged_kv_seq_table(p, s).tolist() == [7, 3, 11] and cow == []
    assert [slots[0], slots[17], slots[32]] == [112, 49, 176]
    tab, lens = pkv.paged_kv_block_tables(p, [s], 5)
    assert tab.tolist() == [[7, 3, 11, -1, -1]] and lens.tolist() == [40]


def _compare(p, m, sids_p, sids_m):
    assert pkv.paged_kv_free_queue(p).tolist() == m.free_queue()
    for a, b in zip(sids_p, sids_m):
        assert pkv.paged_kv_seq_table(p, a).tolist() == m.table(b)
        assert pkv.paged_kv_seq_len(p, a) == m.lens[b]
    for blk in range(m.num_blocks):
        assert pkv.paged_kv_block_refcount(p, blk) == m.ref[blk]


ops = st.lists(st.tuples(st.sampled_from(["create", "append", "fork", "free"]),
                         st.integers(0, 1000), st.integers(0, 70)), min_size=1, max_size=60)


@settings(max_examples=150, deadline=None)
@given(ops=ops, nblocks=st.integers(1, 40), seed=st.integers(0, 2**16))
def test_block_manager_matches_model(ops, nblocks, seed):
    order = np.random.default_rng(seed).permutation(nblocks)
    p = pkv.paged_kv_alloc(nblocks, 1, 64, "f16", initial_free_order=order)
    m = bm.BlockManagerModel(nblocks, 16, order)
    live_p, live_m = [], []
    for op, pick, n in ops:
        if op == "create" or not live_p:
            live_p.append(pkv.paged_kv_seq_create(p))
            live_m.append(m.create())
            continue
        i = pick % len(live_p)
        if op == "append":
            try:
                sm, cm = m.append(live_m[i], n)
            except bm.OutOfBlocks:
                with pytest.raises(pkv.OutOfBlocks):
                    pkv.paged_kv_seq_append(p, live_p[i], n)
                continue
            sp, cp = pkv.paged_kv_seq_append(p, live_p[i], n)
            assert sp.tolist() == sm and cp == cm
        elif op == "fork":
            k = pick % (m.lens[live_m[i]] + 1)
            live_p.append(pkv.paged_kv_seq_fork(p, live_p[i], k))
            live_m.append(m.fork(live_m[i], k))
        elif op == "free":
            pkv.paged_kv_seq_free(p, live_p.pop(i))
            m.release(live_m.pop(i))
        _compare(p, m, live_p, live_m)
    # conservation: every block is either queued or referenced
    referenced = {b for s in live_m for b in m.table(s)}
    assert len(referenced) + m.num_free() == nblocks
    assert pkv.paged_kv_num_free(p) == m.num_free()


step_ops = st.lists(st.tuples(st.sampled_from(["create", "fork", "free", "step"]),
                              st.integers(0, 1000), st.integers(0, 40),
                              st.lists(st.integers(0, 20), min_size=1, max_size=8)),
                    min_size=1, max_size=40)


@settings(max_examples=150, deadline=None)
@given(ops=step_ops, nblocks=st.integers(1, 40), seed=st.integers(0, 2**16))
def test_batched_append_matches_model(ops, nblocks, seed):
    # paged_kv_seqs_append = the per-sequence appends in list order, stopping
    # at the first that cannot be made (the ones before it stay made)
    order = np.random.default_rng(seed).permutation(nblocks)
    p = pkv.paged_kv_alloc(nblocks, 1, 64, "f16", initial_free_order=order)
    m = bm.BlockManagerModel(nblocks, 16, order)
    live_p, live_m = [], []
    for op, pick, n, counts in ops:
        if op == "create" or not live_p:
            live_p.append(pkv.paged_kv_seq_create(p))
            live_m.append(m.create())
            continue
        i = pick % len(live_p)
        if op == "fork":
            k = pick % (m.lens[live_m[i]] + 1)
            live_p.append(pkv.paged_kv_seq_fork(p, live_p[i], k))
            live_m.append(m.fork(live_m[i], k))
        elif op == "free":
            pkv.paged_kv_seq_free(p, live_p.pop(i))
            m.release(live_m.pop(i))
        else:
            idx = [(pick + 7 * j) % len(live_p) for j in range(len(counts))]
            want_slots, want_cow, done = [], [], len(idx)
            for j, (k, c) in enumerate(zip(idx, counts)):
                try:
                    sm, cm = m.append(live_m[k], c)
                except bm.OutOfBlocks:
                    done = j
                    break
                want_slots += sm
                want_cow += cm
            seqs = [live_p[k] for k in idx]
            if done == len(idx):
                sp, cp = pkv.paged_kv_seqs_append(p, seqs, counts)
            else:
                with pytest.raises(pkv.OutOfBlocks) as e:
                    pkv.paged_kv_seqs_append(p, seqs, counts)
                assert e.value.n_done == done
                sp, cp = e.value.slots, e.value.cow
            assert sp.tolist() == want_slots and cp == want_cow
        _compare(p, m, live_p, live_m)


def test_batched_append_defaults_and_errors():
    p = pkv.paged_kv_alloc(8, 1, 64, "f16")
    a, b = pkv.paged_kv_seq_create(p), pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, a, 20)
    c = pkv.paged_kv_seq_fork(p, a, 20)  # shares a partly filled block with a
    shared = int(pkv.paged_kv_seq_table(p, a)[1])
    slots, cow = pkv.paged_kv_seqs_append(p, [a, b, c])  # one token each
    assert [pkv.paged_kv_seq_len(p, x) for x in (a, b, c)] == [21, 1, 21]
    # a copies the shared block; c, its last holder by then, writes in place
    fresh = int(pkv.paged_kv_seq_table(p, a)[1])
    assert cow == [(shared, fresh)] and int(pkv.paged_kv_seq_table(p, c)[1]) == shared
    assert slots.tolist() == [fresh * 16 + 4, int(pkv.paged_kv_seq_table(p, b)[0]) * 16, shared * 16 + 4]
    assert pkv.paged_kv_seqs_append(p, [], None)[0].size == 0
    with pytest.raises(pkv.PagedKVError) as e:  # negative count: nothing changes
        pkv.paged_kv_seqs_append(p, [a, b], [1, -1])
    assert e.value.code == pkv.PKV_EINVAL and pkv.paged_kv_seq_len(p, a) == 21
    with pytest.raises(pkv.PagedKVError) as e:  # unknown sequence part-way
        pkv.paged_kv_seqs_append(p, [a, 12345, b], [2, 1, 1])
    assert e.value.code == pkv.PKV_ESTATE and e.value.n_done == 1 and e.value.slots.size == 2
    assert [pkv.paged_kv_seq_len(p, x) for x in (a, b)] == [23, 1]
    pkv.paged_kv_swap_space(p, 8)
    pkv.paged_kv_seq_swap_out(p, b)
    with pytest.raises(pkv.PagedKVError) as e:  # swapped-out sequence part-way
        pkv.paged_kv_seqs_append(p, [a, b], [1, 1])
    assert e.value.code == pkv.PKV_ESTATE and e.value.n_done == 1


def test_device_entry_points_validate_before_launch():
    # host-side validation returns codes without touching a GPU
    lib = ctypes.CDLL(pkv.LIB_PATH)
    lib.paged_attention_decode.restype = ctypes.c_int
    rc = lib.paged_attention_decode(None, 0, None, None, None, None, 1, None, 1, 32, 8, 96, 16,
                                    ctypes.c_int64(8), 16, ctypes.c_float(0.1), 2, None, ctypes.c_int64(0), None)
    assert rc == pkv.PKV_EUNSUPPORTED
    rc = lib.paged_attention_decode(None, 0, None, None, None, None, 1, None, 1, 32, 8, 128, 16,
                                    ctypes.c_int64(8), 64, ctypes.c_float(0.1), 2, None, ctypes.c_int64(0), None)
    assert rc == pkv.PKV_EINVAL  # max_context_len beyond the table width
    rc = lib.paged_attention_decode(None, 0, None, None, None, None, 4, None, 1, 30, 8, 128, 16,
                                    ctypes.c_int64(8), 64, ctypes.c_float(0.1), 2, None, ctypes.c_int64(0), None)
    assert rc == pkv.PKV_EINVAL  # 30 % 8
    lib.reshape_and_cache.restype = ctypes.c_int
    rc = lib.reshape_and_cache(None, None, ctypes.c_int64(1024), ctypes.c_int64(1024), None, None, None,
                               ctypes.c_int64(4), ctypes.c_int64(8), 8, 128, 16, 2, None)
    assert rc == pkv.PKV_EINVAL
    assert pkv.paged_attention_decode_workspace_bytes(256, 32, 128, 512) == 0
    part = pkv.paged_attention_decode_partition_size()
    assert pkv.paged_attention_decode_workspace_bytes(256, 32, 128, 4096) == 256 * 32 * (-(-4096 // part)) * 130 * 4


def test_fp8_entry_points_validate_before_launch():
    lib = ctypes.CDLL(pkv.LIB_PATH)
    f8, bf16, f32 = pkv.PKV_FP8_E4M3, pkv.PKV_BF16, pkv.PKV_F32
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    i64, flt = ctypes.c_int64, ctypes.c_float
    lib.paged_attention_decode.restype = ctypes.c_int
    # 8-bit pools through the 16-bit entry point
    rc = lib.paged_attention_decode(fake, f32, fake, fake, fake, fake, 4, fake, 1, 32, 8, 128, 16, i64(8), 64,
                                    flt(0.1), f8, fake, i64(1 << 20), None)
    assert rc == pkv.PKV_EINVAL
    lib.paged_attention_decode_fp8.restype = ctypes.c_int

    def dec(q_dtype=bf16, out_dtype=f32, ks=1.0, vs=1.0, d=128):
        return lib.paged_attention_decode_fp8(fake, out_dtype, fake, q_dtype, fake, fake, flt(ks), flt(vs), fake, 4,
                                              fake, 1, 32, 8, d, 16, i64(8), 64, flt(0.1), fake, i64(1 << 20), None)
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("inf"), 1.0), (1.0, float("nan"))):
        assert dec(ks=ks, vs=vs) == pkv.PKV_EINVAL
    assert dec(q_dtype=f32) == pkv.PKV_EINVAL        # queries must be 16-bit
    assert dec(q_dtype=f8) == pkv.PKV_EINVAL
    assert dec(out_dtype=pkv.PKV_F16) == pkv.PKV_EINVAL  # out: f32 or the query's dtype
    assert dec(d=96) == pkv.PKV_EUNSUPPORTED
    lib.reshape_and_cache_fp8.restype = ctypes.c_int

    def write(src=bf16, ks=1.0, vs=1.0):
        return lib.reshape_and_cache_fp8(fake, fake, src, i64(1024), i64(1024), fake, fake, fake, i64(4), i64(8), 8,
                                         128, 16, flt(ks), flt(vs), None)
    assert write(src=f8) == pkv.PKV_EINVAL
    assert write(ks=0.0) == pkv.PKV_EINVAL and write(vs=float("inf")) == pkv.PKV_EINVAL
    assert write(ks=1e-45) == pkv.PKV_EINVAL  # reciprocal overflows


def test_one_call_decode_steps_validate_before_launch():
    # paged_attention_decode_append / _fp8_append check every argument (cache
    # write and attention alike) before launching anything; with fake device
    # pointers and no GPU, a launch would surface as PKV_EHIP instead
    lib = ctypes.CDLL(pkv.LIB_PATH)
    f8, bf16, f32 = pkv.PKV_FP8_E4M3, pkv.PKV_BF16, pkv.PKV_F32
    fake = ctypes.c_void_p(1 << 20)
    i64, flt = ctypes.c_int64, ctypes.c_float
    lib.paged_attention_decode_append.restype = ctypes.c_int

    def app(kv=bf16, k_new=fake, slots=fake, kstride=1024, d=128, max_ctx=64, maxb=4):
        return lib.paged_attention_decode_append(fake, f32, fake, k_new, fake, i64(kstride), i64(1024), slots, fake,
                                                 fake, fake, maxb, fake, 1, 32, 8, d, 16, i64(8), max_ctx, flt(0.1),
                                                 kv, fake, i64(1 << 20), None)
    assert app(kv=f8) == pkv.PKV_EINVAL             # 8-bit pools take the _fp8 call
    assert app(k_new=None) == pkv.PKV_EINVAL
    assert app(slots=None) == pkv.PKV_EINVAL
    assert app(kstride=1000) == pkv.PKV_EINVAL      # shorter than a row of 8 x 128
    assert app(k_new=ctypes.c_void_p((1 << 20) + 2)) == pkv.PKV_EINVAL  # unaligned rows
    assert app(d=96) == pkv.PKV_EUNSUPPORTED
    assert app(max_ctx=80) == pkv.PKV_EINVAL        # beyond the table width: the attention's check
    for kv in (f32, pkv.PKV_F16):                    # fp32 pools write first: still nothing launched
        assert app(kv=kv, max_ctx=80) == pkv.PKV_EINVAL
    lib.paged_attention_decode_fp8_append.restype = ctypes.c_int

    def app8(q_dtype=bf16, ks=1.0, vs=1.0, slots=fake, max_ctx=64):
        return lib.paged_attention_decode_fp8_append(fake, f32, fake, q_dtype, fake, fake, i64(1024), i64(1024), slots,
                                                     fake, fake, flt(ks), flt(vs), fake, 4, fake, 1, 32, 8, 128, 16,
                                                     i64(8), max_ctx, flt(0.1), fake, i64(1 << 20), None)
    assert app8(q_dtype=f32) == pkv.PKV_EINVAL
    assert app8(ks=0.0) == pkv.PKV_EINVAL and app8(vs=float("nan")) == pkv.PKV_EINVAL
    assert app8(ks=1e-45) == pkv.PKV_EINVAL        # reciprocal overflows
    assert app8(slots=None) == pkv.PKV_EINVAL
    assert app8(max_ctx=80) == pkv.PKV_EINVAL


def test_fp8_pool_sizing():
    # one byte per element: half the bytes per token of a 16-bit cache, twice the blocks per budget
    assert pkv.paged_kv_bytes_per_token(32, 8, 128, "fp8_e4m3") == oracle.kv_bytes_per_token(32, 8, 128, 1)
    budget = 54 << 30
    assert pkv.paged_kv_blocks_for_budget(budget, 32, 8, 128, "fp8_e4m3") == oracle.blocks_for_budget(
        budget, 32, 8, 128, 1)
    assert pkv.paged_kv_pool_bytes(1024, 8, 128, "fp8_e4m3") == (1024 * 8 * 16 * 128,) * 2


def _whole_rule(B, Hq, Hkv, d, dtype, L):
    """The whole-context rule as include/pagedkv.h states it."""
    es = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[dtype]
    P, G = B * Hkv, Hq // Hkv
    if es == 4:
        if L > 2048 or G * d * 4 > 1024:
            return False
        if P <= 256:
            return P >= 128 or L <= 1536
        return 448 <= P <= 512 and L * 2 * d * 4 >= 384 * 1024
    if L > 4096:
        return False
    if P <= 256:
        return P >= 128 or L <= 1536
    return 384 <= P <= 512 and L <= 2048


def test_whole_context_rule_as_documented():
    # host-only: paged_attention_decode_whole_context against the header's
    # statement of the rule over a grid of sizes, every K/V dtype
    f = pkv.paged_attention_decode_whole_context
    for dtype in ("f32", "f16", "bf16", "fp8_e4m3"):
        for Hq, Hkv, d in ((32, 8, 128), (32, 4, 64), (64, 8, 128), (8, 2, 64), (4, 2, 128), (40, 40, 128)):
            for B in (1, 8, 15, 16, 31, 32, 47, 48, 56, 64, 65, 128, 129, 256):
                for L in (0, 1, 384, 767, 768, 1535, 1536, 1537, 2048, 2049, 3000, 4096, 4097):
                    assert bool(f(B, Hq, Hkv, d, dtype, L)) == _whole_rule(B, Hq, Hkv, d, dtype, L), \
                        (B, Hq, Hkv, d, dtype, L)
    assert not f(0, 32, 8, 128, "bf16", 100) and not f(8, 30, 4, 64, "f16", 100)
