"""Swap space in the host block manager, through the C ABI: the rules (host
block queue, all-or-nothing swap-out / swap-in, state errors on a swapped-out
sequence, prefix-cache labels across a swap) as fixed cases, and the
allocator against the reference model under random operation sequences that
mix swapping with appends, forks, cached prefills and frees ("The scheduler:
waiting, running, swapped", vLLM Serving deep dive)."""
import ctypes

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import paged_kv_cache_gather_amd as pkv
from oracle import block_manager as bm


def _pool(nblocks, ncpu, order=None, cache=False):
    p = pkv.paged_kv_alloc(nblocks, 1, 64, "bf16", initial_free_order=order)
    pkv.paged_kv_swap_space(p, ncpu)
    if cache:
        pkv.paged_kv_prefix_cache_enable(p)
    return p


def _state_error(fn):
    with pytest.raises(pkv.PagedKVError) as e:
        fn()
    assert e.value.code == pkv.PKV_ESTATE


def test_swap_out_releases_and_swap_in_reallocates():
    p = _pool(8, 4, np.arange(8))
    a = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, a, 40)
    assert pkv.paged_kv_seq_swap_out(p, a).tolist() == [[0, 0], [1, 1], [2, 2]]
    assert pkv.paged_kv_seq_is_swapped(p, a) and pkv.paged_kv_seq_len(p, a) == 40
    assert pkv.paged_kv_free_queue(p).tolist() == [3, 4, 5, 6, 7, 0, 1, 2]
    assert pkv.paged_kv_cpu_free_queue(p).tolist() == [3]
    assert pkv.paged_kv_seq_swap_in(p, a).tolist() == [[0, 3], [1, 4], [2, 5]]
    assert not pkv.paged_kv_seq_is_swapped(p, a)
    assert pkv.paged_kv_seq_table(p, a).tolist() == [3, 4, 5]
    assert pkv.paged_kv_cpu_free_queue(p).tolist() == [3, 0, 1, 2]


def test_shared_blocks_get_private_host_copies():
    p = _pool(8, 8, np.arange(8))
    root = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, root, 40)
    child = pkv.paged_kv_seq_fork(p, root, 40)
    pkv.paged_kv_seq_swap_out(p, root)
    assert [pkv.paged_kv_block_refcount(p, b) for b in (0, 1, 2)] == [1, 1, 1]
    assert pkv.paged_kv_seq_table(p, child).tolist() == [0, 1, 2]
    assert pkv.paged_kv_num_free(p) == 5


def test_a_swapped_out_sequence_only_swaps_in_frees_or_reads():
    p = _pool(8, 4)
    a = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, a, 20)
    pkv.paged_kv_seq_swap_out(p, a)
    _state_error(lambda: pkv.paged_kv_seq_append(p, a, 1))
    _state_error(lambda: pkv.paged_kv_seq_append_tokens(p, a, [1]))
    _state_error(lambda: pkv.paged_kv_seq_fork(p, a, 5))
    _state_error(lambda: pkv.paged_kv_seq_blocks_needed(p, a, 1))
    _state_error(lambda: pkv.paged_kv_block_tables(p, [a], 4))
    _state_error(lambda: pkv.paged_kv_seq_swap_out(p, a))
    _state_error(lambda: pkv.paged_kv_swap_space(p, 16))
    assert pkv.paged_kv_seq_table(p, a).tolist() == [0, 1]  # host block ids
    pkv.paged_kv_seq_free(p, a)
    assert pkv.paged_kv_cpu_free_queue(p).tolist() == [2, 3, 0, 1]
    b = pkv.paged_kv_seq_create(p)
    _state_error(lambda: pkv.paged_kv_seq_swap_in(p, b))


def test_swapping_is_all_or_nothing():
    p = _pool(6, 2, np.arange(6))
    a = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, a, 33)  # 3 blocks, 2 host blocks
    with pytest.raises(pkv.OutOfBlocks):
        pkv.paged_kv_seq_swap_out(p, a)
    assert not pkv.paged_kv_seq_is_swapped(p, a) and pkv.paged_kv_seq_table(p, a).tolist() == [0, 1, 2]
    assert pkv.paged_kv_cpu_free_queue(p).tolist() == [0, 1]
    pkv.paged_kv_swap_space(p, 4)
    pkv.paged_kv_seq_swap_out(p, a)
    b = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, b, 16 * 5)  # leaves one free GPU block
    with pytest.raises(pkv.OutOfBlocks):
        pkv.paged_kv_seq_swap_in(p, a)
    assert pkv.paged_kv_seq_is_swapped(p, a) and pkv.paged_kv_num_free(p) == 1


def test_pairs_buffer_too_small_changes_nothing():
    lib = ctypes.CDLL(pkv.LIB_PATH)
    p = _pool(8, 8)
    a = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, a, 40)
    buf = (ctypes.c_int32 * 4)()
    n = ctypes.c_int64()
    lib.paged_kv_seq_swap_out.restype = ctypes.c_int
    rc = lib.paged_kv_seq_swap_out(p.handle, ctypes.c_int64(a), buf, ctypes.c_int64(2), ctypes.byref(n))
    assert rc == pkv.PKV_EINVAL and not pkv.paged_kv_seq_is_swapped(p, a)


def test_swapped_in_blocks_are_labelled_again_when_their_text_is_not_cached():
    p = _pool(8, 8, np.arange(8), cache=True)
    toks = list(range(40))
    a, _ = pkv.paged_kv_seq_create_cached(p, toks)
    pkv.paged_kv_seq_append_tokens(p, a, toks)
    assert pkv.paged_kv_prefix_cache_stats(p)["cached_blocks"] == 2
    pkv.paged_kv_seq_swap_out(p, a)             # blocks 0, 1 keep their labels in the queue
    b = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, b, 16 * 8)       # takes every block: labels evicted
    assert pkv.paged_kv_prefix_cache_stats(p)["cached_blocks"] == 0
    pkv.paged_kv_seq_free(p, b)
    pkv.paged_kv_seq_swap_in(p, a)
    assert pkv.paged_kv_prefix_cache_stats(p)["cached_blocks"] == 2
    c, n = pkv.paged_kv_seq_create_cached(p, toks + [7])
    assert n == 32 and pkv.paged_kv_seq_table(p, c).tolist() == pkv.paged_kv_seq_table(p, a)[:2].tolist()


def test_swap_blocks_validates_before_launch():
    lib = ctypes.CDLL(pkv.LIB_PATH)
    lib.paged_kv_swap_blocks.restype = ctypes.c_int
    fake = ctypes.c_void_p(1 << 20)
    i64 = ctypes.c_int64

    def call(dtype=pkv.PKV_BF16, n=4, src_nb=8, bs=16, ptr=fake):
        return lib.paged_kv_swap_blocks(ptr, ptr, i64(src_nb), ptr, ptr, i64(8), ptr, n, 8, 128, bs, dtype, None)
    assert call(dtype=7) == pkv.PKV_EINVAL
    assert call(bs=32) == pkv.PKV_EUNSUPPORTED
    assert call(src_nb=0) == pkv.PKV_EINVAL
    assert call(n=-1) == pkv.PKV_EINVAL
    assert call(ptr=None) == pkv.PKV_EINVAL
    assert call(n=0) == pkv.PKV_OK


# ---- against the model --------------------------------------------------
FAM = [np.random.default_rng(300 + f).integers(0, 40, size=200).tolist() for f in range(2)]
ops = st.lists(st.tuples(st.sampled_from(["create", "append", "append_tokens", "fork", "free", "swap_out",
                                          "swap_out", "swap_in", "swap_in", "prefill", "space"]),
                         st.integers(0, 1000), st.integers(0, 60)), min_size=1, max_size=60)


def _compare(p, m, live_p, live_m):
    assert pkv.paged_kv_free_queue(p).tolist() == m.free_queue()
    assert pkv.paged_kv_cpu_free_queue(p).tolist() == m.cpu_free_queue()
    for a, b in zip(live_p, live_m):
        assert pkv.paged_kv_seq_table(p, a).tolist() == m.table(b)
        assert pkv.paged_kv_seq_len(p, a) == m.lens[b]
        assert pkv.paged_kv_seq_is_swapped(p, a) == (b in m.swapped)
    for blk in range(m.num_blocks):
        assert pkv.paged_kv_block_refcount(p, blk) == m.ref[blk]
    assert pkv.paged_kv_prefix_cache_stats(p) == m.cache_stats()


def _both(fp, fm):
    """Run the library call and the model call; both fail the same way or both succeed."""
    try:
        rm = fm()
    except bm.OutOfBlocks:
        with pytest.raises(pkv.OutOfBlocks):
            fp()
        return None, None
    except bm.StateError:
        with pytest.raises(pkv.PagedKVError) as e:
            fp()
        assert e.value.code == pkv.PKV_ESTATE
        return None, None
    return fp(), rm


@settings(max_examples=200, deadline=None)
@given(ops=ops, nblocks=st.integers(1, 30), ncpu=st.integers(0, 20), seed=st.integers(0, 2**16))
def test_swap_matches_model(ops, nblocks, ncpu, seed):
    order = np.random.default_rng(seed).permutation(nblocks)
    p = _pool(nblocks, ncpu, order, cache=True)
    m = bm.BlockManagerModel(nblocks, 16, order)
    m.set_swap_space(ncpu)
    m.enable_caching(True)
    live_p, live_m = [], []
    for op, pick, n in ops:
        if op == "create" or (not live_p and op not in ("prefill", "space")):
            live_p.append(pkv.paged_kv_seq_create(p))
            live_m.append(m.create())
        elif op == "prefill":
            toks = FAM[pick % 2][:n + 1]
            sp, np_ = pkv.paged_kv_seq_create_cached(p, toks)
            sm, nm = m.create_cached(toks)
            assert np_ == nm
            live_p.append(sp)
            live_m.append(sm)
            r = _both(lambda: pkv.paged_kv_seq_append_tokens(p, sp, toks[np_:]), lambda: m.append_tokens(sm, toks[nm:]))
            if r[0] is not None:
                assert r[0][0].tolist() == r[1][0] and r[0][1] == r[1][1]
        elif op == "space":
            r = _both(lambda: pkv.paged_kv_swap_space(p, n % 21), lambda: m.set_swap_space(n % 21))
        else:
            i = pick % len(live_p)
            a, b = live_p[i], live_m[i]
            if op == "append":
                r = _both(lambda: pkv.paged_kv_seq_append(p, a, n), lambda: m.append(b, n))
                if r[0] is not None:
                    assert r[0][0].tolist() == r[1][0] and r[0][1] == r[1][1]
            elif op == "append_tokens":
                toks = FAM[pick % 2][:n]
                r = _both(lambda: pkv.paged_kv_seq_append_tokens(p, a, toks), lambda: m.append_tokens(b, toks))
                if r[0] is not None:
                    assert r[0][0].tolist() == r[1][0] and r[0][1] == r[1][1]
            elif op == "fork":
                k = pick % (m.lens[b] + 1)
                r = _both(lambda: pkv.paged_kv_seq_fork(p, a, k), lambda: m.fork(b, k))
                if r[0] is not None:
                    live_p.append(r[0])
                    live_m.append(r[1])
            elif op == "free":
                pkv.paged_kv_seq_free(p, live_p.pop(i))
                m.release(live_m.pop(i))
            elif op == "swap_out":
                r = _both(lambda: pkv.paged_kv_seq_swap_out(p, a), lambda: m.swap_out(b))
                if r[0] is not None:
                    assert [tuple(x) for x in r[0].tolist()] == r[1]
            elif op == "swap_in":
                r = _both(lambda: pkv.paged_kv_seq_swap_in(p, a), lambda: m.swap_in(b))
                if r[0] is not None:
                    assert [tuple(x) for x in r[0].tolist()] == r[1]
        _compare(p, m, live_p, live_m)
