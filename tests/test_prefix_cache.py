"""Automatic prefix caching in the host block manager, through the C ABI:
the rules the pages state ("Trick 3, Prefix caching", How AI actually answers
you; "Prefix caching (automatic KV reuse)", vLLM Serving deep dive) as fixed
cases, and the allocator against the reference model under random operation
sequences (tables, lengths, free queue, reference counts, cache counters)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import paged_kv_cache_gather_amd as pkv
from oracle import block_manager as bm


def _pool(nblocks, order=None, cache=True):
    p = pkv.paged_kv_alloc(nblocks, 1, 64, "f16", initial_free_order=order)
    if cache:
        pkv.paged_kv_prefix_cache_enable(p)
    return p


def _prefill(p, tokens):
    """A request: reuse what is cached, then append (compute) the rest."""
    s, n = pkv.paged_kv_seq_create_cached(p, tokens)
    pkv.paged_kv_seq_append_tokens(p, s, tokens[n:])
    return s, n


def test_only_full_blocks_are_cached_and_reused():
    p = _pool(32)
    a, n = _prefill(p, list(range(40)))
    assert n == 0
    assert pkv.paged_kv_prefix_cache_stats(p)["cached_blocks"] == 2  # the third block is partial
    b, n = pkv.paged_kv_seq_create_cached(p, list(range(40)) + [99] * 10)
    assert n == 32
    assert pkv.paged_kv_seq_table(p, b).tolist() == pkv.paged_kv_seq_table(p, a)[:2].tolist()
    for blk in pkv.paged_kv_seq_table(p, b):
        assert pkv.paged_kv_block_refcount(p, int(blk)) == 2


def test_a_label_covers_the_whole_text_up_to_its_block():
    p = _pool(32)
    _prefill(p, list(range(32)) + [7])
    # equal second block after a different first block: nothing is reused
    _, n = pkv.paged_kv_seq_create_cached(p, [1000] * 16 + list(range(16, 32)) + [5])
    assert n == 0
    # equal first block, different second block: one block
    _, n = pkv.paged_kv_seq_create_cached(p, list(range(16)) + [2000] * 16 + [5])
    assert n == 16


def test_the_prompts_last_token_is_always_computed():
    p = _pool(32)
    _prefill(p, list(range(48)))
    assert pkv.paged_kv_seq_create_cached(p, list(range(48)))[1] == 32
    assert pkv.paged_kv_seq_create_cached(p, list(range(49)))[1] == 48


def test_unused_cached_blocks_are_evicted_least_recently_released_first():
    p = _pool(6, order=np.arange(6))
    ta, tb = list(range(33)), list(range(100, 133))
    a, _ = _prefill(p, ta)  # blocks 0, 1 (labelled), 2
    b, _ = _prefill(p, tb)  # blocks 3, 4 (labelled), 5
    pkv.paged_kv_seq_free(p, a)
    pkv.paged_kv_seq_free(p, b)
    assert pkv.paged_kv_free_queue(p).tolist() == [0, 1, 2, 3, 4, 5]
    c = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, c, 40)  # takes 0, 1, 2 from the head: a's labels are evicted
    assert pkv.paged_kv_seq_create_cached(p, ta)[1] == 0
    assert pkv.paged_kv_seq_create_cached(p, tb)[1] == 32


def test_a_hit_takes_a_cached_block_out_of_the_free_queue():
    p = _pool(8, order=np.arange(8))
    a, _ = _prefill(p, list(range(40)))
    pkv.paged_kv_seq_free(p, a)
    assert pkv.paged_kv_num_free(p) == 8
    b, n = pkv.paged_kv_seq_create_cached(p, list(range(40)))
    assert n == 32
    table = pkv.paged_kv_seq_table(p, b).tolist()
    assert table == [0, 1]
    assert not set(table) & set(pkv.paged_kv_free_queue(p).tolist())
    assert pkv.paged_kv_num_free(p) == 6


def test_turning_caching_off_drops_every_label():
    p = _pool(16)
    _prefill(p, list(range(40)))
    pkv.paged_kv_prefix_cache_enable(p, False)
    assert pkv.paged_kv_prefix_cache_stats(p)["cached_blocks"] == 0
    pkv.paged_kv_prefix_cache_enable(p, True)
    assert pkv.paged_kv_seq_create_cached(p, list(range(40)))[1] == 0


def test_unknown_tokens_are_never_labelled():
    p = _pool(16)
    s = pkv.paged_kv_seq_create(p)
    pkv.paged_kv_seq_append(p, s, 20)  # no token ids
    pkv.paged_kv_seq_append_tokens(p, s, list(range(20, 40)))
    assert pkv.paged_kv_prefix_cache_stats(p)["cached_blocks"] == 0


def test_a_fork_continues_its_parents_labels():
    p = _pool(16)
    a, _ = _prefill(p, list(range(20)))
    child = pkv.paged_kv_seq_fork(p, a, 20)
    pkv.paged_kv_seq_append_tokens(p, child, list(range(20, 32)))  # fills block 1 (a copy of the shared one)
    assert pkv.paged_kv_seq_create_cached(p, list(range(40)))[1] == 32


def test_the_caching_calls_validate():
    p = _pool(4)
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_kv_seq_append_tokens(p, 12345, [1, 2])
    s, n = pkv.paged_kv_seq_create_cached(p, [])
    assert n == 0 and pkv.paged_kv_seq_len(p, s) == 0


# ---- against the model --------------------------------------------------
FAMILIES = [np.random.default_rng(100 + f).integers(0, 50, size=200).tolist() for f in range(3)]

ops = st.lists(st.tuples(st.sampled_from(["prefill", "prefill", "append_tokens", "append", "fork", "free",
                                          "toggle"]),
                         st.integers(0, 1000), st.integers(0, 70)), min_size=1, max_size=50)


def _compare(p, m, live_p, live_m):
    assert pkv.paged_kv_free_queue(p).tolist() == m.free_queue()
    for a, b in zip(live_p, live_m):
        assert pkv.paged_kv_seq_table(p, a).tolist() == m.table(b)
        assert pkv.paged_kv_seq_len(p, a) == m.lens[b]
    for blk in range(m.num_blocks):
        assert pkv.paged_kv_block_refcount(p, blk) == m.ref[blk]
    assert pkv.paged_kv_prefix_cache_stats(p) == m.cache_stats()


@settings(max_examples=150, deadline=None)
@given(ops=ops, nblocks=st.integers(1, 40), seed=st.integers(0, 2**16))
def test_prefix_cache_matches_model(ops, nblocks, seed):
    rng = np.random.default_rng(seed)
    order = rng.permutation(nblocks)
    p = _pool(nblocks, order)
    m = bm.BlockManagerModel(nblocks, 16, order)
    m.enable_caching(True)
    caching = True
    live_p, live_m = [], []
    for op, pick, n in ops:
        if op == "toggle":
            caching = not caching
            pkv.paged_kv_prefix_cache_enable(p, caching)
            m.enable_caching(caching)
        elif op == "prefill" or not live_p:
            fam = FAMILIES[pick % len(FAMILIES)]
            toks = list(fam[:n + 1])
            if pick % 7 == 0 and len(toks) > 20:  # a prompt that diverges inside
                toks[17] = 999
            sp, np_ = pkv.paged_kv_seq_create_cached(p, toks)
            sm, nm = m.create_cached(toks)
            assert np_ == nm
            live_p.append(sp)
            live_m.append(sm)
            op, n, tail = "append_tokens", len(toks) - nm, toks[nm:]
            i = len(live_p) - 1
        else:
            i = pick % len(live_p)
            tail = FAMILIES[pick % len(FAMILIES)][m.lens[live_m[i]] % 100:][:n]
        if op == "append_tokens":
            try:
                sm_, cm = m.append_tokens(live_m[i], tail)
            except bm.OutOfBlocks:
                with pytest.raises(pkv.OutOfBlocks):
                    pkv.paged_kv_seq_append_tokens(p, live_p[i], tail)
            else:
                sp_, cp = pkv.paged_kv_seq_append_tokens(p, live_p[i], tail)
                assert sp_.tolist() == sm_ and cp == cm
        elif op == "append":
            try:
                sm_, cm = m.append(live_m[i], n)
            except bm.OutOfBlocks:
                with pytest.raises(pkv.OutOfBlocks):
                    pkv.paged_kv_seq_append(p, live_p[i], n)
            else:
                sp_, cp = pkv.paged_kv_seq_append(p, live_p[i], n)
                assert sp_.tolist() == sm_ and cp == cm
        elif op == "fork":
            k = pick % (m.lens[live_m[i]] + 1)
            live_p.append(pkv.paged_kv_seq_fork(p, live_p[i], k))
            live_m.append(m.fork(live_m[i], k))
        elif op == "free":
            pkv.paged_kv_seq_free(p, live_p.pop(i))
            m.release(live_m.pop(i))
        _compare(p, m, live_p, live_m)
