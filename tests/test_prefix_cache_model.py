"""Fixed cases for the prefix-cache rules of the reference block-manager model
(oracle/block_manager.py), run against the model itself, so that the model is
pinned to the pages and not only to the library it is compared with.

The rules ("Trick 3, Prefix caching", How AI actually answers you; "Prefix
caching (automatic KV reuse)", vLLM Serving deep dive; the Automatic Prefix
Caching paragraph of The hands-on guide to LLM Inference with vLLM):
  * a page's fingerprint is built from its own tokens and the fingerprint of
    the page before it, so a hit means the whole text up to that page agrees;
  * only full pages get a fingerprint;
  * a new prompt reuses its leading cached pages; the token whose logits the
    next step needs (the prompt's last) is always computed;
  * unused cached pages are thrown out least recently used first.
Each case is built so that a plausible slip in the model (labelling a partial
block, a label of the block's own tokens only, reusing the last token's
block, evicting in another order, a hit that leaves its block in the queue)
changes the asserted numbers."""
import pytest

from oracle.block_manager import BlockManagerModel, StateError


def _model(n, caching=True):
    m = BlockManagerModel(n, 16)
    m.enable_caching(caching)
    return m


def _prefill(m, tokens):
    s, n = m.create_cached(tokens)
    m.append_tokens(s, tokens[n:])
    return s, n


def test_only_full_blocks_get_a_label():
    m = _model(32)
    a, n = _prefill(m, list(range(40)))  # blocks of 16, 16 and 8 tokens
    assert n == 0
    assert m.cache_stats()["cached_blocks"] == 2
    b, n = m.create_cached(list(range(40)) + [99] * 10)
    assert n == 32 and m.table(b) == m.table(a)[:2]
    assert [m.ref[x] for x in m.table(b)] == [2, 2]
    # the partial third block of a is not shared: b's third block is its own
    m.append_tokens(b, (list(range(40)) + [99] * 10)[32:])
    assert m.table(b)[2] != m.table(a)[2]


def test_a_label_chains_the_text_before_its_block():
    m = _model(32)
    _prefill(m, list(range(32)) + [7])
    # the same second block after a different first block: no hit at all
    assert m.create_cached([1000] * 16 + list(range(16, 32)) + [5])[1] == 0
    # the same first block, then a different second block: one block
    assert m.create_cached(list(range(16)) + [2000] * 16 + [5])[1] == 16
    # the same text: both blocks
    assert m.create_cached(list(range(32)) + [5])[1] == 32


def test_lookup_stops_at_the_first_miss():
    m = _model(32)
    _prefill(m, list(range(64)) + [1])
    toks = list(range(16)) + [500] * 16 + list(range(32, 64)) + [1]  # block 1 differs, 2 and 3 equal
    before = m.cache_stats()  # the counters are cumulative (the first prefill's lookup missed once)
    assert m.create_cached(toks)[1] == 16
    st = m.cache_stats()
    assert st["queried_blocks"] - before["queried_blocks"] == 2
    assert st["hit_blocks"] - before["hit_blocks"] == 1


def test_the_prompts_last_token_is_always_computed():
    m = _model(32)
    _prefill(m, list(range(48)))
    # 48 tokens = 3 full cached blocks, but the last token must be computed
    assert m.create_cached(list(range(48)))[1] == 32
    assert m.create_cached(list(range(49)))[1] == 48
    assert m.create_cached(list(range(16)))[1] == 0
    assert m.create_cached(list(range(17)))[1] == 16


def test_eviction_follows_the_release_order():
    m = BlockManagerModel(6, 16, initial_order=list(range(6)))
    m.enable_caching(True)
    ta, tb = list(range(33)), list(range(100, 133))
    a, _ = _prefill(m, ta)  # blocks 0, 1 labelled, 2 partial
    b, _ = _prefill(m, tb)  # blocks 3, 4 labelled, 5 partial
    m.release(b)  # b first: its blocks are the least recently released
    m.release(a)
    assert m.free_queue() == [3, 4, 5, 0, 1, 2]
    c = m.create()
    m.append(c, 40)  # takes 3, 4, 5 from the head: b's labels go
    assert m.table(c) == [3, 4, 5]
    assert m.create_cached(tb)[1] == 0
    assert m.create_cached(ta)[1] == 32


def test_a_hit_on_a_released_block_takes_it_out_of_the_queue():
    m = BlockManagerModel(8, 16, initial_order=list(range(8)))
    m.enable_caching(True)
    a, _ = _prefill(m, list(range(40)))
    m.release(a)
    assert m.num_free() == 8
    b, n = m.create_cached(list(range(40)))
    assert n == 32 and m.table(b) == [0, 1]
    assert not set(m.table(b)) & set(m.free_queue())
    assert m.num_free() == 6 and [m.ref[x] for x in (0, 1)] == [1, 1]


def test_caching_off_drops_every_label():
    m = _model(16)
    _prefill(m, list(range(40)))
    m.enable_caching(False)
    assert m.cache_stats()["cached_blocks"] == 0
    m.enable_caching(True)
    assert m.create_cached(list(range(40)))[1] == 0


def test_tokens_of_unknown_text_are_never_labelled():
    m = _model(16)
    s = m.create()
    m.append(s, 20)
    m.append_tokens(s, list(range(20, 40)))
    assert m.cache_stats()["cached_blocks"] == 0


def test_a_block_already_cached_is_not_labelled_twice():
    m = _model(16)
    a, _ = _prefill(m, list(range(17)))
    s = m.create()  # the same text computed again without a lookup
    m.append_tokens(s, list(range(17)))
    assert m.cache_stats()["cached_blocks"] == 1
    assert m.create_cached(list(range(17)))[1] == 16


def test_a_fork_continues_its_parents_labels():
    m = _model(16)
    a, _ = _prefill(m, list(range(20)))
    child = m.fork(a, 20)
    m.append_tokens(child, list(range(20, 32)))  # fills the copy of the shared partial block
    assert m.create_cached(list(range(40)))[1] == 32


def test_swapped_sequences_are_not_forked():
    m = _model(16)
    m.set_swap_space(4)
    a, _ = _prefill(m, list(range(20)))
    m.swap_out(a)
    with pytest.raises(StateError):
        m.fork(a, 4)
