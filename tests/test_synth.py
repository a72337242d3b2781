"""The seeded input generator: determinism, distribution, dtype rounding
against library conversions, and the workload recipes.  CPU only."""
import numpy as np
import pytest
import torch

import synth


def test_lowbias32_known_values():
    # lowbias32 is a bijection on 32-bit words with lowbias32(0) == 0
    assert synth.lowbias32(0) == 0
    x = np.arange(1 << 16, dtype=np.uint32)
    assert np.unique(synth.lowbias32(x)).size == x.size


def test_values_deterministic_and_regenerable():
    a = synth.values(0, synth.KIND_K, 5, 0, 40, 4, 16, "bf16")
    b = synth.values(0, synth.KIND_K, 5, 0, 40, 4, 16, "bf16")
    assert np.array_equal(a, b)
    # any sub-range regenerates the same elements
    c = synth.values(0, synth.KIND_K, 5, 17, 23, 4, 16, "bf16")
    assert np.array_equal(a[17:23], c)
    # different stream -> different values
    assert not np.array_equal(a, synth.values(0, synth.KIND_V, 5, 0, 40, 4, 16, "bf16"))
    assert not np.array_equal(a, synth.values(1, synth.KIND_K, 5, 0, 40, 4, 16, "bf16"))


def test_normal_table_moments():
    x = synth.normal_table("f32").view(np.float32).astype(np.float64)
    assert abs(x.mean()) < 1e-6
    assert abs(x.std() - 1.0) < 2e-3
    assert np.array_equal(x, -x[::-1])


def test_bf16_table_is_round_to_nearest_even():
    x32 = synth.normal_table("f32").view(np.float32)
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.normal_table("bf16"), ref)


def test_f16_table_matches_numpy():
    x32 = synth.normal_table("f32").view(np.float32)
    assert np.array_equal(synth.normal_table("f16"), x32.astype(np.float16).view(np.uint16))


def test_value_distribution():
    v = synth.values(3, synth.KIND_Q, 0, 0, 4096, 8, 64, "f32").view(np.float32).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


@pytest.mark.parametrize("name", synth.WORKLOADS)
def test_workload_recipes(name):
    w = synth.make_workload(name, seed=0)
    assert sorted(w.free_order.tolist()) == list(range(w.num_blocks))
    if name == "toy_f32_decode":
        assert w.decode_lens.tolist() == [4, 7, 2] and w.dtype == "f32" and w.num_blocks == 8
    if name == "tinyllama_decode":
        assert w.n_decode == 64 and w.decode_lens.min() >= 128 and w.decode_lens.max() <= 2048
    if name == "llama3_8b_decode":
        assert w.n_decode == 256 and w.decode_lens.min() >= 512 and w.decode_lens.max() <= 4096
        assert np.array_equal(w.prefix_group, np.arange(256) // 8)
        assert np.array_equal(w.prefix_len, np.minimum(w.decode_lens - 1, 1024))
    if name == "opt13b_decode":
        assert np.all(w.decode_lens == 2048) and w.n_q_heads == w.n_kv_heads == 40
    if name == "llama3_8b_mixed":
        assert w.n_chunks == 16 and np.all(w.chunk_qlen == 512)
        assert w.chunk_ctx.max() + 512 <= 8192
        assert w.n_decode == 240 and w.decode_lens.min() >= 256 and w.decode_lens.max() <= 8192
        assert int(w.decode_lens.sum() + w.chunk_qlen.sum()) > 0
    # same seed, same workload
    w2 = synth.make_workload(name, seed=0)
    assert np.array_equal(w.decode_lens, w2.decode_lens) and np.array_equal(w.free_order, w2.free_order)


def test_shared_prefix_tokens_come_from_group_stream():
    w = synth.make_workload("llama3_8b_decode", seed=0)
    a, _ = w.kv("decode", 0, 0, 64)
    b, _ = w.kv("decode", 1, 0, 64)
    assert np.array_equal(a, b)  # same group, inside the prefix
    s = 9  # group 1
    pl = int(w.prefix_len[s])
    x, _ = w.kv("decode", s, pl - 2, pl + 2)
    y, _ = w.kv("decode", 8, pl - 2, pl)
    assert np.array_equal(x[:2], y)
