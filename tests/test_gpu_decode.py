"""GPU parity of paged decode attention (append + partition pass + split-K
reduce) against the fp64 oracle, on the five workload shapes at sizes the
oracle finishes quickly, on sampled sequences of the full-size workloads, and
on the edge cases: one key, partition boundaries, empty context, placement
invariance and run-to-run determinism."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, decode_reference, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _run_decode(w, out_dtype=None, fill="host"):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(w, DEV, fill=fill, out_dtype=out_dtype)
    b.append_decode()
    out = b.new_decode_out()
    b.attend_decode(out)
    torch.cuda.synchronize()
    return b, out


def _check_both_paths(w, b, out, out_dtype):
    """out (the one-call attention, whichever path the batch's sizes pick)
    and the two-call form (always split-context, shared runs included) on
    the same batch, both against the oracle."""
    split = b.new_decode_out()
    b.attend_decode_split(split)
    torch.cuda.synchronize()
    _check_all(w, out, out_dtype)
    _check_all(w, split, out_dtype)


def _check_all(w, out, out_dtype, seqs=None):
    atol, rtol = tolerance(w.dtype, out_dtype)
    got = out.double().cpu().numpy()
    for s in (range(w.n_decode) if seqs is None else seqs):
        assert_close(f"{w.name} seq {s} L={int(w.decode_lens[s])}", got[s], decode_reference(w, s), atol, rtol)


def test_config1_toy_f32():
    w = synth.make_workload("toy_f32_decode", seed=0)
    print(f"decode {w.name}", flush=True)
    _, out = _run_decode(w)
    _check_all(w, out, "f32")


SMALL = [
    # name, Hq, Hkv, d, dtype, lens
    ("tinyllama_small", 32, 4, 64, "f16", [128, 700, 1500, 2048, 129, 513]),
    ("llama3_small", 32, 8, 128, "bf16", [512, 1024, 1025, 4096, 2000, 777]),
    ("opt13b_small", 40, 40, 128, "f16", [2048, 2048, 1, 31]),
    ("gqa2_small", 8, 4, 128, "bf16", [3, 16, 17, 511, 512, 1537]),
    ("gqa16_small", 32, 2, 64, "bf16", [100, 900]),
    ("gqa8_d128_edges", 64, 8, 128, "bf16", [3, 16, 17, 511, 512, 513, 1537, 3000]),
    ("gqa16_d128_f16", 32, 2, 128, "f16", [1, 100, 511, 512, 513, 2049]),
    ("f32_d128", 8, 2, 128, "f32", [5, 600]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,lens", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("out_kind", ["f32", "kv"])
def test_decode_small(name, Hq, Hkv, d, dtype, lens, out_kind):
    out_dtype = "f32" if out_kind == "f32" else dtype
    if dtype == "f32" and out_kind == "kv":
        pytest.skip("same as f32")
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 2048, seed=3, decode_lens=lens)
    print(f"decode {name} out={out_dtype}", flush=True)
    b, out = _run_decode(w, out_dtype)
    _check_both_paths(w, b, out, out_dtype)


def test_decode_long_contexts():
    # 9 to 33 partitions of 512 tokens: the split-context merge takes its
    # partials in batches of 8, so counts on both sides of 8, 16 and 32
    lens = [4097, 4608, 8192, 8193, 12000, 16500]
    w = synth.custom_workload("llama3_long", 32, 8, 128, "bf16", 4096, seed=6, decode_lens=lens)
    for out_dtype in ("f32", "bf16"):
        print(f"decode llama3_long out={out_dtype}", flush=True)
        _, out = _run_decode(w, out_dtype, fill="device")
        _check_all(w, out, out_dtype)
    w = synth.custom_workload("long_shared", 32, 8, 128, "bf16", 4096, seed=7, decode_lens=[9000, 9000, 5000],
                              prefix_len=[8800, 8800, 0], prefix_group=[0, 0, -1])
    print("decode long_shared", flush=True)
    _, out = _run_decode(w, "f32", fill="device")
    _check_all(w, out, "f32")
    # G = 1: a run window of 32 sequences probes 16 partitions per round, so
    # 18 shared partitions take two rounds
    w = synth.custom_workload("long_shared_mha", 4, 4, 64, "f16", 4096, seed=8, decode_lens=[9000, 5000, 9000, 8801],
                              prefix_len=[8800, 0, 8800, 8800], prefix_group=[0, -1, 0, 0])
    print("decode long_shared_mha", flush=True)
    _, out = _run_decode(w, "f32", fill="device")
    _check_all(w, out, "f32")


def test_decode_shared_prefix_with_copy_on_write():
    # groups of 4 sharing prefixes whose last block is partly filled, so the
    # first private append of each member copies that block
    lens = [40, 41, 700, 1030, 35, 100, 513, 1100]
    plen = [33, 33, 33, 33, 20, 20, 20, 20]
    w = synth.custom_workload("prefix_cow", 32, 8, 128, "bf16", 1024, seed=5, decode_lens=lens,
                              prefix_len=plen, prefix_group=[0, 0, 0, 0, 1, 1, 1, 1])
    print("decode prefix_cow", flush=True)
    b, out = _run_decode(w, "f32")
    _check_both_paths(w, b, out, "f32")


SHARED_RUNS = [
    # name, Hq, Hkv, d, dtype, lens, prefix_len, prefix_group
    ("runs_gqa4", 32, 8, 128, "bf16",
     [1500, 1200, 2000, 1101, 1102, 700, 900, 800, 512, 513, 1024, 1024],
     [1100, 1100, 1100, 1100, 1100, 600, 600, 0, 511, 512, 1023, 1023],
     [0, 0, 0, 0, 0, 1, 1, -1, 2, 2, 3, 3]),
    ("runs_mha", 8, 8, 128, "f16", [1300, 1300, 1030, 600], [1200, 1200, 1029, 0], [0, 0, 0, -1]),
    ("runs_gqa8", 32, 4, 64, "f16", [1100, 1100, 1100], [1024, 1024, 1024], [0, 0, 0]),
    ("runs_gqa2", 8, 4, 128, "bf16", [2100] * 9, [2048] * 9, [0] * 9),
    # a group of six over sequences 5..10 straddles the 8-sequence window of
    # G = 4 (two runs of three); its shared prefix ends inside a block
    ("runs_cross_window", 32, 8, 128, "bf16", [600] * 5 + [1100, 1500, 1030, 2049, 1100, 1200] + [700],
     [0] * 5 + [1029] * 6 + [0], [-1] * 5 + [0] * 6 + [-1]),
    ("runs_f16_d64", 16, 4, 64, "f16", [1030, 1030, 1536, 3000, 520], [1025, 1025, 1025, 1025, 0],
     [0, 0, 0, 0, -1]),
    # groups interleaved inside the window (runs are sets of members, not
    # ranges); group 2's 600-token prefix shares the first block of the second
    # partition but not the rest, so its members agree on the first id only
    ("runs_interleaved", 32, 8, 128, "bf16",
     [1500, 1700, 1101, 2100, 900, 1200, 1601, 800, 1300, 1650, 700, 1000, 600, 2000, 1150, 610],
     [1100, 1600, 1100, 1600, 600, 1100, 1600, 0, 1100, 1600, 600, 600, 0, 1600, 1100, 600],
     [0, 1, 0, 1, 2, 0, 1, -1, 0, 1, 2, 2, -1, 1, 0, 2]),
    ("runs_interleaved_gqa8", 32, 4, 64, "f16",
     [1100, 700, 1500, 800, 900, 1031, 650, 2000, 1200, 1040, 620, 300],
     [1030, 600, 1030, 600, 600, 1030, 600, 1030, 1030, 1030, 600, 0],
     [0, 1, 0, 1, 1, 0, 1, 0, 0, 0, 1, -1]),
    # one run window of 32 sequences at G = 1, three groups dealt round robin
    ("runs_interleaved_mha", 4, 4, 64, "f16",
     [1200 + 13 * i if i % 3 == 0 else (700 + 7 * i if i % 3 == 1 else 530 + i) for i in range(30)] + [90, 1700, 40, 600],
     [1100 if i % 3 == 0 else (600 if i % 3 == 1 else 520) for i in range(30)] + [0, 0, 0, 0],
     [i % 3 for i in range(30)] + [-1, -1, -1, -1]),
    # the class leader (lowest member with the partition's first block id)
    # took a shorter prefix: members 1-4 agree with each other on every id of
    # the second partition but not with it, so they stay per-sequence there
    ("runs_leader_differs", 32, 8, 128, "bf16", [1500, 1300, 1400, 1200, 1100, 700],
     [600, 1100, 1100, 1100, 1050, 0], [0, 0, 0, 0, 0, -1]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,lens,plen,pgroup", SHARED_RUNS, ids=[c[0] for c in SHARED_RUNS])
def test_decode_shared_partition_runs(name, Hq, Hkv, d, dtype, lens, plen, pgroup):
    # sequences of one 32 / G-sequence window whose full 512-token partitions
    # use the same blocks are served by one MFMA workgroup; groups cross the
    # window, interleave inside it, some members end exactly at a partition
    # edge
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 4096, seed=13, decode_lens=lens, prefix_len=plen,
                              prefix_group=pgroup)
    print(f"decode {name}", flush=True)
    b, out = _run_decode(w, "f32")
    _check_both_paths(w, b, out, "f32")


@pytest.mark.parametrize("name", ["tinyllama_decode", "llama3_8b_decode", "opt13b_decode"])
def test_decode_full_size_sampled(name):
    w = synth.make_workload(name, seed=0)
    print(f"decode full {w.name}", flush=True)
    b, out = _run_decode(w, None, fill="device")
    got = out.float()
    assert torch.isfinite(got).all()
    rng = np.random.default_rng(synth.WORKLOADS.index(name) + 1)
    sample = sorted(set(rng.choice(w.n_decode, size=6, replace=False).tolist()
                        + [int(np.argmax(w.decode_lens)), int(np.argmin(w.decode_lens))]))
    _check_all(w, out, w.dtype, sample)


FUSED = [
    # name, Hq, Hkv, d, dtype, lens, prefix_len, prefix_group
    ("fused_shared_cow", 32, 8, 128, "bf16", [1100, 1100, 1500, 1030, 600, 17, 1, 2049, 513],
     [1030, 1030, 1030, 1029, 0, 0, 0, 0, 0], [0, 0, 0, 0, -1, -1, -1, -1, -1]),
    ("fused_f16_d64", 32, 4, 64, "f16", [700, 700, 129, 2048], [600, 600, 0, 0], [0, 0, -1, -1]),
    ("fused_f32", 8, 2, 64, "f32", [5, 600, 1], [0, 0, 0], [-1, -1, -1]),
    # MHA (32-sequence run windows) and G = 16 (2-sequence windows)
    ("fused_mha", 8, 8, 128, "f16", [1700, 1700, 600, 1030], [1200, 1200, 0, 1029], [0, 0, -1, 0]),
    ("fused_gqa16", 32, 2, 64, "bf16", [900, 900, 100, 513, 513], [600, 600, 0, 512, 512], [0, 0, -1, 1, 1]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,lens,plen,pgroup", FUSED, ids=[c[0] for c in FUSED])
def test_decode_append_in_one_call(name, Hq, Hkv, d, dtype, lens, plen, pgroup):
    # paged_attention_decode_append = reshape_and_cache + paged_attention_decode,
    # bit for bit (output and pools), and within tolerance of the oracle
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 1024, seed=23, decode_lens=lens, prefix_len=plen,
                              prefix_group=pgroup)
    print(f"decode_append {name}", flush=True)
    sep = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    one = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    out_sep, out_one = sep.new_decode_out(), one.new_decode_out()
    sep.append_decode()
    sep.attend_decode(out_sep)
    one.step_decode(out_one)
    torch.cuda.synchronize()
    assert torch.equal(out_sep.view(torch.int32), out_one.view(torch.int32))
    assert torch.equal(sep.k_pool.view(torch.uint8), one.k_pool.view(torch.uint8))
    assert torch.equal(sep.v_pool.view(torch.uint8), one.v_pool.view(torch.uint8))
    _check_all(w, out_one, "f32")


@pytest.mark.parametrize("lens", [[300, 40, 900], [300, 40, 2100]], ids=["whole_context", "split"])
def test_decode_append_skips_padding_slots(lens):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload("fused_pad", 32, 8, 128, "bf16", 512, seed=24, decode_lens=lens)
    sep = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    one = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    for b in (sep, one):
        b.decode.slots[1] = -1  # this row is not written
    out_sep, out_one = sep.new_decode_out(), one.new_decode_out()
    sep.append_decode()
    sep.attend_decode(out_sep)
    one.step_decode(out_one)
    torch.cuda.synchronize()
    assert torch.equal(out_sep.view(torch.int32), out_one.view(torch.int32))
    assert torch.equal(sep.k_pool.view(torch.uint8), one.k_pool.view(torch.uint8))
    assert torch.equal(sep.v_pool.view(torch.uint8), one.v_pool.view(torch.uint8))


def test_decode_large_batch_sampled():
    # 3000 short sequences: 375 run windows, groups of 8 and 5 sharing
    # prefixes, lengths from 1 to 1100 (most single-partition)
    n = 3000
    rng = np.random.default_rng(17)
    lens = rng.integers(1, 1101, size=n)
    group = np.where(np.arange(n) % 16 < 13, (np.arange(n) // 8) % 40, -1)
    plen = np.where(group >= 0, np.minimum(lens - 1, 520), 0)
    w = synth.custom_workload("large_batch", 32, 8, 128, "bf16", 70000, seed=18, decode_lens=lens,
                              prefix_len=plen, prefix_group=group)
    print("decode large_batch", flush=True)
    b, out = _run_decode(w, "f32", fill="device")
    assert torch.isfinite(out.float()).all()
    sample = sorted(set(rng.choice(n, size=40, replace=False).tolist() + [0, 7, 8, n - 1, int(np.argmax(lens))]))
    _check_all(w, out, "f32", sample)


def test_config3_step_sampled_with_bf16_out():
    # the workload the benchmark times: the Llama-3-8B decode batch, bf16 out, same launch shape
    w = synth.make_workload("llama3_8b_decode", seed=0)
    b, out = _run_decode(w, "bf16", fill="device")
    _check_all(w, out, "bf16", [0, 7, 8, 100, 255])


def test_single_key_returns_its_value_exactly():
    # both paths: this small batch takes the whole-context launch in one
    # call; the two-call form always splits
    w = synth.custom_workload("one_key", 32, 8, 128, "bf16", 64, seed=9, decode_lens=[1, 1, 1])
    b, out = _run_decode(w, "f32")
    split = b.new_decode_out()
    b.attend_decode_split(split)
    torch.cuda.synchronize()
    import oracle
    for o in (out, split):
        got = o.cpu().numpy()
        for s in range(3):
            _, v = w.kv("decode", s, 0, 1)
            ref = np.repeat(oracle.decode("bf16", v)[0], 4, axis=0)
            assert np.array_equal(got[s].astype(np.float64), ref)


def test_empty_context_gives_zeros():
    import paged_kv_cache_gather_amd as pkv
    B, Hq, Hkv, d, nb = 2, 8, 2, 64, 8
    kp = torch.zeros(nb * Hkv * 16 * d, dtype=torch.float16, device=DEV)
    vp = torch.zeros_like(kp)
    q = torch.randn(B, Hq, d, device=DEV).half()
    out = torch.full((B, Hq, d), 7.0, device=DEV)
    tables = torch.zeros(B, 4, dtype=torch.int32, device=DEV)
    lens = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    ws = torch.empty(pkv.paged_attention_decode_workspace_bytes(B, Hq, d, 64) // 4 + 1, device=DEV)
    pkv.paged_attention_decode(out, q, kp, vp, tables, lens, 64, Hkv, nb, 0.125, workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    out.fill_(7.0)  # the split path (two calls)
    pkv.paged_attention_decode_partitions(out, q, kp, vp, tables, lens, 64, Hkv, nb, 0.125, workspace=ws)
    pkv.paged_attention_decode_reduce(out, q, kp, vp, tables, lens, 64, Hkv, nb, 0.125, workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_placement_invariance_and_determinism():
    # same logical K/V under two different free-queue orders: bit-identical outputs
    lens = [900, 1500, 33, 2048]
    outs = []
    for seed in (11, 12):
        w = synth.custom_workload("placement", 32, 8, 128, "bf16", 1024, seed=4, decode_lens=lens)
        w.free_order = np.random.default_rng(seed).permutation(1024).astype(np.int32)
        b, out = _run_decode(w, "f32")
        assert not np.array_equal(b.decode.tables_host, outs[0][0]) if outs else True
        outs.append((b.decode.tables_host, out.cpu().numpy()))
        out2 = b.new_decode_out()
        b.attend_decode(out2)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())
    assert np.array_equal(outs[0][1], outs[1][1])


def test_long_context_two_level_scores_closed_form():
    # 16500 bf16 tokens (33 partitions) through a shuffled block table; keys
    # +u_g for the first 6100 tokens and -u_g after, so every score is +-a_h and
    # the output is a closed form of two plain sums, computed here without the
    # oracle: out = (e^a S_A + e^-a S_B) / (n_A e^a + n_B e^-a)  (a = 0: mean of V)
    import math
    import paged_kv_cache_gather_amd as pkv
    rng = np.random.default_rng(31)
    L, Hkv, G, d, bs, n_a = 16500, 2, 4, 128, 16, 6100
    Hq, scale, dt = Hkv * G, 1.0 / math.sqrt(128), torch.bfloat16
    u = torch.from_numpy(rng.standard_normal((Hkv, d)).astype(np.float32)).to(dt)
    k_rows = torch.empty((L, Hkv, d), dtype=dt)
    k_rows[:n_a] = u
    k_rows[n_a:] = -u
    v_rows = torch.from_numpy(rng.standard_normal((L, Hkv, d)).astype(np.float32)).to(dt)
    nblk = -(-L // bs)
    nb = nblk + 9
    table = rng.permutation(nb)[:nblk].astype(np.int32)
    t = np.arange(L)
    slots = torch.from_numpy((table[t // bs].astype(np.int64) * bs + t % bs)).to(DEV)
    k_pool = torch.zeros(nb * Hkv * bs * d, dtype=dt, device=DEV)
    v_pool = torch.zeros_like(k_pool)
    print("decode closed form, 16500 tokens", flush=True)
    pkv.reshape_and_cache(k_rows.reshape(L, Hkv * d).to(DEV), v_rows.reshape(L, Hkv * d).to(DEV), k_pool, v_pool,
                          slots, nb, Hkv, d)
    c = [0.0, 3.0, 12.0, -16.0] * Hkv
    u64 = u.double().numpy()
    q = torch.stack([torch.from_numpy(c[h] * u64[h // G] / np.dot(u64[h // G], u64[h // G])) for h in range(Hq)])
    q = q.to(dt)
    out = torch.empty((1, Hq, d), dtype=torch.float32, device=DEV)
    ws = torch.empty(pkv.paged_attention_decode_workspace_bytes(1, Hq, d, L) // 4 + 1, dtype=torch.float32,
                     device=DEV)
    pkv.paged_attention_decode(out, q[None].to(DEV), k_pool, v_pool, torch.from_numpy(table[None]).to(DEV),
                               torch.tensor([L], dtype=torch.int32, device=DEV), L, Hkv, nb, scale, ws)
    torch.cuda.synchronize()
    got = out[0].double().cpu().numpy()
    vv = v_rows.double().numpy()
    q64 = q.double().numpy()
    atol, rtol = tolerance("bf16", "f32")
    for h in range(Hq):
        g = h // G
        a = scale * float(np.dot(q64[h], u64[g]))
        sa, sb = vv[:n_a, g].sum(axis=0), vv[n_a:, g].sum(axis=0)
        exp = (math.exp(a) * sa + math.exp(-a) * sb) / (n_a * math.exp(a) + (L - n_a) * math.exp(-a))
        assert_close(f"closed form head {h} (a = {a:.3f})", got[h], exp, atol, rtol)
