"""GPU parity of the 8-bit (E4M3) KV cache.

* The quantising cache write (reshape_and_cache_fp8) against the oracle's
  quantiser, code for code, over values that cover the format: subnormal and
  normal magnitudes, exact ties, saturation, infinities, signed zeros, NaN.
* The plain copy of codes and the block copy on 8-bit pools, byte for byte.
* Decode attention over 8-bit pools (paged_attention_decode_fp8) against the
  fp64 oracle on the dequantised cache, on the decode shapes of the
  benchmark plan, partition edges, shared-prefix runs and the empty context,
  plus sampled sequences of the full Llama-3-8B-shaped workload.
The 8-bit cache itself is the "Quantization" option of the vLLM Serving deep
dive; the E4M3 format and the scale rule are the library's reading."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.conftest import gpu_available
from tests.helpers import (FP8_K_SCALE, FP8_V_SCALE, assert_close, decode_reference_fp8, tolerance)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _codes_values():
    v = oracle.decode("fp8_e4m3", np.arange(0x7f, dtype=np.uint8))
    return v, (v[:-1] + v[1:]) / 2


def _test_values(rng, shape, scale):
    """fp32 values in units of `scale` that exercise every rounding case."""
    n = int(np.prod(shape))
    vals, mids = _codes_values()
    x = np.exp2(rng.uniform(-12, 10.5, n)) * rng.choice([-1.0, 1.0], n)  # up to ~1400: saturation
    pick = rng.random(n)
    x = np.where(pick < 0.15, rng.choice(mids, n) * rng.choice([-1.0, 1.0], n), x)   # ties
    x = np.where((pick >= 0.15) & (pick < 0.25), rng.choice(vals, n) * rng.choice([-1.0, 1.0], n), x)
    x = (x * scale).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 448 * scale, 464 * scale, -470 * scale,
                         1e-30, -1e-30, 2.0 ** -10 * scale, 3 * 2.0 ** -10 * scale], np.float32)
    x[:specials.size] = specials
    return x.reshape(shape)


def _compare_codes(name, got, exp):
    nan = (exp & 0x7f) == 0x7f
    assert np.all((got[nan] & 0x7f) == 0x7f), f"{name}: NaN input lost"
    bad = (got != exp) & ~nan
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} codes differ; first at byte {i}: got {got[i]:#04x} "
                             f"want {exp[i]:#04x}")


@pytest.mark.parametrize("src", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [1.0, 0.37])
def test_quantising_write_matches_oracle_codes(src, d, scale):
    import paged_kv_cache_gather_amd as pkv
    print(f"fp8 write src={src} d={d} scale={scale}", flush=True)
    rng = np.random.default_rng(zlib.crc32(f"{src}/{d}/{scale}".encode()))
    nb, H, T = 24, 4, 300
    ks, vs = scale, scale * 1.5
    xk = _test_values(rng, (T, H * d), ks)
    xv = _test_values(rng, (T, H * d), vs)
    # the source dtype's own values (exact in fp32) are what both sides quantise
    k_src = torch.from_numpy(xk).to(TORCH[src])
    v_src = torch.from_numpy(xv).to(TORCH[src])
    # a token stride wider than the row, for one case
    pad = 16 if (src == "f16" and d == 128) else 0
    kbuf = torch.zeros((T, H * d + pad), dtype=TORCH[src])
    kbuf[:, :H * d] = k_src
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[rng.choice(T, 10, replace=False)] = -1
    kp = torch.zeros(nb * H * 16 * d, dtype=torch.uint8, device=DEV)
    vp = torch.zeros_like(kp)
    key_dev = kbuf.to(DEV)[:, :H * d] if pad else k_src.to(DEV)
    pkv.reshape_and_cache_fp8(key_dev, v_src.to(DEV), kp, vp, torch.from_numpy(slots).to(DEV), nb, H, d, ks, vs)
    torch.cuda.synchronize()
    ek = np.zeros(kp.numel(), np.uint8)
    ev = np.zeros_like(ek)
    ck = oracle.quantize_e4m3(k_src.float().numpy(), ks).reshape(T, H, d)
    cv = oracle.quantize_e4m3(v_src.float().numpy(), vs).reshape(T, H, d)
    oracle.scatter("fp8_e4m3", ck, cv, ek, ev, slots, nb, 16, H, d)
    _compare_codes("k_pool", kp.cpu().numpy(), ek)
    _compare_codes("v_pool", vp.cpu().numpy(), ev)


def test_plain_write_and_block_copy_of_codes():
    import paged_kv_cache_gather_amd as pkv
    rng = np.random.default_rng(5)
    nb, H, d, T = 16, 2, 128, 77
    ck = rng.integers(0, 256, size=(T, H, d), dtype=np.uint8)
    cv = rng.integers(0, 256, size=(T, H, d), dtype=np.uint8)
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    kp = torch.zeros(nb * H * 16 * d, dtype=torch.uint8, device=DEV)
    vp = torch.zeros_like(kp)
    pkv.reshape_and_cache(torch.from_numpy(ck.reshape(T, -1)).to(DEV), torch.from_numpy(cv.reshape(T, -1)).to(DEV),
                          kp, vp, torch.from_numpy(slots).to(DEV), nb, H, d)
    ek = np.zeros(kp.numel(), np.uint8)
    ev = np.zeros_like(ek)
    oracle.scatter("fp8_e4m3", ck, cv, ek, ev, slots, nb, 16, H, d)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), ek) and np.array_equal(vp.cpu().numpy(), ev)
    pairs = np.array([[3, 9], [0, 15], [7, 7], [40, 2]], np.int32)  # last pair outside the pool: skipped
    pkv.paged_kv_copy_blocks(kp, vp, torch.from_numpy(pairs).to(DEV), nb, H, d)
    oracle.copy_blocks("fp8_e4m3", ek, ev, pairs[:3], nb, 16, H, d)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), ek) and np.array_equal(vp.cpu().numpy(), ev)


def _run_decode_fp8(w, out_dtype, fill="host"):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    b = DeviceBatch(w, DEV, fill=fill, out_dtype=out_dtype, kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE,
                    v_scale=FP8_V_SCALE)
    b.append_decode()
    out = b.new_decode_out()
    b.attend_decode(out)
    torch.cuda.synchronize()
    return b, out


def _check(w, out, out_dtype, seqs=None):
    atol, rtol = tolerance(w.dtype, out_dtype)
    got = out.double().cpu().numpy()
    for s in (range(w.n_decode) if seqs is None else seqs):
        assert_close(f"{w.name} fp8 seq {s} L={int(w.decode_lens[s])}", got[s], decode_reference_fp8(w, s),
                     atol, rtol)


FP8_DECODE = [
    # name, Hq, Hkv, d, q dtype, lens
    ("llama3_edges", 32, 8, 128, "bf16", [1, 15, 16, 17, 511, 512, 513, 1029, 2048, 3001]),
    ("tinyllama_small", 32, 4, 64, "f16", [128, 700, 1500, 2048, 129, 513]),
    ("opt13b_small", 40, 40, 128, "f16", [2048, 1, 31, 600]),
    ("gqa2_small", 8, 4, 128, "bf16", [3, 16, 17, 511, 512, 1537]),
    ("gqa8_d64", 32, 4, 64, "bf16", [100, 900, 1024]),
    ("gqa16_d64", 32, 2, 64, "bf16", [100, 900]),
    ("gqa16_d128", 16, 1, 128, "f16", [1000, 513, 64]),
    ("long_contexts", 32, 8, 128, "bf16", [4609, 8192, 9001]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,lens", FP8_DECODE, ids=[c[0] for c in FP8_DECODE])
@pytest.mark.parametrize("out_kind", ["f32", "q"])
def test_decode_fp8_small(name, Hq, Hkv, d, dtype, lens, out_kind):
    out_dtype = "f32" if out_kind == "f32" else dtype
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 2048, seed=21, decode_lens=lens)
    print(f"fp8 decode {name} out={out_dtype}", flush=True)
    _, out = _run_decode_fp8(w, out_dtype)
    _check(w, out, out_dtype)


WHOLE_LENS = [1, 15, 16, 17, 100, 511, 512, 513, 1024, 1500, 2047, 2048, 3071, 4096]
FP8_WHOLE = [
    # name, Hq, Hkv, d, q dtype
    ("whole_tinyllama_f16", 32, 4, 64, "f16"),
    ("whole_gqa4_d128_bf16", 32, 8, 128, "bf16"),
    ("whole_gqa16_d128_f16", 32, 2, 128, "f16"),
    ("whole_mha_d64_bf16", 8, 8, 64, "bf16"),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype", FP8_WHOLE, ids=[c[0] for c in FP8_WHOLE])
def test_decode_fp8_whole_context(name, Hq, Hkv, d, dtype):
    # short contexts, 128 (sequence, KV head) pairs: the whole-context launch,
    # against the dequantised oracle and against the split path; the one-call
    # step (quantising write inside the launch) bit for bit against the write
    # followed by the attention
    import paged_kv_cache_gather_amd as pkv
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    n = -(-128 // Hkv)
    lens = [WHOLE_LENS[i % len(WHOLE_LENS)] for i in range(max(n, len(WHOLE_LENS)))]
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 8192, seed=27, decode_lens=lens)
    kw = dict(fill="host", out_dtype="f32", kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    sep, one = DeviceBatch(w, DEV, **kw), DeviceBatch(w, DEV, **kw)
    assert pkv.paged_attention_decode_whole_context(w.n_decode, Hq, Hkv, d, "fp8_e4m3", sep.decode.max_context_len)
    print(f"fp8 whole context {name}", flush=True)
    out_sep, out_one, out_split = sep.new_decode_out(), one.new_decode_out(), sep.new_decode_out()
    sep.append_decode()
    sep.attend_decode(out_sep)
    sep.attend_decode_split(out_split)
    one.step_decode(out_one)
    torch.cuda.synchronize()
    assert torch.equal(out_sep.view(torch.int32), out_one.view(torch.int32))
    assert torch.equal(sep.k_pool.view(torch.uint8), one.k_pool.view(torch.uint8))
    assert torch.equal(sep.v_pool.view(torch.uint8), one.v_pool.view(torch.uint8))
    _check(w, out_one, "f32")
    atol, rtol = tolerance(dtype, "f32")
    got, split = out_one.double().cpu().numpy(), out_split.double().cpu().numpy()
    for s in range(w.n_decode):
        assert_close(f"{name} whole vs split seq {s}", got[s], split[s], 2 * atol, 2 * rtol)


FP8_FUSED = [
    # name, Hq, Hkv, d, q dtype, lens, prefix_len, prefix_group
    ("fused8_shared_cow", 32, 8, 128, "bf16", [1100, 1100, 1500, 1030, 600, 17, 1, 2049],
     [1030, 1030, 1030, 1029, 0, 0, 0, 0], [0, 0, 0, 0, -1, -1, -1, -1]),
    ("fused8_f16_d64", 32, 4, 64, "f16", [700, 700, 129, 513], [600, 600, 0, 0], [0, 0, -1, -1]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,lens,plen,pgroup", FP8_FUSED, ids=[c[0] for c in FP8_FUSED])
def test_decode_fp8_append_in_one_call(name, Hq, Hkv, d, dtype, lens, plen, pgroup):
    # paged_attention_decode_fp8_append = reshape_and_cache_fp8 +
    # paged_attention_decode_fp8, bit for bit (output and pools)
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 1024, seed=25, decode_lens=lens, prefix_len=plen,
                              prefix_group=pgroup)
    print(f"fp8 decode_append {name}", flush=True)
    kw = dict(fill="host", out_dtype="f32", kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    sep, one = DeviceBatch(w, DEV, **kw), DeviceBatch(w, DEV, **kw)
    out_sep, out_one = sep.new_decode_out(), one.new_decode_out()
    sep.append_decode()
    sep.attend_decode(out_sep)
    one.step_decode(out_one)
    torch.cuda.synchronize()
    assert torch.equal(out_sep.view(torch.int32), out_one.view(torch.int32))
    assert torch.equal(sep.k_pool.view(torch.uint8), one.k_pool.view(torch.uint8))
    assert torch.equal(sep.v_pool.view(torch.uint8), one.v_pool.view(torch.uint8))
    _check(w, out_one, "f32")


FP8_RUNS = [
    # name, Hq, Hkv, d, dtype, lens, prefix_len, prefix_group
    ("runs_gqa4", 32, 8, 128, "bf16",
     [1500, 1200, 2000, 1101, 1102, 700, 900, 800, 512, 513, 1024, 1024],
     [1100, 1100, 1100, 1100, 1100, 600, 600, 0, 511, 512, 1023, 1023],
     [0, 0, 0, 0, 0, 1, 1, -1, 2, 2, 3, 3]),
    ("runs_cross_window", 32, 8, 128, "bf16", [600] * 5 + [1100, 1500, 1030, 2049, 1100, 1200] + [700],
     [0] * 5 + [1029] * 6 + [0], [-1] * 5 + [0] * 6 + [-1]),
    ("runs_f16_d64", 16, 4, 64, "f16", [1030, 1030, 1536, 3000, 520], [1025, 1025, 1025, 1025, 0],
     [0, 0, 0, 0, -1]),
    ("runs_mha", 8, 8, 128, "f16", [1300, 1300, 1030, 600], [1200, 1200, 1029, 0], [0, 0, 0, -1]),
]


@pytest.mark.parametrize("name,Hq,Hkv,d,dtype,lens,plen,pgroup", FP8_RUNS, ids=[c[0] for c in FP8_RUNS])
def test_decode_fp8_shared_partition_runs(name, Hq, Hkv, d, dtype, lens, plen, pgroup):
    w = synth.custom_workload(name, Hq, Hkv, d, dtype, 4096, seed=13, decode_lens=lens, prefix_len=plen,
                              prefix_group=pgroup)
    print(f"fp8 decode {name}", flush=True)
    _, out = _run_decode_fp8(w, "f32")
    _check(w, out, "f32")


def test_decode_fp8_full_size_sampled():
    # the Llama-3-8B-shaped workload (256 sequences, groups of 8 sharing a
    # 1024-token prefix) in the launch shape the benchmark times, bf16 out
    w = synth.make_workload("llama3_8b_decode", seed=0)
    print("fp8 decode full llama3_8b_decode", flush=True)
    b, out = _run_decode_fp8(w, "bf16", fill="device")
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(3)
    sample = sorted(set(rng.choice(w.n_decode, size=5, replace=False).tolist()
                        + [0, 7, 8, int(np.argmax(w.decode_lens)), int(np.argmin(w.decode_lens))]))
    _check(w, out, "bf16", sample)


def test_decode_fp8_empty_context_gives_zeros_and_bad_scales_are_rejected():
    import paged_kv_cache_gather_amd as pkv
    B, Hq, Hkv, d, nb = 2, 8, 2, 64, 8
    kp = torch.zeros(nb * Hkv * 16 * d, dtype=torch.uint8, device=DEV)
    vp = torch.zeros_like(kp)
    q = torch.randn(B, Hq, d, device=DEV).half()
    out = torch.full((B, Hq, d), 7.0, device=DEV)
    tables = torch.zeros(B, 4, dtype=torch.int32, device=DEV)
    lens = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    ws = torch.empty(pkv.paged_attention_decode_workspace_bytes(B, Hq, d, 64) // 4 + 1, device=DEV)
    pkv.paged_attention_decode_fp8(out, q, kp, vp, tables, lens, 64, Hkv, nb, 0.125, 0.5, 0.5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan"))):
        with pytest.raises(pkv.PagedKVError):
            pkv.paged_attention_decode_fp8(out, q, kp, vp, tables, lens, 64, Hkv, nb, 0.125, ks, vs, workspace=ws)
