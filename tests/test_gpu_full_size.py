"""GPU parity at full size: every output of the launches the benchmark times
against the fp64 oracle, on the workloads at their stated sizes.

* the one-call decode step (paged_attention_decode_append) of the
  TinyLlama-, Llama-3-8B- and OPT-13B-shaped batches, every sequence, output
  in the KV dtype (the benchmark's launch);
* the mixed chunked-prefill + decode step (16 chunks of 512 queries over
  contexts up to 7680, 240 decodes up to 8192 keys): all 240 decodes and all
  8192 prefill rows;
* the 8-bit step over the Llama-3-8B-shaped batch, every sequence;
* verify attention of 5 new tokens for each of 256 sequences, every row.

Each sequence's inputs are regenerated on the host from the seeded
generator; nothing on the oracle side reads the device pools."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.helpers import (FP8_K_SCALE, FP8_V_SCALE, assert_close, decode_references, prefill_references,
                           tolerance)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _check_decode(w, out, out_dtype, refs, name):
    atol, rtol = tolerance(w.dtype, out_dtype)
    got = out.double().cpu().numpy()
    for s, ref in refs.items():
        assert_close(f"{name} seq {s} L={int(w.decode_lens[s])}", got[s], ref, atol, rtol)


@pytest.mark.parametrize("name", ["tinyllama_decode", "llama3_8b_decode", "opt13b_decode"])
def test_decode_step_every_sequence(name):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.make_workload(name, seed=0)
    print(f"full-size decode step {w.name}: {w.n_decode} sequences", flush=True)
    b = DeviceBatch(w, DEV, fill="device")
    out = b.new_decode_out()
    b.step_decode(out)
    torch.cuda.synchronize()
    refs = decode_references(w, range(w.n_decode))
    _check_decode(w, out, w.dtype, refs, w.name)


def test_decode_fp8_step_every_sequence():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.make_workload("llama3_8b_decode", seed=0)
    print(f"full-size 8-bit decode step {w.name}", flush=True)
    b = DeviceBatch(w, DEV, fill="device", kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    out = b.new_decode_out()
    b.step_decode(out)
    torch.cuda.synchronize()
    refs = decode_references(w, range(w.n_decode), fp8=True)
    _check_decode(w, out, w.dtype, refs, w.name + " fp8")


@pytest.fixture(scope="module")
def mixed():
    """The mixed step as the benchmark runs it: both appends, then prefill
    attention and decode attention (partition pass, then merge)."""
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.make_workload("llama3_8b_mixed", seed=0)
    print(f"full-size mixed step {w.name}", flush=True)
    b = DeviceBatch(w, DEV, fill="device")
    outp, outd = b.new_prefill_out(), b.new_decode_out()
    b.append_prefill()
    b.append_decode()
    b.attend_prefill(outp)
    b.attend_decode_split(outd)
    torch.cuda.synchronize()
    res = (w, outp.double().cpu().numpy(), outd)
    del b
    torch.cuda.empty_cache()
    return res


def test_mixed_step_every_decode(mixed):
    w, _, outd = mixed
    refs = decode_references(w, range(w.n_decode))
    _check_decode(w, outd, w.dtype, refs, w.name + " decode")


@pytest.mark.parametrize("half", [0, 1])
def test_mixed_step_every_prefill_row(mixed, half):
    w, gotp, _ = mixed
    atol, rtol = tolerance(w.dtype, w.dtype)
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    chunks = range(half * w.n_chunks // 2, (half + 1) * w.n_chunks // 2)
    for c in chunks:
        print(f"  chunk {c}: ctx {int(w.chunk_ctx[c])}, {int(w.chunk_qlen[c])} rows", flush=True)
        ref = prefill_references(w, [c])[c]
        assert_close(f"{w.name} chunk {c} ctx={int(w.chunk_ctx[c])}", gotp[cu[c]:cu[c + 1]], ref, atol, rtol)


def test_verify_every_row():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    from tests.helpers import prefill_reference, oracle_workers
    from concurrent.futures import ThreadPoolExecutor
    lens = synth.make_workload("llama3_8b_decode", 0).decode_lens
    w = synth.custom_workload("llama3_8b_verify", 32, 8, 128, "bf16", 70000, 0, chunk_ctx=lens - 1,
                              chunk_qlen=np.full(lens.size, 5))
    print("full-size verify: 256 sequences x 5 new tokens", flush=True)
    b = DeviceBatch(w, DEV, fill="device")
    b.append_prefill()
    out = b.new_prefill_out()
    b.attend_verify(out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(w.chunk_qlen)])
    with ThreadPoolExecutor(oracle_workers()) as ex:
        refs = list(ex.map(lambda c: prefill_reference(w, c, n_threads=1), range(w.n_chunks)))
    atol, rtol = tolerance("bf16", "bf16")
    for c, ref in enumerate(refs):
        assert_close(f"verify seq {c} ctx={int(w.chunk_ctx[c])}", got[cu[c]:cu[c + 1]], ref, atol, rtol)
