"""Whole steps captured in a HIP graph and replayed.

The library allocates nothing, clears nothing with memset and never
synchronises inside its entry points, so a step — the cache write, then the
attention (partition pass and merge) — can be captured from torch's current
stream and replayed.  Each step is run eagerly once, captured, and replayed
several times with eager work (refilling the outputs) and synchronisations in
between; every replay must reproduce the eager outputs bit for bit."""
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.helpers import FP8_K_SCALE, FP8_V_SCALE

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _replays_match(step, outs, replays=4):
    side = torch.cuda.Stream(device=DEV)  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager, off the default stream (also creates lazily sized buffers)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [_bits(o).clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(replays):
        for o in outs:
            o.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(_bits(o), r), f"replay {i} differs from the eager step"


def _decode_batch(**kw):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    # shared prefixes (so the shared-run kernel has work), several partitions
    w = synth.custom_workload("graph_decode", 32, 8, 128, "bf16", 2048, seed=41,
                              decode_lens=[1100, 1100, 1500, 2100, 600, 17, 1, 3000],
                              prefix_len=[1030, 1030, 1030, 1030, 0, 0, 0, 0], prefix_group=[0, 0, 0, 0, -1, -1, -1, -1])
    return DeviceBatch(w, DEV, fill="host", out_dtype="bf16", **kw)


def test_decode_step_replays():
    b = _decode_batch()
    out = b.new_decode_out()
    print("graph decode bf16", flush=True)

    def step():
        b.append_decode()
        b.attend_decode(out)

    _replays_match(step, [out])


def test_decode_step_in_one_call_replays():
    b = _decode_batch()
    out = b.new_decode_out()
    print("graph decode_append", flush=True)
    _replays_match(lambda: b.step_decode(out), [out])


def test_decode_step_over_an_8bit_cache_replays():
    b = _decode_batch(kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    out = b.new_decode_out()
    print("graph decode fp8", flush=True)

    def step():
        b.append_decode()
        b.attend_decode(out)

    _replays_match(step, [out])


def test_decode_step_in_one_call_over_an_8bit_cache_replays():
    b = _decode_batch(kv_cache="fp8_e4m3", k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    out = b.new_decode_out()
    print("graph decode_fp8_append", flush=True)
    _replays_match(lambda: b.step_decode(out), [out])


def test_prefill_and_verify_steps_replay():
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    w = synth.custom_workload("graph_chunks", 32, 8, 128, "bf16", 2048, seed=43, chunk_ctx=[0, 700, 1500],
                              chunk_qlen=[40, 5, 64])
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    out_p, out_v = b.new_prefill_out(), b.new_prefill_out()
    print("graph prefill + verify", flush=True)

    def step():
        b.append_prefill()
        b.attend_prefill(out_p)
        b.attend_verify(out_v)

    _replays_match(step, [out_p, out_v])
