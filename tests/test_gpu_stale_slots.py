"""Slots of the pool outside every context — the unwritten tail of a
sequence's last block, blocks no table names — hold whatever an earlier
owner left there (the pages' "Memory sharing" and "Life of a prompt" block
reuse: a freed block returns to the queue with its bytes).  No output may
depend on them: chunked prefill, verify and decode are run over the same
batch with those slots left as written, set to +300 and set to -300, and
every output must be identical bit for bit.  Chunks end inside a 16-token
query tile, so the rows that pad the last tile are exercised as well."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _valid_slots(b):
    """[num_blocks, 16] mask of the slots inside some context of the batch."""
    w = b.w
    valid = np.zeros((w.num_blocks, 16), dtype=bool)
    spans = []
    if b.prefill is not None:
        lens = (w.chunk_ctx + w.chunk_qlen).astype(np.int64)
        spans += [(b.prefill.tables_host[c], int(lens[c])) for c in range(w.n_chunks)]
    if b.decode is not None:
        spans += [(b.decode.tables_host[s], int(b.decode.lens[s])) for s in range(w.n_decode)]
    for tab, L in spans:
        for j in range(-(-L // 16)):
            valid[tab[j], :min(16, L - 16 * j)] = True
    return torch.from_numpy(valid).to(DEV)


def _poison(b, valid, value):
    w = b.w
    x = 16 // b.k_pool.element_size()
    k = b.k_pool.view(w.num_blocks, w.n_kv_heads, w.head_dim // x, 16, x)
    v = b.v_pool.view(w.num_blocks, w.n_kv_heads, w.head_dim, 16)
    inv = ~valid
    k.masked_fill_(inv[:, None, None, :, None], value)
    v.masked_fill_(inv[:, None, None, :], value)


def _outputs(b):
    pre = torch.empty(tuple(b.prefill.q.shape), dtype=torch.float32, device=DEV)
    ver = torch.empty_like(pre)
    dec = torch.empty((b.w.n_decode, b.w.n_q_heads, b.w.head_dim), dtype=torch.float32, device=DEV)
    b.attend_prefill(pre)
    b.attend_verify(ver)
    b.attend_decode(dec)
    torch.cuda.synchronize()
    return pre, ver, dec


@pytest.mark.parametrize("Hq,Hkv,d,dtype", [(32, 8, 128, "bf16"), (16, 8, 128, "f16"), (32, 4, 64, "bf16"),
                                            (8, 8, 128, "bf16")], ids=["g4_d128_bf16", "g2_d128_f16",
                                                                         "g8_d64_bf16", "g1_d128_bf16"])
def test_slots_outside_the_contexts_change_no_output(Hq, Hkv, d, dtype):
    from paged_kv_cache_gather_amd.batch import DeviceBatch
    print(f"stale slots: Hq {Hq} Hkv {Hkv} d {d} {dtype}", flush=True)
    # chunk lengths end inside a query tile; contexts end inside a block and
    # inside a 64-key step; decode lengths likewise, one spanning partitions
    w = synth.custom_workload(f"stale_{dtype}_{d}_{Hq}_{Hkv}", Hq, Hkv, d, dtype, 1024, seed=61,
                              chunk_ctx=[0, 1, 17, 100, 700], chunk_qlen=[5, 61, 33, 3, 61],
                              decode_lens=[1, 15, 33, 517, 1300])
    b = DeviceBatch(w, DEV, fill="host", out_dtype="f32")
    b.append_prefill()
    b.append_decode()
    torch.cuda.synchronize()
    base = _outputs(b)
    valid = _valid_slots(b)
    assert (~valid).any()
    for value in (300.0, -300.0):
        _poison(b, valid, value)
        torch.cuda.synchronize()
        got = _outputs(b)
        for name, a, g in zip(("prefill", "verify", "decode"), base, got):
            assert not torch.isnan(g).any(), name
            nd = int((a != g).sum())
            assert nd == 0, f"{name}: {nd} elements change when slots outside the contexts hold {value}"
