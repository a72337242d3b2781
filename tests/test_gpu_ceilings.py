"""The measurement calls the benchmark sets beside the attention kernels:
paged_kv_read_tiles (a read-only pass over pool tiles) reads the tiles its
list names, and paged_kv_mfma_rate runs in every mode; both reject bad
arguments."""
import pytest
import torch

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"
MAGIC = 0x9E3779B9  # the XOR value at which the read pass writes its sink


def test_read_tiles_reads_the_listed_tiles():
    import paged_kv_cache_gather_amd as pkv
    # four 64-byte tiles per pool; tile 2 of v_pool holds one word equal to
    # MAGIC, every other byte is zero, so the sink is written exactly when
    # that tile is read
    k = torch.zeros(4 * 16, dtype=torch.int32, device=DEV)
    v = torch.zeros(4 * 16, dtype=torch.int32, device=DEV)
    v[2 * 16 + 5] = MAGIC - (1 << 32)  # the same 32 bits as a signed int32
    for tiles, n_k, hit in (([0, 1, 2], 1, True), ([0, 1, 3], 1, False), ([2, 0, 1], 3, False),
                            ([3, 2], 0, True)):
        sink = torch.zeros(1, dtype=torch.int32, device=DEV)
        t = torch.tensor(tiles, dtype=torch.int64, device=DEV)
        pkv.paged_kv_read_tiles(k, v, t, n_k, len(tiles), 64, sink)
        torch.cuda.synchronize()
        got = int(sink.item()) & 0xFFFFFFFF
        assert got == (MAGIC if hit else 0), (tiles, n_k, hex(got))
    # contiguous read of k_pool only, streaming and plain loads
    for streaming in (True, False):
        sink = torch.zeros(1, dtype=torch.int32, device=DEV)
        pkv.paged_kv_read_tiles(v, None, None, 4, 4, 64, sink, streaming=streaming)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == MAGIC


def test_read_tiles_rejects_bad_arguments():
    import paged_kv_cache_gather_amd as pkv
    k = torch.zeros(64, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    t = torch.zeros(2, dtype=torch.int64, device=DEV)
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_kv_read_tiles(k, k, t, 3, 2, 64, sink)  # more K tiles than tiles
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_kv_read_tiles(k, k, t, 1, 2, 24, sink)  # not a multiple of 16
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_kv_read_tiles(k, None, None, 1, 2, 64, sink)  # contiguous reads take k_pool only


def test_mfma_rate_runs_every_mode_and_rejects_bad_arguments():
    import paged_kv_cache_gather_amd as pkv
    sink = torch.zeros(1, dtype=torch.float32, device=DEV)
    for mode in range(4):
        pkv.paged_kv_mfma_rate(mode, 8, 16, sink)
    torch.cuda.synchronize()
    assert float(sink.item()) == 0.0
    for mode, n_wg, iters in ((4, 8, 16), (-1, 8, 16), (0, 0, 16), (0, 65536, 16), (0, 8, 0)):
        with pytest.raises(pkv.PagedKVError):
            pkv.paged_kv_mfma_rate(mode, n_wg, iters, sink)
