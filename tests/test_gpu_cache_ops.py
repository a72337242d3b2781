"""GPU parity of the cache writes and of the generator's device fill:
bit-exact against the oracle's host scatter / block copy and numpy."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

DEV = "cuda:0"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CONT = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
VIEW = {"f32": (np.int32, torch.int32), "f16": (np.int16, torch.int16), "bf16": (np.int16, torch.int16)}


def _to_dev(bits, dtype):
    nv, tv = VIEW[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(nv)).to(DEV).view(TDT[dtype])


def _to_host(t, dtype):
    nv, tv = VIEW[dtype]
    return t.view(tv).cpu().numpy().view(CONT[dtype])


@pytest.mark.parametrize("dtype,H,d", [("bf16", 8, 128), ("f16", 4, 64), ("f32", 2, 64), ("f16", 40, 128)])
def test_reshape_and_cache_bit_exact(dtype, H, d):
    import paged_kv_cache_gather_amd as pkv
    print(f"reshape_and_cache {dtype} H={H} d={d}", flush=True)
    rng = np.random.default_rng(1)
    nb, T = 64, 300
    info = np.iinfo(CONT[dtype])
    kbits = rng.integers(0, info.max, size=(T, H, d), dtype=np.uint64).astype(CONT[dtype])
    vbits = rng.integers(0, info.max, size=(T, H, d), dtype=np.uint64).astype(CONT[dtype])
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[::7] = -1  # padding tokens are skipped
    n = oracle.pool_elems(nb, 16, H, d)
    kp_ref = np.zeros(n, CONT[dtype])
    vp_ref = np.zeros(n, CONT[dtype])
    oracle.scatter(dtype, kbits, vbits, kp_ref, vp_ref, slots, nb, 16, H, d)
    kp = torch.zeros(n, dtype=TDT[dtype], device=DEV)
    vp = torch.zeros_like(kp)
    pkv.reshape_and_cache(_to_dev(kbits, dtype).view(T, -1), _to_dev(vbits, dtype).view(T, -1), kp, vp,
                          torch.from_numpy(slots).to(DEV), nb, H, d)
    torch.cuda.synchronize()
    assert np.array_equal(_to_host(kp, dtype), kp_ref)
    assert np.array_equal(_to_host(vp, dtype), vp_ref)


def test_reshape_and_cache_strided_rows():
    # key/value as column slices of a fused [T, q | k | v] projection buffer
    import paged_kv_cache_gather_amd as pkv
    rng = np.random.default_rng(2)
    T, Hq, H, d, nb = 37, 32, 8, 128, 16
    fused = rng.integers(0, 65535, size=(T, (Hq + 2 * H) * d), dtype=np.uint64).astype(np.uint16)
    fd = _to_dev(fused, "bf16")
    kcols = slice(Hq * d, (Hq + H) * d)
    vcols = slice((Hq + H) * d, (Hq + 2 * H) * d)
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    n = oracle.pool_elems(nb, 16, H, d)
    kp_ref = np.zeros(n, np.uint16)
    vp_ref = np.zeros(n, np.uint16)
    oracle.scatter("bf16", fused[:, kcols].reshape(T, H, d), fused[:, vcols].reshape(T, H, d), kp_ref, vp_ref,
                   slots, nb, 16, H, d)
    kp = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    pkv.reshape_and_cache(fd[:, kcols], fd[:, vcols], kp, vp, torch.from_numpy(slots).to(DEV), nb, H, d)
    torch.cuda.synchronize()
    assert np.array_equal(_to_host(kp, "bf16"), kp_ref)
    assert np.array_equal(_to_host(vp, "bf16"), vp_ref)


def test_copy_blocks_bit_exact():
    import paged_kv_cache_gather_amd as pkv
    rng = np.random.default_rng(3)
    nb, H, d = 32, 8, 128
    n = oracle.pool_elems(nb, 16, H, d)
    k0 = rng.integers(0, 65535, size=n, dtype=np.uint64).astype(np.uint16)
    v0 = rng.integers(0, 65535, size=n, dtype=np.uint64).astype(np.uint16)
    pairs = np.array([[3, 17], [5, 6], [31, 0]], np.int32)
    kr, vr = k0.copy(), v0.copy()
    oracle.copy_blocks("bf16", kr, vr, pairs, nb, 16, H, d)
    kp, vp = _to_dev(k0, "bf16"), _to_dev(v0, "bf16")
    pkv.paged_kv_copy_blocks(kp, vp, torch.from_numpy(pairs).to(DEV), nb, H, d)
    torch.cuda.synchronize()
    assert np.array_equal(_to_host(kp, "bf16"), kr)
    assert np.array_equal(_to_host(vp, "bf16"), vr)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_device_fill_matches_host_generator(dtype):
    key = synth.stream_key(7, synth.KIND_V, 12345)
    t0, t1, H, d = 1000, 1333, 8, 128
    t = torch.empty((t1 - t0, H, d), dtype=TDT[dtype], device=DEV)
    synth.fill_device(t, t0, t1, H, d, key, dtype)
    torch.cuda.synchronize()
    ref = synth.values(7, synth.KIND_V, 12345, t0, t1, H, d, dtype)
    assert np.array_equal(_to_host(t, dtype).reshape(ref.shape), ref)
