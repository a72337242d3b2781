"""Pins of the oracle's 8-bit cache codec (E4M3 decoding and quantisation).

The pages say the KV cache may be stored in 8 bits ("Quantization", vLLM
Serving deep dive; the bytes-per-element note of the KV-size formula in The
hands-on guide to LLM Inference with vLLM) without fixing the format or a
scale rule.  The oracle reads them as OCP E4M3 with one fp32 scale per pool.
These tests tie its codec to things other than itself: the format's defining
values, PyTorch's own float8_e4m3fn conversion (a library routine), and the
properties round-to-nearest must have.
"""
import math

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_encode(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decoder_all_codes_match_torch():
    ours, ref = oracle.decode("fp8_e4m3", ALL), _torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_decoder_defining_values():
    v = oracle.decode("fp8_e4m3", ALL)
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0                  # exponent field 7 = bias
    assert v[0x3c] == 1.5
    assert v[0x7e] == 448.0 and v[0xfe] == -448.0
    assert math.isnan(v[0x7f]) and math.isnan(v[0xff])
    assert np.all(np.diff(v[:0x7f]) > 0)   # codes 0..0x7e increase strictly
    assert np.array_equal(v[0x80:0xff], -v[0x00:0x7f])


def test_encoder_matches_torch_on_codes_and_midpoints():
    vals = oracle.decode("fp8_e4m3", ALL[:0x7f])
    mids = (vals[:-1] + vals[1:]) / 2     # exact ties, fp32-representable
    x = np.concatenate([vals, mids, -vals, -mids]).astype(np.float32)
    assert np.array_equal(oracle.quantize_e4m3(x, 1.0), _torch_encode(x))


def test_encoder_matches_torch_on_random_in_range_values():
    rng = np.random.default_rng(0)
    y = (np.exp2(rng.uniform(-14, 8.8, 100000)) * rng.choice([-1, 1], 100000)).astype(np.float32)
    y = y[np.abs(y) <= 448]
    assert np.array_equal(oracle.quantize_e4m3(y, 1.0), _torch_encode(y))


def test_ties_go_to_the_even_code():
    v = oracle.decode("fp8_e4m3", ALL[:0x7f])
    for c in range(0x7e):
        mid = np.float32((v[c] + v[c + 1]) / 2)
        got = int(oracle.quantize_e4m3(np.array([mid]), 1.0)[0])
        assert got == (c if c % 2 == 0 else c + 1)


def test_saturation_and_nan():
    x = np.array([448, 449, 463.9, 464, 480, 1e30, np.inf, -500, -np.inf, np.nan, -np.nan], np.float32)
    got = oracle.quantize_e4m3(x, 1.0).tolist()
    assert got[:9] == [0x7e] * 6 + [0x7e, 0xfe, 0xfe]
    assert got[9] & 0x7f == 0x7f and got[10] & 0x7f == 0x7f


def test_round_trip_of_every_finite_code():
    finite = np.array([c for c in range(256) if c & 0x7f != 0x7f], np.uint8)
    vals = oracle.decode("fp8_e4m3", finite).astype(np.float32)
    assert np.array_equal(oracle.quantize_e4m3(vals, 1.0), finite)


def test_rounding_error_within_half_a_step():
    rng = np.random.default_rng(1)
    y = (np.exp2(rng.uniform(-12, 8.7, 50000)) * rng.choice([-1, 1], 50000)).astype(np.float32)
    back = oracle.decode("fp8_e4m3", oracle.quantize_e4m3(y, 1.0))
    err = np.abs(back - y.astype(np.float64))
    # normal range: half of a relative step 2^-3; subnormal range: half of 2^-9
    bound = np.where(np.abs(y) >= 2.0 ** -6, np.abs(y) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err <= bound)


@pytest.mark.parametrize("scale", [0.25, 2.0, 16.0, 2.0 ** -7])
def test_scale_divides_on_the_way_in_and_multiplies_on_the_way_out(scale):
    # power-of-two scales are exact: a representable value times the scale
    # quantises back to its own code and dequantises to the product
    finite = np.array([c for c in range(256) if c & 0x7f != 0x7f], np.uint8)
    vals = oracle.decode("fp8_e4m3", finite)
    x = (vals * scale).astype(np.float32)
    codes = oracle.quantize_e4m3(x, scale)
    assert np.array_equal(codes, finite)
    assert np.array_equal(oracle.dequantize_e4m3(codes, scale), vals * scale)


def test_non_power_of_two_scale_uses_the_fp32_reciprocal():
    # 1/3 is inexact in fp32, so x * fl(1/3) and x / 3 can land on opposite
    # sides of a tie: here the product hits the midpoint of codes 9 and 10
    # exactly (ties to even: 10) while the quotient falls just below it (9)
    inv = np.float32(1.0) / np.float32(3.0)
    assert inv == oracle.e4m3_inv_scale(3.0)
    x = np.float32(0.0556640587747097)
    assert np.float32(x * inv) == np.float32(0.0185546875)
    assert np.float32(x / np.float32(3.0)) < np.float32(0.0185546875)
    assert oracle.quantize_e4m3(np.array([x]), 3.0)[0] == 10


def test_fp8_pool_bytes_halve_bf16():
    # "Quantization", vLLM Serving deep dive: an 8-bit cache roughly doubles
    # the tokens a memory budget holds
    b16 = oracle.kv_bytes_per_token(32, 8, 128, oracle.ESIZE["bf16"])
    b8 = oracle.kv_bytes_per_token(32, 8, 128, oracle.ESIZE["fp8_e4m3"])
    assert b16 == 2 * b8
    budget = 40 * 2 ** 30
    assert oracle.blocks_for_budget(budget, 32, 8, 128, 1) == 2 * oracle.blocks_for_budget(budget, 32, 8, 128, 2)


def test_fp8_scatter_gather_roundtrip():
    rng = np.random.default_rng(2)
    nb, H, d, T = 6, 2, 64, 37
    bits = rng.integers(0, 256, size=(T, H, d), dtype=np.uint8)
    bits[(bits & 0x7f) == 0x7f] = 0  # no NaN codes, so values compare
    vbits = rng.integers(0, 256, size=(T, H, d), dtype=np.uint8)
    vbits[(vbits & 0x7f) == 0x7f] = 0
    kp = np.zeros(nb * H * 16 * d, np.uint8)
    vp = np.zeros_like(kp)
    table = rng.permutation(nb)[:3].astype(np.int32)
    slots = [oracle.slot(table, t, 16) for t in range(T)]
    oracle.scatter("fp8_e4m3", bits, vbits, kp, vp, slots, nb, 16, H, d)
    k, v = oracle.gather("fp8_e4m3", kp, vp, nb, 16, H, d, table, T)
    assert np.array_equal(k, oracle.decode("fp8_e4m3", bits))
    assert np.array_equal(v, oracle.decode("fp8_e4m3", vbits))
    # K layout: 16 one-byte dims of a token form one 16-byte chunk
    t, g, j = 21, 1, 37
    blk, off = table[t // 16], t % 16
    assert kp[(((blk * H + g) * (d // 16) + j // 16) * 16 + off) * 16 + j % 16] == bits[t, g, j]
    assert vp[((blk * H + g) * d + j) * 16 + off] == vbits[t, g, j]
