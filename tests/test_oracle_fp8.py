"""Pins of the oracle's E4M3 codec, bfloat16 rounding and block quantiser.

The codec is checked against the OCP 8-bit floating point specification's
closed form and against PyTorch's own float8_e4m3fn conversion (a separate
library implementation); the bf16 rounding against PyTorch's float32 ->
bfloat16 cast; the quantiser against its defining properties.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3_values(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_e4m3_codes(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch_e4m3_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0),
    (0xB8, -1.0), (0xFE, -448.0), (0x80, -0.0),
])
def test_decode_spec_values(code, value):
    # Values from the OFP8 E4M3 definition: bias 7, subnormal step 2^-9,
    # min normal 2^-6, max normal 1.75 * 2^8 = 448.
    got = oracle.e4m3_decode(np.array([code], np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_encode_midpoints_round_to_even():
    pos = np.arange(0, 0x7E, dtype=np.uint8)
    lo = oracle.e4m3_decode(pos)
    hi = oracle.e4m3_decode(pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)   # midpoints are exact in fp32
    got = oracle.e4m3_encode(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    # Just off the midpoint goes to the nearer neighbour.
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    assert np.array_equal(oracle.e4m3_encode(up), pos + 1)
    assert np.array_equal(oracle.e4m3_encode(dn), pos)
    # Worked cases: 1 + 1/16 is halfway between 1 and 1.125 -> 1 (even code 0x38);
    # 1 + 3/16 is halfway between 1.125 and 1.25 -> 1.25 (even code 0x3A).
    assert oracle.e4m3_encode(np.float32([1.0625, 1.1875])).tolist() == [0x38, 0x3A]


def test_encode_saturates():
    x = np.float32([448.0, 460.0, 464.0, 1e4, 3e38, -449.0, -1e6])
    assert oracle.e4m3_encode(x).tolist() == [0x7E] * 5 + [0xFE] * 2


def test_encode_matches_torch_in_range():
    g = np.random.Generator(np.random.PCG64(11))
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * np.float32(50.0),
        (g.random(100000).astype(np.float32) - 0.5) * np.float32(0.05),   # subnormal region
        (g.random(100000).astype(np.float32) * np.float32(447.0)),
    ])
    x = x[np.abs(x) < 448.0]
    assert np.array_equal(oracle.e4m3_encode(x), torch_e4m3_codes(x))


def test_round_bf16_matches_torch():
    g = np.random.Generator(np.random.PCG64(12))
    bits = g.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    # force exact ties (low half = 0x8000) on a quarter of them
    tie = g.random(bits.size) < 0.25
    bits = np.where(tie, (bits & 0xFFFF0000) | 0x8000, bits).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    ours = oracle.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_quantize_block_properties():
    g = np.random.Generator(np.random.PCG64(13))
    x = g.standard_normal((512, 128)).astype(np.float32) * np.exp2(
        g.integers(-20, 20, size=(512, 1))).astype(np.float32)
    codes, scales = oracle.quantize(x)
    amax = np.abs(x).max(axis=1)
    # scale is the float32 quotient amax / 448
    assert np.array_equal(scales, (amax / np.float32(448.0)).astype(np.float32))
    # the amax element lands on +-448
    arg = np.abs(x).argmax(axis=1)
    top = codes[np.arange(512), arg]
    assert np.all((top & 0x7F) == 0x7E)
    # every code is the correctly rounded E4M3 value of the float32 quotient
    q = (x / scales[:, None]).astype(np.float32)
    assert np.array_equal(codes, torch_e4m3_codes(q))
    # dequantisation error: half a step, relative 2^-4 for normals, 2^-10*scale below
    deq = oracle.dequantize(codes, scales)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))


def test_quantize_zero_row_and_power_of_two_scaling():
    x = np.zeros((2, 128), np.float32)
    x[1] = np.linspace(-3, 5, 128, dtype=np.float32)
    codes, scales = oracle.quantize(x)
    assert scales[0] == 1.0 and np.all((codes[0] & 0x7F) == 0)
    c2, s2 = oracle.quantize(x[1:] * np.float32(8.0))
    assert np.array_equal(c2, codes[1:]) and s2[0] == scales[1] * 8
