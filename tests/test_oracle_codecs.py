"""Pins of the oracle's storage decoders against library routines and known values."""

import math

import numpy as np
import torch

import oracle


def test_fp8_table_matches_torch_for_all_256_codes():
    ours = oracle.fp8_e4m3fn_table()
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], lib[~nan])


def test_fp8_known_values():
    t = oracle.fp8_e4m3fn_table()
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                         # largest subnormal
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    finite = t[np.isfinite(t)]
    assert len(np.unique(finite)) == 253                    # +0 and -0 compare equal


def test_fp8_encode_decode_roundtrip_within_half_ulp():
    x = torch.linspace(-448, 448, 20001, dtype=torch.float32)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    dec = oracle.decode_fp8_e4m3fn(codes)
    xs = x.double().numpy()
    # relative spacing of e4m3 normals is 2^-3, so RNE error <= 2^-4 relative (or 2^-10 abs)
    err = np.abs(dec - xs)
    assert np.all(err <= np.maximum(np.abs(xs) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=50000).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = oracle.decode_bf16_bits(bits)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_int8_and_f32_decode():
    a = np.arange(-128, 128).astype(np.int8)
    assert np.array_equal(oracle.decode_storage(a, "int8"), np.arange(-128, 128, dtype=np.float64))
    f = np.array([1.5, -2.25, 3e-8], dtype=np.float32)
    assert np.array_equal(oracle.decode_storage(f, "f32"), f.astype(np.float64))


def test_f16_decode_matches_torch_for_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    ours = oracle.decode_f16_bits(bits)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 * 1023                           # exponent 31 with a nonzero mantissa
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_f16_known_values():
    d = lambda b: float(oracle.decode_storage(np.array([b], dtype=np.uint16), "f16")[0])
    assert d(0x3C00) == 1.0 and d(0xC000) == -2.0
    assert d(0x7BFF) == 65504.0                             # largest finite
    assert d(0x0001) == 2.0 ** -24                          # smallest subnormal
    assert d(0x03FF) == 1023 * 2.0 ** -24                   # largest subnormal
    assert d(0x0400) == 2.0 ** -14                          # smallest normal
    assert d(0x3555) == 1365 / 4096                         # 0.333251953125
    assert d(0x7C00) == float("inf") and d(0xFC00) == -float("inf")
    assert math.isnan(d(0x7E00))
