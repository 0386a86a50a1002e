"""Storage decoders for the oracle, written from the formats' definitions.

Test infrastructure only (see the package docstring).

* bf16: the upper 16 bits of an IEEE-754 binary32; decoding is exact.
* f16: IEEE-754 binary16, 1 sign bit, 5 exponent bits with bias 15, 10
  mantissa bits; exponent field 0 encodes subnormals m/1024 * 2^-14, field 31
  infinities (m = 0) and NaNs. Queries and outputs only (aiter #5628 "tune MTP
  work budgets and planned reduction", Validation: the FP16 cases of the
  decode tests).
* int8: a two's-complement integer code; the value is the code itself, later
  multiplied by its fp32 scale (hipfire #760 "split packed-Q8 verifier KV
  scans", Summary: int8 "Q8" KV; the per-token-per-head scale is this
  project's reading of that undefined layout).
* fp8 e4m3fn (OCP 8-bit floating point, E4M3 with no infinities): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits. Exponent field 0 encodes
  subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; the largest
  finite magnitude is 1.75 * 2^8 = 448. The pages only say "FP8 KV with
  per-token FP32 scales" (aiter #5628 "tune MTP work budgets and planned
  reduction", Performance); e4m3fn is the reading, being the format gfx950
  converts natively.
"""

from __future__ import annotations

import numpy as np


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns widen to NaN
        return u32.view(np.float32).astype(np.float64)


def decode_f16_bits(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (uint16) -> float64, exactly, from the field layout."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((u >> 15) & 1, -1.0, 1.0)
    e = (u >> 10) & 0x1F
    m = (u & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = sign * (m / 1024.0) * 2.0 ** (-14)
    special = np.where(m == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 0x1F, special, normal))


def _fp8_e4m3fn_scalar(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def fp8_e4m3fn_table() -> np.ndarray:
    """float64 value of each of the 256 e4m3fn codes, from the definition above."""
    return np.array([_fp8_e4m3fn_scalar(c) for c in range(256)], dtype=np.float64)


_FP8_TABLE = fp8_e4m3fn_table()


def decode_fp8_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """fp8 e4m3fn codes (uint8) -> float64, exactly."""
    return _FP8_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_storage(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a storage array of ``dtype`` ("f32", "bf16", "f16", "int8", "fp8") to float64."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16_bits(arr)
    if dtype == "f16":
        return decode_f16_bits(arr)
    if dtype == "int8":
        return np.asarray(arr, dtype=np.int8).astype(np.float64)
    if dtype == "fp8":
        return decode_fp8_e4m3fn(arr)
    raise ValueError(f"unknown storage dtype {dtype!r}")
