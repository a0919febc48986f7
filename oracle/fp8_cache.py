"""FP8 latent cache rows for the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The softved article ("Multi-Head Latent Attention...", "Practical
Implementation Tips for MLA in LLM Serving") advises applying quantization on
top of MLA to cut the cache further, and its "Understanding KV Cache" section
counts quantization among the techniques that only partly relieve the cache;
neither names a format or a scale.  Reading taken here:

* The latent part c (R values) of a cached row is stored in FP8 E4M3 as the
  OCP 8-bit floating point specification defines it: 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
  (m * 2^-9); no infinities; S.1111.111 is NaN; the largest finite value is
  448.
* One power-of-two scale per row, s = 2^ceil(log2(max|c| / 448)) (s = 1 for
  an all-zero c), so max|c| / s lies in (224, 448]; code_i is c_i / s
  rounded to the nearest E4M3 value, ties to the even code.  A stored value
  reads back as s * value(code_i), exact in float32 and bfloat16.
* The rope key (Dr values) stays bfloat16.
* Memory layout of one row, 16-byte aligned, R + 2 Dr + 16 bytes (656 at
  R = 512, Dr = 64): R code bytes, Dr little-endian bfloat16 values, the
  float32 scale, 12 zero bytes.

Pins: ``tests/test_oracle_pins.py`` checks the decoder on all 256 codes and
the rounding against torch's float8_e4m3fn (a library routine), closed forms
(448, 2^-9, ties to even) and the scale rule.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_value", "e4m3_round", "fp8_row_scale", "quantize_rows_fp8",
           "dequantize_rows_fp8", "fp8_row_bytes", "pack_rows_fp8", "unpack_rows_fp8",
           "fp8_store_rows"]

E4M3_MAX = 448.0


def e4m3_value(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8), from the field definition."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite codes in increasing value (code k has value
# _GRID[k], so the order of codes is the order of values)
_GRID = e4m3_value(np.arange(127))


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 code to each x, ties to the even code; |x| beyond 448
    saturates to +-448 (the scale rule never produces such values)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_GRID, a, side="left")          # first grid value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _GRID[lo], _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


def fp8_row_scale(c) -> np.ndarray:
    """Per-row power-of-two scale: 2^ceil(log2(max|c| / 448)), 1 for zero rows."""
    amax = np.max(np.abs(np.asarray(c, dtype=np.float64)), axis=-1)
    safe = np.where(amax > 0, amax, E4M3_MAX)
    return np.exp2(np.ceil(np.log2(safe / E4M3_MAX)))


def _bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 (ties to even), on the float64 bit pattern."""
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).view(np.uint64)
    drop = np.uint64(52 - 7)
    lsb = (bits >> drop) & np.uint64(1)
    half = np.uint64((1 << (52 - 7 - 1)) - 1)
    return (((bits + half + lsb) >> drop) << drop).view(np.float64)


def quantize_rows_fp8(rows, R: int):
    """rows [..., R + Dr] -> (codes uint8 [..., R], scales [...], rope [..., Dr] in bf16)."""
    rows = np.asarray(rows, dtype=np.float64)
    c, kr = rows[..., :R], rows[..., R:]
    s = fp8_row_scale(c)
    return e4m3_round(c / s[..., None]), s, _bf16_round(kr)


def dequantize_rows_fp8(codes, scales, rope) -> np.ndarray:
    """The values a reader of stored rows sees: [s * value(code) | rope]."""
    c = e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[..., None]
    return np.concatenate([c, np.asarray(rope, dtype=np.float64)], axis=-1)


def fp8_store_rows(rows, R: int) -> np.ndarray:
    """Value a row holds after being written to an FP8 cache."""
    return dequantize_rows_fp8(*quantize_rows_fp8(rows, R))


def fp8_row_bytes(R: int, Dr: int) -> int:
    return R + 2 * Dr + 16


def pack_rows_fp8(codes, scales, rope) -> np.ndarray:
    """Rows in the memory layout: uint8 [..., R + 2 Dr + 16]."""
    codes = np.asarray(codes, dtype=np.uint8)
    lead, R = codes.shape[:-1], codes.shape[-1]
    rope = np.asarray(rope, dtype=np.float64)
    Dr = rope.shape[-1]
    out = np.zeros(lead + (fp8_row_bytes(R, Dr),), dtype=np.uint8)
    out[..., :R] = codes
    # bfloat16 is the top half of the float32 bit pattern (exact for rounded values)
    rb = (np.ascontiguousarray(_bf16_round(rope).astype(np.float32)).view(np.uint32)
          >> np.uint32(16)).astype("<u2")
    out[..., R:R + 2 * Dr] = np.ascontiguousarray(rb).view(np.uint8).reshape(lead + (2 * Dr,))
    sc = np.ascontiguousarray(np.asarray(scales, dtype="<f4")).reshape(lead + (1,))
    out[..., R + 2 * Dr:R + 2 * Dr + 4] = sc.view(np.uint8).reshape(lead + (4,))
    return out


def unpack_rows_fp8(raw, R: int, Dr: int):
    """Inverse of pack_rows_fp8: (codes, scales, rope as float64)."""
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    lead = raw.shape[:-1]
    codes = raw[..., :R].copy()
    rb = np.ascontiguousarray(raw[..., R:R + 2 * Dr]).view("<u2").astype(np.uint32) << np.uint32(16)
    rope = rb.view(np.float32).astype(np.float64).reshape(lead + (Dr,))
    scales = np.ascontiguousarray(raw[..., R + 2 * Dr:R + 2 * Dr + 4]).view("<f4").astype(
        np.float64).reshape(lead)
    return codes, scales, rope
