"""OCP FP8 E4M3 ("fn") codec, written from the format definition.  Test infrastructure.

The pages only say that the KV cache may be stored as FP8 ("NVIDIA TensorRT-LLM详解：
架构、KV Cache、调度与部署实践", §13, KvCacheConfig(dtype="fp8")) and that FP8 data is
converted back to 16-bit precision before accumulation ("TensorRT-LLM", 关键机制,
量化方案).  The bit format comes from the OCP 8-bit floating point specification:

  bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa
  exponent 0          subnormal:  (-1)^s * m/8 * 2^(1-7)
  exponent 1..15      normal:     (-1)^s * (1 + m/8) * 2^(e-7)
  S.1111.111          NaN (the only non-finite code; there are no infinities)
  largest finite      S.1111.110 = 448

Encoding (the reading used throughout this project): round to nearest, ties to the
code with an even mantissa; magnitudes >= 448 (and infinities) saturate to 448 with
their sign; NaN maps to the NaN code with its sign.
"""
from __future__ import annotations

import numpy as np


def _value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_value(c) for c in range(256)], dtype=np.float64)
_TABLE.setflags(write=False)
# Non-negative finite magnitudes, codes 0x00..0x7E, increasing with the code.
_POS = _TABLE[:0x7F].copy()


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    return _TABLE


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_e4m3(x) -> np.ndarray:
    """Values (float32 or float64; the float32 callers' values are exact in float64)
    -> uint8 codes by round-to-nearest-even with saturation at +-448."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    sign = np.signbit(flat).astype(np.uint8) << 7
    a = np.abs(flat)
    nan = np.isnan(flat)
    sat = ~nan & (a >= 448.0)
    mid = ~nan & ~sat
    am = a[mid]
    # largest code whose magnitude is <= a, and the next one up
    lo = np.searchsorted(_POS, am, side="right") - 1
    hi = np.minimum(lo + 1, 0x7E)
    dlo = am - _POS[lo]
    dhi = _POS[hi] - am
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    out[mid] = code | sign[mid]
    out[sat] = np.uint8(0x7E) | sign[sat]
    out[nan] = np.uint8(0x7F) | sign[nan]
    return out.reshape(x.shape)
