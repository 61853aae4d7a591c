"""OCP MXFP4 codec, written from the Microscaling (MX) format definition.  Test
infrastructure.

The pages name a 4-bit KV cache only as a storage choice ("NVIDIA TensorRT-LLM详解：
架构、KV Cache、调度与部署实践", §13, the quantization recipes and
KvCacheConfig(dtype="nvfp4")); that format is NVIDIA's.  The 4-bit cache here is the
open OCP Microscaling one, MXFP4, taken from the OCP MX v1.0 specification:

  block     32 consecutive elements share one scale X
  scale     E8M0: one byte E, X = 2^(E - 127); E = 255 is NaN (never produced here)
  element   FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa
            exponent 0: (-1)^s * m/2 ; exponent 1..3: (-1)^s * (1 + m/2) * 2^(e-1)
            magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities, no NaN
  value     element value * X

Encoding, the specification's conversion of a block of higher-precision values:
  shared exponent  floor(log2(max_i |x_i|)) - 2   (2 = largest exponent of E2M1),
                   clamped to the E8M0 range [-127, 127]; a block of zeros takes -127
  elements         x_i / X rounded to the nearest E2M1 value, ties to the even
                   mantissa, magnitudes above 6 clamped to 6; the sign bit is x_i's.

A cached K or V row of head_dim D (a multiple of 32) is D/32 blocks along D, each
encoded by itself, so every appended token is encoded alone.  This module's logical
form of a row is D codes (one per byte, 0..15) followed by D/32 scale bytes.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
EMAX_ELEM = 2                  # largest unbiased exponent of E2M1 (6 = 1.5 * 2^2)
SCALE_BIAS = 127

# E2M1 magnitudes by the 3 low code bits, increasing with the code
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_MAG.setflags(write=False)


def decode_fp4(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64 element values (code 8 is -0.0)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = _MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def scale_value(scale_bytes) -> np.ndarray:
    """E8M0 bytes -> float64 scales 2^(E - 127) (NaN for 255)."""
    e = np.asarray(scale_bytes, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - SCALE_BIAS))


def shared_exponent(amax) -> np.ndarray:
    """Block scale exponent from the block's largest magnitude (>= 0, finite)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)               # amax = f * 2^ex, f in [0.5, 1): floor(log2) = ex - 1
    e = np.clip(ex.astype(np.int64) - 1 - EMAX_ELEM, -SCALE_BIAS, SCALE_BIAS)
    return np.where(amax > 0, e, -SCALE_BIAS)


def round_e2m1(q) -> np.ndarray:
    """Non-negative magnitudes -> E2M1 magnitude codes 0..7: nearest value, ties to the
    code with an even mantissa (even code), above 6 clamped to 6."""
    q = np.asarray(q, dtype=np.float64)
    lo = np.clip(np.searchsorted(_MAG, q, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    dlo = q - _MAG[lo]
    dhi = _MAG[hi] - q
    pick_hi = (hi != lo) & ((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)))
    return np.where(pick_hi, hi, lo).astype(np.uint8)


def mx_encode(x) -> tuple[np.ndarray, np.ndarray]:
    """Values [..., D] (finite; D a multiple of 32) -> (codes [..., D] uint8 0..15,
    scale bytes [..., D/32] uint8)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % BLOCK == 0, D
    blocks = x.reshape(x.shape[:-1] + (D // BLOCK, BLOCK))
    e = shared_exponent(np.abs(blocks).max(axis=-1))
    q = np.abs(blocks) / np.ldexp(1.0, e)[..., None]      # exact: a power-of-two scale
    mag = round_e2m1(q)
    sign = np.signbit(blocks).astype(np.uint8) << 3
    codes = (mag | sign).reshape(x.shape)
    return codes.astype(np.uint8), (e + SCALE_BIAS).astype(np.uint8)


def mx_decode(codes, scale_bytes) -> np.ndarray:
    """(codes [..., D], scale bytes [..., D/32]) -> float64 values [..., D]."""
    codes = np.asarray(codes, dtype=np.uint8)
    D = codes.shape[-1]
    v = decode_fp4(codes).reshape(codes.shape[:-1] + (D // BLOCK, BLOCK))
    return (v * scale_value(scale_bytes)[..., None]).reshape(codes.shape)
