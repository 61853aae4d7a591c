"""Pins of the oracle's OCP MXFP4 codec against the format definition: the E2M1 bit
layout, torch's independent E8M0 decoding, exact round trips of representable blocks,
the round-to-nearest-even ties, clamping, the error bound, and an exhaustive search
on small blocks."""
import math

import numpy as np
import pytest
import torch

from oracle.mxfp4 import decode_fp4, mx_decode, mx_encode, scale_value, shared_exponent


def e2m1_from_bits(code: int) -> float:
    """E2M1 value straight from its bit fields (sign, 2-bit exponent with bias 1, 1-bit
    mantissa; exponent 0 is subnormal)."""
    s = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    return s * (m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))


def test_fp4_table_from_bit_fields():
    for c in range(16):
        assert decode_fp4(np.uint8(c)) == e2m1_from_bits(c), c
    assert decode_fp4(np.uint8(7)) == 6.0 and decode_fp4(np.uint8(15)) == -6.0   # largest normal
    assert decode_fp4(np.uint8(1)) == 0.5                                       # only subnormal
    assert np.signbit(decode_fp4(np.uint8(8)))                                  # -0


def test_scale_bytes_match_torch_e8m0():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = scale_value(b)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127


def test_shared_exponent_closed_form():
    # floor(log2 amax) - 2, clamped to [-127, 127]; zero blocks take -127
    for a in [1.0, 1.5, 2.0, 3.999, 4.0, 6.0, 7.99, 0.3, 2.0 ** -100, 2.0 ** 120, 3e38]:
        want = max(-127, min(127, math.floor(math.log2(a)) - 2))
        assert shared_exponent(a) == want, a
    assert shared_exponent(0.0) == -127
    assert shared_exponent(2.0 ** -133) == -127        # a bf16 subnormal


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_representable_blocks_round_trip(seed):
    """A block of E2M1 values times 2^k whose largest magnitude is 4 or 6 (so the
    encoder picks exactly that 2^k) encodes back to the same codes and scale."""
    rng = np.random.default_rng(seed)
    n = 200
    codes = rng.integers(0, 16, size=(n, 32)).astype(np.uint8)
    codes[:, rng.integers(0, 32, n)] = 0                   # some zeros
    top = rng.integers(0, 32, n)
    codes[np.arange(n), top] = rng.choice([6, 7, 14, 15], n)  # magnitude 4 or 6 present
    k = rng.integers(-120, 120, n)
    x = decode_fp4(codes) * np.ldexp(1.0, k)[:, None]
    c2, s2 = mx_encode(x)
    assert np.array_equal(s2[:, 0].astype(int) - 127, k)
    # -0 and +0 keep their sign bit
    assert np.array_equal(c2, codes)
    assert np.array_equal(mx_decode(c2, s2), x)


def test_ties_round_to_even_mantissa():
    # scale fixed at 2^0 by an element of magnitude 4; then each tie point
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for q, want in ties.items():
        x = np.zeros(32)
        x[0] = 4.0
        x[5] = q
        x[9] = -q
        c, s = mx_encode(x)
        assert s[0] == 127
        v = mx_decode(c, s)
        assert v[5] == want and v[9] == -want, q
    # just off the ties go to the nearer value
    for q, want in {0.2500001: 0.5, 0.7499999: 0.5, 4.9999: 4.0, 5.0001: 6.0}.items():
        x = np.zeros(32)
        x[0], x[3] = 4.0, q
        assert mx_decode(*mx_encode(x))[3] == want, q


def test_clamp_above_six():
    # max 7.9 -> scale 2^(2-2) = 1; 7.9 and 6.5 clamp to 6
    x = np.zeros(32)
    x[0], x[1], x[2] = 7.9, -6.5, 5.5
    c, s = mx_encode(x)
    assert s[0] == 127
    v = mx_decode(c, s)
    assert v[0] == 6.0 and v[1] == -6.0 and v[2] == 6.0


def test_zero_and_negative_zero():
    x = np.zeros(64)
    x[40] = -0.0
    c, s = mx_encode(x)
    assert np.array_equal(s, [0, 0])
    assert c[40] == 8 and np.count_nonzero(c) == 1


@pytest.mark.parametrize("seed", [3, 4])
def test_error_bound_gaussian_rows(seed):
    """|x - dequant(x)| <= X * (half the E2M1 spacing at |x|/X), and <= 2X in the
    clamped range (6, 8)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-5, 5, (64, 1)))
    c, s = mx_encode(x)
    v = mx_decode(c, s)
    X = np.repeat(scale_value(s), 32, axis=-1)
    q = np.abs(x) / X
    assert q.max() < 8.0
    half = np.select([q <= 2.0, q <= 4.0, q <= 6.0], [0.25, 0.5, 1.0], 2.0)
    assert np.all(np.abs(x - v) <= half * X)
    # the block maximum lands in [4, 8) scale units
    qb = q.reshape(64, 4, 32).max(axis=-1)
    assert np.all((qb >= 4.0) & (qb < 8.0))


def test_exhaustive_nearest_on_small_blocks():
    """Each element's code is the nearest of all 16 codes to x / X (ties: even
    mantissa), found by brute force."""
    rng = np.random.default_rng(5)
    allv = np.array([e2m1_from_bits(c) for c in range(16)])
    for _ in range(50):
        x = rng.standard_normal(32) * 3.0
        x[rng.integers(0, 32)] = rng.choice([0.25, 0.75, 2.5, 5.0]) * 2.0 ** (
            math.floor(math.log2(np.abs(x).max())) - 2)    # a tie point now and then
        c, s = mx_encode(x)
        X = 2.0 ** (int(s[0]) - 127)
        assert X == 2.0 ** (math.floor(math.log2(np.abs(x).max())) - 2)
        for i in range(32):
            q = x[i] / X
            d = np.abs(allv - min(max(q, -6.0), 6.0))
            best = np.flatnonzero(d == d.min())
            # among equal distances the code with mantissa bit 0; same sign as x
            cands = [b for b in best if (b & 8) == (8 if np.signbit(x[i]) else 0)] or list(best)
            pick = [b for b in cands if b & 1 == 0] or cands
            assert allv[c[i]] == allv[pick[0]], (q, c[i], pick)
