"""Pins of the oracle's OCP E4M3 codec against the format definition and an
independent library cast (torch.float8_e4m3fn)."""
import numpy as np
import pytest
import torch

from oracle import decode_table, encode_e4m3


def torch_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_table_matches_torch_float8_e4m3fn():
    ours, ref = decode_table(), torch_table()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zeros too
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_table_counts_and_extremes():
    t = decode_table()
    assert t.shape == (256,)
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    fin = t[~np.isnan(t)]
    assert fin.size == 254
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x38] == 1.0


def test_roundtrip_every_finite_code():
    t = decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], np.uint8)
    back = encode_e4m3(t[codes])
    # -0 and +0 both round-trip to their own code
    assert np.array_equal(back, codes)


def test_monotone():
    x = np.linspace(-460, 460, 200001)
    v = decode_table()[encode_e4m3(x)]
    assert np.all(np.diff(v) >= 0)


def test_midpoints_round_to_even_code():
    t = decode_table()
    pos = t[:0x7F]
    for c in range(0, 0x7E):
        mid = (pos[c] + pos[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert encode_e4m3(np.float64(mid)) == want, hex(c)
        assert encode_e4m3(np.float64(-mid)) == want | 0x80


def test_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(50),
        rng.uniform(-448, 448, 200000).astype(np.float32),
        (rng.standard_normal(200000) * 2.0 ** -8).astype(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_e4m3(x), ref)


def test_saturation_and_nan():
    x = np.array([448.0, 449.0, 464.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert encode_e4m3(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    n = encode_e4m3(np.array([np.nan, -np.nan], np.float32))
    assert (n & 0x7F).tolist() == [0x7F, 0x7F]


@pytest.mark.parametrize("v", [2.0 ** -10, 2.0 ** -11])
def test_tiny_values_round_to_zero(v):
    assert encode_e4m3(np.float64(v)) == 0
    assert encode_e4m3(np.float64(-v)) == 0x80
