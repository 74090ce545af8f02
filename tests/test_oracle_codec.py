"""Pins of the oracle's bf16 widening and OCP E4M3 codec.

The pages do not fix the fp8 format (only that an fp8 KV cache halves the bytes).
The codec is pinned by the format definition's own fixed points and by
PyTorch's float8_e4m3fn conversion, a library routine written independently.
"""

import numpy as np
import pytest
import torch

import oracle

TABLE = oracle.e4m3_value_table()


def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x4049, 0x0001],
                    dtype=np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 0.0 and np.signbit(v[3])
    assert v[4] == np.inf and v[5] == -np.inf
    assert v[6] == 3.140625
    assert v[7] == 2.0 ** -133          # smallest bf16 subnormal
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_bf16_widening_matches_torch():
    g = np.random.default_rng(1)
    x = torch.from_numpy(g.standard_normal(4096).astype(np.float32) * 100).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x.double().numpy())


def test_e4m3_fixed_points():
    assert TABLE[0x38] == 1.0                 # e=7, m=0
    assert TABLE[0x3F] == 1.875
    assert TABLE[0x7E] == 448.0               # largest finite
    assert TABLE[0xFE] == -448.0
    assert TABLE[0x08] == 2.0 ** -6           # smallest normal
    assert TABLE[0x01] == 2.0 ** -9           # smallest subnormal
    assert TABLE[0x07] == 7 * 2.0 ** -9
    assert TABLE[0x00] == 0.0 and not np.signbit(TABLE[0x00])
    assert TABLE[0x80] == 0.0 and np.signbit(TABLE[0x80])
    assert np.isnan(TABLE[0x7F]) and np.isnan(TABLE[0xFF])
    assert np.sum(np.isnan(TABLE)) == 2
    pos = TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)           # monotone in the code


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    ours = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_e4m3_ties_to_even():
    # midpoints of adjacent codes go to the code with an even mantissa
    for c in range(0, 0x7E):
        mid = (TABLE[c] + TABLE[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == want, hex(c)
        assert oracle.e4m3_encode(np.array([-mid]))[0] == want | 0x80
    assert oracle.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00     # half the smallest subnormal
    assert oracle.e4m3_encode(np.array([-(2.0 ** -10)]))[0] == 0x80
    assert oracle.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02


def test_e4m3_saturation_nan_and_zero():
    y = np.array([448.0, 449.0, 463.9, 464.0, 465.0, 1e9, np.inf, -np.inf, -500.0, np.nan,
                  -np.nan, 0.0, -0.0], dtype=np.float64)
    got = oracle.e4m3_encode(y)
    assert list(got[:7]) == [0x7E] * 7
    assert got[7] == 0xFE and got[8] == 0xFE
    assert got[9] == 0x7F
    assert got[10] == 0xFF
    assert got[11] == 0x00 and got[12] == 0x80


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * 50,
        g.standard_normal(50000).astype(np.float32) * 1e-2,
        (g.random(50000).astype(np.float32) - 0.5) * 896,
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def test_e4m3_brute_force_nearest():
    # exhaustive nearest-value search over all finite codes on random inputs
    g = np.random.default_rng(3)
    x = (g.standard_normal(3000) * 30).astype(np.float32).astype(np.float64)
    finite = np.array([c for c in range(256) if not np.isnan(TABLE[c])])
    vals = TABLE[finite]
    got = oracle.e4m3_encode(x)
    for xi, gi in zip(x, got):
        dist = np.abs(vals - xi)
        best = finite[dist == dist.min()]
        best = best[np.signbit(TABLE[best]) == np.signbit(xi)] if len(best) > 1 else best
        if len(best) > 1:
            best = best[(best & 1) == 0]
        assert gi == best[0]


def test_e4m3_scaled_widening_matches_torch():
    # every finite code times a float32 scale: torch's float8_e4m3fn decode in
    # float64 times the scale (exact: 4 significant bits times 24)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for s in (np.float32(0.0123), np.float32(3.0), np.float32(448.0 / 7.3)):
        got = oracle.attention.widen(codes, "fp8", s)
        assert np.array_equal(got, ref * float(s))
        assert np.array_equal(np.signbit(got), np.signbit(ref))


@pytest.mark.parametrize("inv_scale", [1.0, 0.125, 3.0])
def test_table_mapped_quantise_equals_the_oracle(inv_scale):
    """The GPU tests quantise gigabyte pools by mapping each bf16 pattern
    through the oracle's codes for all 65536 patterns (helpers.oracle_quantise_bf16).
    That is the oracle's own result element for element: checked here on every
    pattern and on a random pool-shaped sample."""
    from helpers import oracle_quantise_bf16
    every = np.arange(1 << 16, dtype=np.uint16)
    assert np.array_equal(oracle_quantise_bf16(every, inv_scale), oracle.quantise(every, "bf16", inv_scale))
    g = np.random.default_rng([7, int(inv_scale * 8)])
    pool = g.integers(0, 1 << 16, size=(5, 2, 16, 64), dtype=np.uint16)
    assert np.array_equal(oracle_quantise_bf16(pool, inv_scale), oracle.quantise(pool, "bf16", inv_scale))
