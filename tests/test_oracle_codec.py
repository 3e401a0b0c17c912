"""Pins of the oracle's group codec (CPU only).

Each check is fixed by mathematics or by an independent brute force, not by
re-typing the oracle's formula:
* fp16 directed rounding vs a search over every finite fp16 value;
* quantization error <= half a step and codes equal to the exact nearest
  grid point (rational arithmetic, ties to the even code);
* the grid [z, z + L*s] covers [min, max];
* constant and single-value groups are lossless;
* 4-bit code == 4*hi + lo for all 16 codes; pack/unpack over all 256 bytes;
* hand-derived fixtures (tests/golden/codec_cases.txt).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_f16_sorted():
    h = np.arange(65536, dtype=np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    return np.unique(h.astype(np.float64))


def _all_bf16_finite():
    b = np.arange(65536, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_f16_round_down_exhaustive_bf16():
    grid = _all_finite_f16_sorted()
    x = _all_bf16_finite()
    x = x[np.abs(x) <= 65504.0]
    z = codec.f16_round_down(x).astype(np.float64)
    idx = np.searchsorted(grid, x.astype(np.float64), side="right") - 1
    assert np.array_equal(z, grid[idx])


def test_f16_round_up_random_f32():
    rng = np.random.default_rng(1)
    grid = _all_finite_f16_sorted()
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(7.0),
        (rng.random(50000) * 1e-4).astype(np.float32),
        rng.integers(-2000, 2000, 1000).astype(np.float32) / np.float32(64.0),
    ])
    s = codec.f16_round_up(x).astype(np.float64)
    idx = np.searchsorted(grid, x.astype(np.float64), side="left")
    assert np.array_equal(s, grid[idx])
    zd = codec.f16_round_down(x).astype(np.float64)
    idx2 = np.searchsorted(grid, x.astype(np.float64), side="right") - 1
    assert np.array_equal(zd, grid[idx2])


def _bf16(x):
    """float -> nearest bf16 value (as float32), ties to even."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32)
    return (r << 16).view(np.float32)


def _random_groups(rng, n_groups, n, outlier=False):
    x = rng.standard_normal((n_groups, n)).astype(np.float32)
    if outlier:
        x[:, rng.integers(0, n)] *= 10
    return _bf16(x)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("n", [1, 2, 7, 32])
def test_half_step_bound_and_cover(bits, n):
    rng = np.random.default_rng(10 + bits * 100 + n)
    for outlier in (False, True):
        x = _random_groups(rng, 400, n, outlier)
        c, s, z = codec.quantize(x, bits, axis=-1)
        s64 = s.astype(np.float64)[:, None]
        z64 = z.astype(np.float64)[:, None]
        xh = codec.dequantize(c, s.astype(np.float64)[:, None], z64)
        err = np.abs(xh - x.astype(np.float64))
        # half a step, plus the fp32 rounding slack of the code computation
        assert np.all(err <= s64 * (0.5 + 2.0 ** -20) + 0.0)
        assert np.all(z64[:, 0] <= x.min(axis=1))
        top = codec.levels(bits)
        assert np.all(z64[:, 0] + top * s64[:, 0] >= x.max(axis=1))
        assert c.max() <= top


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_exact_nearest_grid_point(bits):
    rng = np.random.default_rng(77 + bits)
    x = _random_groups(rng, 60, 32, outlier=True)
    c, s, z = codec.quantize(x, bits, axis=-1)
    top = codec.levels(bits)
    for gi in range(x.shape[0]):
        S, Z = Fraction(float(s[gi])), Fraction(float(z[gi]))
        for xi, ci in zip(x[gi], c[gi]):
            X = Fraction(float(xi))
            if S == 0:
                assert ci == 0
                continue
            d = [abs(X - (k * S + Z)) for k in range(top + 1)]
            best = min(d)
            winners = [k for k in range(top + 1) if d[k] == best]
            if len(winners) == 1:
                # fp32 rounding of (x - z)/s can only flip a decision when the
                # exact quotient is within 2^-20 of a half-integer
                q = (X - Z) / S
                frac = q - int(q)
                if abs(frac - Fraction(1, 2)) > Fraction(1, 1 << 20):
                    assert ci == winners[0], (gi, float(xi), int(ci), winners)
            else:
                assert ci in winners and ci % 2 == 0


def test_constant_and_single_value_groups_lossless():
    rng = np.random.default_rng(5)
    vals = _bf16(rng.standard_normal(300).astype(np.float32) * 3)
    for bits in (2, 4):
        const = np.repeat(vals[:, None], 32, axis=1)
        c, s, z = codec.quantize(const, bits, axis=-1)
        xh = codec.dequantize(c, s.astype(np.float64)[:, None], z.astype(np.float64)[:, None])
        assert np.array_equal(xh, const.astype(np.float64))
        assert np.all(s == 0) and np.all(c == 0)
        one = vals[:, None]
        c1, s1, z1 = codec.quantize(one, bits, axis=-1)
        xh1 = codec.dequantize(c1, s1.astype(np.float64)[:, None], z1.astype(np.float64)[:, None])
        assert np.array_equal(xh1, one.astype(np.float64))


def test_plane_split_all_codes():
    c = np.arange(16, dtype=np.uint8)
    hi, lo = codec.split_planes(c)
    assert np.all(hi <= 3) and np.all(lo <= 3)
    assert np.array_equal(codec.join_planes(hi, lo), c)
    assert np.array_equal(hi.astype(int) * 4 + lo.astype(int), np.arange(16))


def test_pack_unpack_all_bytes():
    b = np.arange(256, dtype=np.uint8)[None, :]
    codes = codec.unpack_row(b)
    assert codes.shape == (1, 1024)
    # channel 4k + i sits at bits [2i, 2i+1] of byte k
    for k in (0, 1, 77, 255):
        for i in range(4):
            assert codes[0, 4 * k + i] == (k >> (2 * i)) & 3
    assert np.array_equal(codec.pack_row(codes), b)


def _load_codec_cases():
    cases = []
    with open(os.path.join(GOLDEN, "codec_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            bits, xs, z, s, cs = [p.strip() for p in line.split("|")]
            cases.append((int(bits), [float(v) for v in xs.split()], float(z), float(s),
                          [int(v) for v in cs.split()]))
    return cases


@pytest.mark.parametrize("case", _load_codec_cases())
def test_golden_codec_cases(case):
    bits, xs, z, s, cs = case
    x = np.asarray(xs, np.float32)
    assert np.array_equal(_bf16(x), x), "fixture inputs must be exact bf16 values"
    c, s_got, z_got = codec.quantize(x[None, :], bits, axis=-1)
    assert float(z_got[0]) == z
    assert float(s_got[0]) == s
    assert c[0].tolist() == cs
