"""Pins for the oracle's element formats (E2M1, E4M3): spec tables, a
library cast, independent formulas and brute force.  CPU only."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode


# ---------------------------------------------------------------- decoders

def test_e2m1_decode_matches_spec_table(golden):
    rows = golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = e2m1_decode(int(code))
        assert got == float(val)
        assert np.signbit(got) == val.startswith("-")


def test_e4m3_decode_landmarks(golden):
    for byte, val in golden("e4m3_landmarks.txt"):
        got = float(e4m3_decode(int(byte, 16)))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_e4m3_decode_all_256_vs_torch_cast():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = b.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    ours = e4m3_decode(np.arange(256))
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(lib[~nan], ours[~nan])
    assert np.array_equal(np.signbit(lib[~nan]), np.signbit(ours[~nan]))


def test_e4m3_grid_is_monotone():
    g = e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(g) > 0) and g[0] == 0 and g[-1] == 448.0


# ---------------------------------------------------- independent encoders

def _e2m1_formula(y):
    """Round-half-even on the E2M1 grid written as exponent/mantissa
    arithmetic (1 mantissa bit, subnormal spacing 0.5), saturating at 6."""
    a = min(abs(float(y)), 6.0)
    if a < 1.0:
        v = float(np.rint(a / 0.5)) * 0.5
    else:
        e = int(np.floor(np.log2(a)))
        q = float(np.rint(a / 2.0 ** e * 2.0)) / 2.0
        v = min(q * 2.0 ** e, 6.0)
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    return mags.index(v) | (8 if np.signbit(y) else 0)


def _brute_nearest_even(v, grid):
    """Exact nearest grid index by rational distances; ties to even index."""
    fv = Fraction(float(v))
    d = [abs(fv - Fraction(float(g))) for g in grid]
    best = min(d)
    cands = [i for i, di in enumerate(d) if di == best]
    even = [i for i in cands if i % 2 == 0]
    return even[0] if even else cands[0]


def _e4m3_formula(s):
    """Round-half-even onto E4M3 (3 mantissa bits, bias 7, subnormal
    spacing 2^-9 below 2^-6), saturating at 448, via exponent arithmetic."""
    s = min(float(s), 448.0)
    if s < 2.0 ** -6:
        m = int(np.rint(s * 512.0))
        return m                         # m == 8 is the smallest normal, 0x08
    e = int(np.floor(np.log2(s)))
    q = int(np.rint((s / 2.0 ** e - 1.0) * 8.0))
    if q == 8:
        e, q = e + 1, 0
    b = ((e + 7) << 3) | q
    return min(b, 0x7E)


def test_e2m1_threshold_table(golden):
    for y, code in golden("e2m1_rounding.txt"):
        yf = np.float32(float(y))
        assert int(e2m1_encode(yf)) == int(code), y
        assert int(e2m1_encode(-yf)) == int(code) | 8, y


def test_e2m1_ties_and_neighbours_three_ways():
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    pts = []
    for a, b in zip(grid[:-1], grid[1:]):
        m = np.float32((a + b) / 2)
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(10))]
    pts += [np.float32(v) for v in grid] + [np.float32(6.5), np.float32(1e30)]
    for y in pts:
        want = _brute_nearest_even(min(float(y), 6.0), grid)
        assert int(e2m1_encode(y)) == want == _e2m1_formula(y), y
        assert int(e2m1_encode(-y)) == want | 8


def test_e2m1_dense_sweep_vs_formula():
    rng = np.random.default_rng(11)
    y = np.concatenate([
        np.linspace(0, 8, 200001, dtype=np.float32),
        rng.uniform(-8, 8, 20000).astype(np.float32),
    ])
    ours = e2m1_encode(y)
    ref = np.array([_e2m1_formula(v) for v in y], dtype=np.uint8)
    assert np.array_equal(ours, ref)


def test_e2m1_sign_of_zero_and_underflow():
    assert int(e2m1_encode(np.float32(0.0))) == 0
    assert int(e2m1_encode(np.float32(-0.0))) == 8
    assert int(e2m1_encode(np.float32(-0.2))) == 8
    assert int(e2m1_encode(np.float32(-1e-30))) == 8
    assert int(e2m1_encode(np.float32(-100.0))) == 15


def test_e4m3_ties_and_neighbours_three_ways():
    grid = e4m3_decode(np.arange(0x7F))
    pts = []
    for a, b in zip(grid[:-1], grid[1:]):
        m = np.float32((a + b) / 2)
        assert float(m) == (a + b) / 2          # every midpoint is binary32-exact
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    pts += [np.float32(v) for v in grid]
    pts = np.array(pts, dtype=np.float32)
    ours = e4m3_encode(pts)
    for v, b in zip(pts, ours):
        want = _brute_nearest_even(v, grid)
        assert int(b) == want == _e4m3_formula(v), float(v)


def test_e4m3_saturation():
    v = np.array([448.0, 448.5, 463.99, 464.0, 464.01, 480.0, 1e5, 3e38], np.float32)
    assert np.all(e4m3_encode(v) == 0x7E)


def test_e4m3_rejects_negative_and_nonfinite():
    for bad in (-1.0, np.inf, np.nan):
        with pytest.raises(ValueError):
            e4m3_encode(np.float32(bad))


def test_e4m3_encode_dense_sweep_vs_torch_cast():
    """Every binary32 value in [2^-12, 448] (about 1.8e8 values, one binade
    at a time) against torch's float8_e4m3fn cast, a library routine that
    rounds to nearest even.  Below 2^-12 a strided sample is used."""
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(448.0).view(np.uint32)
    step = 1 << 23
    for start in range(int(lo), int(hi) + 1, step):
        u = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        s = u.view(np.float32)
        lib = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ours = e4m3_encode(s)
        bad = np.nonzero(lib != ours)[0]
        assert bad.size == 0, (float(s[bad[0]]), int(lib[bad[0]]), int(ours[bad[0]]))
    tiny = np.arange(0, int(lo), 4099, dtype=np.uint32).view(np.float32)
    lib = torch.from_numpy(tiny).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(lib, e4m3_encode(tiny))
