"""Pins for oracle.formats: decode tables and the E4M3 encoder."""

import os
from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_decode_matches_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt")) if l.strip() and not l.startswith("#")]
    codes = np.array([int(r[0]) for r in rows])
    vals = np.array([float(r[1]) for r in rows])
    got = F.e2m1_decode(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))


def test_e4m3_decode_matches_torch_all_256():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3fn_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert F.E4M3_MAX == 448.0


def test_e8m0_decode_closed_form():
    b = np.arange(255)
    assert np.array_equal(F.e8m0_decode(b), np.ldexp(1.0, b - 127))
    assert np.isnan(F.e8m0_decode(255))


def _torch_e4m3(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_rne_in_range():
    vals = F.e4m3fn_decode(np.arange(127))  # non-negative finite
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [464.0]]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000))).astype(np.float32)
    x = np.concatenate([pts, up, dn, rnd, [0.0]]).astype(np.float32)
    x = x[np.abs(x) <= 464.0]
    x = np.concatenate([x, -x])
    assert np.array_equal(F.e4m3fn_encode(x), _torch_e4m3(x))


def test_e4m3_encode_saturates():
    x = np.array([464.0001, 480, 1e6, 3.0e38], dtype=np.float32)
    assert np.all(F.e4m3fn_encode(x) == 0x7E)
    assert np.all(F.e4m3fn_encode(-x) == 0xFE)


def test_e4m3_encode_small_values():
    # Half the smallest subnormal (2^-10) ties to zero; just above rounds up.
    assert F.e4m3fn_encode(2.0 ** -10) == 0
    assert F.e4m3fn_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 1
    assert F.e4m3fn_encode(3 * 2.0 ** -10) == 2  # 1.5 * 2^-9 ties to even mantissa 2
    assert F.e4m3fn_encode(0.0) == 0


def _nearest_e2m1_exact(absx, s):
    """Exact rational nearest E2M1 magnitude code, ties to even code, saturating."""
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    r = Fraction(absx) / Fraction(s)
    best = None
    for c, m in enumerate(mags):
        d = abs(r - m)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e2m1_nearest_code_exact_on_ties_and_neighbours():
    scales = F.e4m3fn_decode(np.arange(1, 127))  # every positive finite E4M3 scale
    ts = [0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6.5, 7]
    xs, ss = [], []
    for s in scales:
        for t in ts:
            x = np.float32(t * s)
            for v in (x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))):
                xs.append(float(v))
                ss.append(float(s))
    got = F.e2m1_nearest_code(np.array(xs), np.array(ss))
    want = np.array([_nearest_e2m1_exact(x, s) for x, s in zip(xs, ss)])
    assert np.array_equal(got, want)


def test_e2m1_nearest_code_saturates_huge_quotients():
    # Quotients far beyond 6 (where float64 distances to every candidate round
    # to the same value) must still pick 6.0, the nearest magnitude.
    scales = F.e4m3fn_decode(np.array([1, 8, 0x38, 0x7E]))
    xs = np.array([3e38, 1e30, 6.5e10, 1e8], dtype=np.float32)
    for s in scales:
        for x in xs:
            assert F.e2m1_nearest_code(np.array([x]), np.array([s]))[0] == _nearest_e2m1_exact(float(x), float(s)) == 7
