"""Pins for oracle.quant: FP4 (E2M1 + E4M3/16) and MXFP8 (E4M3 + E8M0/32)."""

from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F
from oracle import quant as Q
from oracle import layout as L

MAGS = [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _threshold_code(absx, s):
    """Independent statement of the E2M1 rounding as thresholds on |x| / s (exact)."""
    r = Fraction(float(absx)) / Fraction(float(s))
    c = 0
    for t, code, strict in ((Fraction(1, 4), 1, True), (Fraction(3, 4), 2, False), (Fraction(5, 4), 3, True),
                            (Fraction(7, 4), 4, False), (Fraction(5, 2), 5, True), (Fraction(7, 2), 6, False),
                            (Fraction(5), 7, True)):
        if (r > t) if strict else (r >= t):
            c = code
    return c


def _pack(codes):
    codes = np.asarray(codes)
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def test_fp4_hand_example_nibble_order_and_sign():
    # Group of 16 with amax 6 -> scale = E4M3(1.0) = 0x38; values sit on the grid.
    x = np.array([6, -6, 0.5, -0.5, 1, 1.5, -2, 3, 4, -4, 0, -0.0, 0.25, -0.25, 2.5, 5], dtype=np.float32)
    codes, scales = Q.fp4_quantize(x[None, :])
    assert scales.tolist() == [[0x38]]
    # codes per channel: 6->7, -6->F, .5->1, -.5->9, 1->2, 1.5->3, -2->C, 3->5, 4->6, -4->E,
    # 0->0, -0->0, .25->0 (tie to even), -.25->0 (zero magnitude drops sign), 2.5->4 (tie), 5->6 (tie)
    want = [0xF7, 0x91, 0x32, 0x5C, 0xE6, 0x00, 0x00, 0x64]
    assert codes[0].tolist() == want


def test_fp4_exhaustive_ties_every_scale():
    scales = F.e4m3fn_decode(np.arange(1, 127))
    ts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 0.1, 5.9]
    rows = []
    for s in scales:
        amax = np.float32(6.0 * s)  # exact, so amax/6 == s exactly and the scale code is s's
        for t in ts:
            x = np.float32(t * s)
            vals = [amax, x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0)),
                    -x, -np.nextafter(x, np.float32(np.inf))]
            vals += [np.float32(0)] * (16 - len(vals))
            rows.append(vals)
    X = np.array(rows, dtype=np.float32)
    codes, sc = Q.fp4_quantize(X)
    exp_scale = np.repeat(np.arange(1, 127), len(ts)).astype(np.uint8)
    assert np.array_equal(sc[:, 0], exp_scale)
    s_rows = np.repeat(scales, len(ts))
    for i in range(X.shape[0]):
        want = []
        for v in X[i]:
            m = _threshold_code(abs(v), s_rows[i])
            want.append(m | (8 if (v < 0 and m != 0) else 0))
        assert codes[i].tolist() == _pack(want).tolist(), (i, X[i], s_rows[i])


def test_fp4_scale_rule_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((512, 64)) * np.exp2(rng.integers(-14, 10, (512, 1)))).astype(np.float32)
    _, sc = Q.fp4_quantize(x)
    amax = np.abs(x.reshape(512, 4, 16)).max(-1)
    q = (amax / np.float32(6)).astype(np.float32)
    want = torch.tensor(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(sc, want)


def test_fp4_zero_group_and_roundtrip_and_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 576)).astype(np.float32)
    x[0, :16] = 0
    x[1, 16:32] = -0.0
    codes, sc = Q.fp4_quantize(x)
    assert sc[0, 0] == 0 and np.all(codes[0, :8] == 0)
    assert sc[1, 1] == 0 and np.all(codes[1, 8:16] == 0)
    y = Q.fp4_dequantize(codes, sc, 576)
    s = np.repeat(F.e4m3fn_decode(sc), 16, axis=1)
    r = np.abs(x) / np.where(s > 0, s, 1)
    gap = np.where(r <= 2, 0.5, np.where(r <= 4, 1.0, 2.0))
    ok = (r <= 6) & (s > 0)
    assert np.all(np.abs(y - x)[ok] <= (gap * s / 2)[ok] * (1 + 1e-12))
    # Dequantised values are fixed points of the quantiser (grid round-trip).
    codes2, sc2 = Q.fp4_quantize(y.astype(np.float32))
    y2 = Q.fp4_dequantize(codes2, sc2, 576)
    assert np.array_equal(y2, y)
    # Row layout: 576 channels -> 288 code bytes + 36 scale bytes.
    assert codes.shape == (300, 288) and sc.shape == (300, 36)
    assert codes.shape[1] + sc.shape[1] == L.fp4_e4m3_16_entry_bytes(576)


def test_mxfp8_exponent_closed_form_and_roundtrip():
    # amax = 2^k exactly -> shared exponent k - 8, element value 2^8 = 256.
    for k in range(-100, 100, 7):
        x = np.zeros((1, 32), np.float32)
        x[0, 3] = np.float32(2.0 ** k)
        v, s = Q.mxfp8_quantize(x)
        assert s[0, 0] == k - 8 + 127
        assert F.e4m3fn_decode(v[0, 3]) == 256.0
    z = np.zeros((1, 32), np.float32)
    v, s = Q.mxfp8_quantize(z)
    assert s[0, 0] == 127 and np.all(v == 0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 576)).astype(np.float32)
    v, s = Q.mxfp8_quantize(x)
    y = Q.mxfp8_dequantize(v, s, 576)
    # E4M3 keeps 4 significant bits: relative error <= 2^-4 for normal elements,
    # absolute error <= half the subnormal step (2^-10 * scale) below them.
    sc = np.repeat(F.e8m0_decode(s), 32, axis=1)
    err = np.abs(y - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * sc)
    sat = np.abs(x) > 448 * sc  # top of the binade saturates to 448 * scale
    assert np.all(err[~sat] <= bound[~sat] * (1 + 1e-12))
    assert np.array_equal(err[sat], np.abs(x)[sat] - 448 * sc[sat])
    # The largest element of each group lands in [256, 448].
    g = np.abs(F.e4m3fn_decode(v)).reshape(200, 18, 32).max(-1)
    assert np.all((g >= 256) & (g <= 448))
    assert v.shape[1] + s.shape[1] == L.mxfp8_entry_bytes(576)


def test_mxfp8_saturates_top_of_binade():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.float32(500.0)  # floor(log2) = 8 -> exponent 0 -> 500 saturates to 448
    v, s = Q.mxfp8_quantize(x)
    assert s[0, 0] == 127 and v[0, 0] == 0x7E


def test_fp4_huge_and_tiny_groups():
    # amax/6 saturates the scale at 448; the huge elements saturate to +-6.
    x = np.array([[3e38, -3e38] + [1.0] * 14], dtype=np.float32)
    codes, sc = Q.fp4_quantize(x)
    assert sc.tolist() == [[0x7E]]
    assert codes[0].tolist() == [0xF7] + [0] * 7
    # float32 subnormals and values whose scale rounds to zero give all-zero codes.
    x = np.array([[1e-40] * 8 + [-3e-39] * 8, [2.0 ** -12] * 16], dtype=np.float32)
    codes, sc = Q.fp4_quantize(x)
    assert sc.tolist() == [[0], [0]] and np.all(codes == 0)


def test_mxfp4_shared_exponent_and_ties_at_several_exponents():
    """MXFP4 (OCP MX): shared exponent floor(log2 amax) - 2; elements rounded to
    the nearest E2M1 magnitude of x / 2^X, ties to the even code, saturating at 6
    -- checked with the exact-rational threshold statement on every tie and its
    float32 neighbours, at shared exponents -6 .. 6."""
    ts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 0.1, 5.9, 6.0, 7.5]
    rows, Xs = [], []
    for X in range(-6, 7):
        s = 2.0 ** X
        amax = np.float32(7.9 * s)          # floor(log2(7.9 * 2^X)) = X + 2
        for t in ts:
            x = np.float32(t * s)
            vals = [amax, x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0)), -x,
                    -np.nextafter(x, np.float32(np.inf))]
            vals += [np.float32(0)] * (32 - len(vals))
            rows.append(vals)
            Xs.append(X)
    Xa = np.array(rows, dtype=np.float32)
    codes, sc = Q.mxfp4_quantize(Xa)
    assert np.array_equal(sc[:, 0], np.array(Xs) + 127)
    for i in range(Xa.shape[0]):
        s = 2.0 ** Xs[i]
        got = np.empty(32, np.int64)
        got[0::2], got[1::2] = codes[i] & 0xF, codes[i] >> 4
        for j in range(32):
            v = float(Xa[i, j])
            want = _threshold_code(abs(v), s)
            if v < 0 and want:
                want |= 8
            assert got[j] == want, (Xs[i], v, got[j], want)


def test_mxfp4_zero_group_round_trip_and_entry_bytes():
    x = np.zeros((1, 128), np.float32)
    c, s = Q.mxfp4_quantize(x)
    assert s.tolist() == [[127] * 4] and not c.any()
    # grid points of four different exponents round-trip exactly
    rng = np.random.default_rng(0)
    grid = np.array(MAGS, np.float64)
    y = np.empty((3, 128))
    for r in range(3):
        for blk in range(4):
            X = int(rng.integers(-4, 5))
            vals = rng.choice(grid, 32) * rng.choice([-1, 1], 32) * 2.0 ** X
            vals[0] = 6 * 2.0 ** X                  # sets the block's exponent to X
            y[r, 32 * blk: 32 * blk + 32] = vals
    c, s = Q.mxfp4_quantize(y.astype(np.float32))
    assert c.shape == (3, 64) and s.shape == (3, 4)     # 64 code bytes + 4 scale bytes = 68 per entry
    assert np.array_equal(Q.mxfp4_dequantize(c, s, 128), y)
    # the shared exponent's closed form on powers of two, clamped to the E8M0 range
    amax = np.array([2.0 ** e for e in (-140, -130, -3, 0, 1, 2, 5, 127)], np.float32)
    want = np.clip(np.array([-140, -130, -3, 0, 1, 2, 5, 127]) - 2 + 127, 0, 254)
    assert np.array_equal(Q.mxfp4_shared_exponent_code(amax), want)
