"""Bit-level number formats used by the caches (oracle; test infrastructure).

The main KV cache stores E2M1 values with one E4M3 scale per 16 channels
([blog] CSA2 paragraph; [facts] storage components, main KV group).  The
sliding-window cache stores E4M3 values with one E8M0 scale per 32 channels
([facts] storage components, SWA window group; [atlas] number format).
The pages name the formats only; their bit layouts are those of the OCP MX
v1.0 specification:

  E2M1   1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0 is
         subnormal (value = mantissa * 0.5).  No inf/NaN.
  E4M3FN 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 is
         subnormal (value = mantissa/8 * 2^-6).  S.1111.111 is NaN; no inf.
         Largest finite magnitude 448.
  E8M0   8-bit unsigned exponent, value 2^(e-127); 0xFF is NaN.

Encoders are defined as "nearest representable value, ties to the code with
an even mantissa LSB, saturating at the largest finite value": written out
as a search over the decoded table, with no bit tricks.

Parity: pinned by exhaustive decode tables against the OCP definitions and
against torch.float8_e4m3fn (an independent implementation), and the E4M3
encoder against torch's RNE cast on every representable value, every
midpoint and their float32 neighbours (tests/test_oracle_formats.py).
"""

import numpy as np


def e2m1_decode(code):
    """Decode 4-bit E2M1 codes (array of ints 0..15) to float64."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.power(2.0, e - 1))
    return sign * mag


def e4m3fn_decode(byte):
    """Decode E4M3FN bytes (array of ints 0..255) to float64 (NaN for 0x7F/0xFF)."""
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e8m0_decode(byte):
    """Decode E8M0 scale bytes to float64 powers of two (NaN for 0xFF)."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.power(2.0, b.astype(np.float64) - 127.0))


# Non-negative finite E4M3FN values, indexed by their 7-bit magnitude code.
_E4M3_POS = e4m3fn_decode(np.arange(0, 127))
E4M3_MAX = float(_E4M3_POS[-1])  # 448


def e4m3fn_encode(x):
    """Encode float values to E4M3FN bytes: nearest value, ties to even code, saturating.

    Magnitudes above 448 saturate to 448 (code 0x7E); the sign is kept except
    that a magnitude rounding to zero keeps the sign of x (torch agrees).
    NaN inputs are out of contract.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # Index of the first table value >= a (clamped into the table).
    hi = np.searchsorted(_E4M3_POS, a, side="left")
    hi = np.clip(hi, 0, len(_E4M3_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_E4M3_POS) - 1)
    d_hi = np.abs(_E4M3_POS[hi] - a)
    d_lo = np.abs(a - _E4M3_POS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a >= E4M3_MAX, 126, code)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def e2m1_nearest_code(absx, scale):
    """Magnitude code (0..7) of the E2M1 value v minimising |absx - v*scale|.

    This is the E2M1 value nearest the real quotient absx/scale, found without
    forming the quotient.  A quotient above 6 saturates to code 7 (6.0); that
    test, absx > 6*scale, is exact.  Below it absx <= 6*scale, v*scale is
    exact in float64 (at most 6 significant bits) and absx is a float32, so
    the distances are exact whenever absx is within 2^28 of the candidates,
    which covers every case where two candidates come close to tying; ties go
    to the even code.  scale must be > 0.
    """
    a = np.asarray(absx, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    a, s = np.broadcast_arrays(a, s)
    sat = a > 6.0 * s
    a = np.where(sat, 6.0 * s, a)
    mags = e2m1_decode(np.arange(8))
    dist = np.abs(a[..., None] - mags * s[..., None])  # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    # Among equally near codes prefer the even one (a tie involves two
    # neighbouring codes, exactly one of which is even).
    even = (np.arange(8) % 2 == 0)
    pick_even = cand & even
    has_even = pick_even.any(axis=-1, keepdims=True)
    cand = np.where(has_even, pick_even, cand)
    return np.where(sat, 7, np.argmax(cand, axis=-1)).astype(np.int64)
