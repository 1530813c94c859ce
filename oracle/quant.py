"""Cache quantisers (oracle; test infrastructure).

fp4_quantize -- main KV write.  [blog] CSA2 paragraph: FP4 main KV in E2M1
with one E4M3 scale per 16 channels; [facts] main KV group: 256 data bytes
followed by 32 scale bytes per 512-element entry; [map] technique tree,
inference quantization: the cache is quantised after RoPE, so every channel
of the row (RoPE channels included) goes through the same quantiser.

The pages give no scale or rounding rule.  Reading taken here (the plainest
one the format admits):
  amax  = max |x| over the 16-channel group (float32);
  scale = E4M3 nearest to float32(amax / 6) (RNE, saturating at 448), so the
          largest element maps near the top E2M1 magnitude 6;
  code  = E2M1 value nearest the exact quotient |x| / scale, ties to the even
          code, saturating at 6; a zero scale gives all-zero codes;
  sign  = sign of x, except that a zero magnitude is stored as +0 (0x0).
Packing: channel 2i in the low nibble of byte i, channel 2i+1 in the high
nibble (OCP MX convention).

mxfp8_quantize -- sliding-window cache write ([facts] SWA window group: FP8
E4M3 data with one E8M0 scale per 32 channels, 512 + 16 bytes; [atlas]: the
sliding-window cache stays FP8).  No rule on the pages; reading: the OCP MX
v1.0 conversion -- shared exponent floor(log2(amax)) - 8 (8 = largest E4M3
exponent), clamped to the E8M0 range, code 127 for an all-zero group;
elements are E4M3 RNE-with-saturation of x / 2^shared_exp.

mxfp4_quantize -- indexer K write ([facts] indexer K groups: MXFP4, E2M1
values with one E8M0 scale per 32 channels, 64 + 4 = 68 bytes per 128-channel
entry).  No rule on the pages; reading: the OCP MX v1.0 conversion -- shared
exponent floor(log2(amax)) - 2 (2 = largest E2M1 exponent), clamped to the
E8M0 range, code 127 for an all-zero group; elements are the E2M1 value
nearest x / 2^shared_exp, ties to the even code, saturating at 6 (the same
nearest-value rule as fp4_quantize, with the power-of-two scale).

Parity: fp4_quantize pinned by an exhaustive tie/threshold sweep over all 126
positive finite scales written with exact rational arithmetic, by round-trip
of grid points and by the error bound of half a grid gap; mxfp8_quantize by
the closed-form exponent on powers of two and by round-trip; mxfp4_quantize by
an exact-rational nearest-value sweep on ties and neighbours of every
threshold at several shared exponents, the exponent closed form and
round-trip (tests/test_oracle_quant.py).
"""

import numpy as np

from .formats import e2m1_decode, e2m1_nearest_code, e4m3fn_decode, e4m3fn_encode, e8m0_decode


def fp4_scale_code(amax_f32):
    """E4M3 scale byte for a group whose float32 amax is given."""
    amax = np.asarray(amax_f32, dtype=np.float32)
    q = (amax / np.float32(6.0)).astype(np.float32)  # IEEE float32 division
    return e4m3fn_encode(q.astype(np.float64))


def fp4_quantize(x):
    """Quantise float32 rows [rows][d] to (codes [rows][d/2] u8, scales [rows][d/16] u8)."""
    x = np.asarray(x, dtype=np.float32)
    rows, d = x.shape
    assert d % 16 == 0
    g = x.reshape(rows, d // 16, 16)
    amax = np.abs(g).max(axis=-1)  # float32
    scode = fp4_scale_code(amax)  # [rows][d/16]
    s = e4m3fn_decode(scode)  # float64, exact
    absx = np.abs(g).astype(np.float64)
    s_b = np.broadcast_to(s[..., None], absx.shape)
    safe_s = np.where(s_b > 0, s_b, 1.0)
    mag = e2m1_nearest_code(absx, safe_s)
    mag = np.where(s_b > 0, mag, 0)
    neg = (g < 0) & (mag != 0)
    code = (mag | (neg.astype(np.int64) << 3)).reshape(rows, d)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scode.astype(np.uint8)


def fp4_dequantize(codes, scales, d):
    """Decode packed E2M1 codes and E4M3 scales to float64 rows [rows][d]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    lo = codes[:, : d // 2] & 0xF
    hi = codes[:, : d // 2] >> 4
    c = np.empty((rows, d), dtype=np.int64)
    c[:, 0::2] = lo
    c[:, 1::2] = hi
    v = e2m1_decode(c).reshape(rows, d // 16, 16)
    s = e4m3fn_decode(scales[:, : d // 16])
    return (v * s[..., None]).reshape(rows, d)


def mxfp8_shared_exponent_code(amax_f32):
    """E8M0 scale byte for a 32-channel group of float32 amax."""
    amax = np.asarray(amax_f32, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    _, ex = np.frexp(safe)  # safe = m * 2^ex with m in [0.5, 1): floor(log2) = ex - 1
    e = (ex - 1) - 8
    code = np.clip(e + 127, 0, 254)
    return np.where(amax > 0, code, 127).astype(np.uint8)


def mxfp8_quantize(x):
    """Quantise float32 rows [rows][d] to (values [rows][d] u8 E4M3, scales [rows][d/32] u8 E8M0)."""
    x = np.asarray(x, dtype=np.float32)
    rows, d = x.shape
    assert d % 32 == 0
    g = x.reshape(rows, d // 32, 32)
    amax = np.abs(g).max(axis=-1)
    scode = mxfp8_shared_exponent_code(amax)
    scale = e8m0_decode(scode)  # exact power of two
    vals = e4m3fn_encode(g.astype(np.float64) / scale[..., None]).reshape(rows, d)
    return vals, scode


def mxfp8_dequantize(vals, scales, d):
    """Decode E4M3 values with E8M0 per-32 scales to float64 rows [rows][d]."""
    vals = np.asarray(vals, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows = vals.shape[0]
    v = e4m3fn_decode(vals[:, :d]).reshape(rows, d // 32, 32)
    s = e8m0_decode(scales[:, : d // 32])
    return (v * s[..., None]).reshape(rows, d)


def mxfp4_shared_exponent_code(amax_f32):
    """E8M0 scale byte of a 32-channel group for E2M1 elements."""
    amax = np.asarray(amax_f32, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    _, ex = np.frexp(safe)  # floor(log2(amax)) = ex - 1
    e = (ex - 1) - 2
    code = np.clip(e + 127, 0, 254)
    return np.where(amax > 0, code, 127).astype(np.uint8)


def mxfp4_quantize(x):
    """Quantise float32 rows [rows][d] to (codes [rows][d/2] u8 packed E2M1, scales [rows][d/32] u8 E8M0)."""
    x = np.asarray(x, dtype=np.float32)
    rows, d = x.shape
    assert d % 32 == 0
    g = x.reshape(rows, d // 32, 32)
    amax = np.abs(g).max(axis=-1)
    scode = mxfp4_shared_exponent_code(amax)
    s = e8m0_decode(scode)  # exact power of two
    absx = np.abs(g).astype(np.float64)
    mag = e2m1_nearest_code(absx, np.broadcast_to(s[..., None], absx.shape))
    neg = (g < 0) & (mag != 0)
    code = (mag | (neg.astype(np.int64) << 3)).reshape(rows, d)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scode


def mxfp4_dequantize(codes, scales, d):
    """Decode packed E2M1 codes with E8M0 per-32 scales to float64 rows [rows][d]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    c = np.empty((rows, d), dtype=np.int64)
    c[:, 0::2] = codes[:, : d // 2] & 0xF
    c[:, 1::2] = codes[:, : d // 2] >> 4
    v = e2m1_decode(c).reshape(rows, d // 32, 32)
    return (v * e8m0_decode(scales[:, : d // 32])[..., None]).reshape(rows, d)
