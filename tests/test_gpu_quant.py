"""GPU parity of the cache writers against the oracle: bit-exact codes and scales."""

import numpy as np
import torch

import fp4_kv_cache_index_amd as csa2
from fp4_kv_cache_index_amd import inputs
from oracle import formats as F
from oracle import quant as Q
from tests.gpu_util import announce, gpu, np_, require_gpu


def _tie_rows():
    """Rows that sit on every E2M1 threshold (and their float32 neighbours) for
    every positive finite E4M3 scale, plus zero, signed-zero and extreme groups."""
    scales = F.e4m3fn_decode(np.arange(1, 127))
    ts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.99]
    rows = []
    for s in scales:
        for t in ts:
            x = np.float32(t * s)
            v = [np.float32(6 * s), x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0)),
                 -x, -np.nextafter(x, np.float32(np.inf)), np.float32(-0.0)]
            v += [np.float32(t * s * 0.5)] * (16 - len(v))
            rows.append(v)
    rows.append([0.0] * 16)
    rows.append([-0.0] * 16)
    rows.append([1e-40] * 8 + [-3e-39] * 8)           # float32 subnormals
    rows.append([3e38, -3e38] + [1.0] * 14)            # saturating scale
    rows.append([2.0 ** -12] * 16)                     # scale rounds to zero
    x = np.array(rows, dtype=np.float32)
    pad = (-x.shape[0]) % 36
    x = np.concatenate([x, np.zeros((pad, 16), np.float32)])
    return x.reshape(-1, 576)


@gpu
def test_fp4_quantize_bit_exact_tiny_config():
    require_gpu()
    wl = inputs.WORKLOADS["tiny"]
    announce("kv_fp4_quantize tiny 4096x576")
    x = inputs.shared_cache_inputs(wl, device="cuda")["kv_x"][0]
    codes, scales = csa2.kv_fp4_quantize(x)
    torch.cuda.synchronize()
    want_c, want_s = Q.fp4_quantize(np_(x))
    assert np.array_equal(np_(codes), want_c)
    assert np.array_equal(np_(scales), want_s)


@gpu
def test_fp4_quantize_ties_extremes_and_ragged_rows():
    require_gpu()
    announce("kv_fp4_quantize ties/extremes")
    x = _tie_rows()
    for n in (1, 3, x.shape[0]):
        xt = torch.tensor(x[:n], device="cuda")
        codes, scales = csa2.kv_fp4_quantize(xt)
        torch.cuda.synchronize()
        want_c, want_s = Q.fp4_quantize(x[:n])
        assert np.array_equal(np_(scales), want_s), n
        assert np.array_equal(np_(codes), want_c), n


@gpu
def test_fp4_quantize_into_interleaved_rows():
    require_gpu()
    announce("kv_fp4_quantize interleaved 324-byte rows")
    x = inputs.normal_f32((2, 1000, 576), 9, 0, "kv", device="cuda") * 3.0
    cache = torch.full((2, 1000, 324), 0xAB, dtype=torch.uint8, device="cuda")
    csa2.kv_fp4_quantize(x, codes=cache[..., :288], scales=cache[..., 288:])
    torch.cuda.synchronize()
    want_c, want_s = Q.fp4_quantize(np_(x).reshape(-1, 576))
    got = np_(cache).reshape(-1, 324)
    assert np.array_equal(got[:, :288], want_c)
    assert np.array_equal(got[:, 288:], want_s)


@gpu
def test_swa_fp8_quantize_bit_exact():
    require_gpu()
    announce("swa_fp8_quantize")
    x = inputs.normal_f32((3, 128, 576), 4, 0, "swa", device="cuda")
    mag = torch.logspace(-30, 30, 128, device="cuda").reshape(1, 128, 1)
    x = (x * mag).contiguous()
    x[0, 0, :32] = 0.0
    x[0, 1, :32] = -0.0
    x[0, 2, :] = 1e-44
    x[0, 3, 0] = 500.0
    vals, scales = csa2.swa_fp8_quantize(x)
    torch.cuda.synchronize()
    want_v, want_s = Q.mxfp8_quantize(np_(x).reshape(-1, 576))
    assert np.array_equal(np_(scales).reshape(-1, 18), want_s)
    assert np.array_equal(np_(vals).reshape(-1, 576), want_v)
