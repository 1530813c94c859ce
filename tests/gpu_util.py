"""Helpers shared by the GPU parity tests (not a test module)."""

import sys

import numpy as np
import pytest
import torch

gpu = pytest.mark.gpu


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import fp4_kv_cache_index_amd as csa2
    csa2.lib()  # raises if the library is missing: no fallback


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def np_(t):
    return t.detach().cpu().numpy()


def rowwise_rel_err(got, want):
    """max over rows of max|got - want| / max|want| (rows = all but the last axis)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    num = np.abs(got - want).max(axis=-1)
    den = np.abs(want).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


ATTN_TOL = 2e-3        # per (row, head): max|o - o_ref| / max|o_ref|
LSE_TOL = 2e-3         # absolute, natural log
