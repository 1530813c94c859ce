"""Pins for oracle.layout against the byte counts printed on the fact sheet."""

import os

from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    g = {}
    for line in open(os.path.join(GOLDEN, "layout_bytes.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            g[k] = int(v)
    return g


def test_entry_and_global_bytes():
    g = _golden()
    main = L.fp4_e4m3_16_entry_bytes(512)
    idx = L.mxfp4_entry_bytes(128)
    swa = L.mxfp8_entry_bytes(512)
    assert (main, idx, swa) == (g["main_kv_entry_bytes"], g["indexer_k_entry_bytes"], g["swa_entry_bytes"])
    # encoder: 3 owner layers, 2 tokens per entry; decoder: 1 owner layer, 1 token per entry
    groups = [(3, 2, main), (3, 2, idx), (1, 1, main), (1, 1, idx)]
    assert L.global_bytes_per_token(groups) == g["global_bytes_per_token"]


def test_bf16_payload_figures():
    g = _golden()
    b = L.bf16_entry_bytes
    groups = [(3, 2, b(512)), (3, 2, b(128)), (1, 1, b(512)), (1, 1, b(128))]
    windows = [(40, 128, b(512))]
    assert L.global_bytes_per_token(groups) == g["bf16_global_bytes_per_token"]
    total = L.bytes_at_context(groups, windows, 131072)
    assert total == g["bf16_bytes_per_sequence_131072"]
    assert total / 131072 == g["bf16_bytes_per_token_incl_swa"]
