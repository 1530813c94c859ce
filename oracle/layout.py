"""Per-entry byte layout of the caches (oracle; test infrastructure).

[facts] storage components of attn.kv_groups give, per entry:
  main KV    512 elements of 4 bits + 32 E4M3 scales  -> 256 + 32 = 288 B
  indexer K  128 elements of 4 bits + 4 E8M0 scales   ->  64 +  4 =  68 B
  SWA        512 elements of 8 bits + 16 E8M0 scales  -> 512 + 16 = 528 B
and the KV-bytes calculations give the global growth per token as the sum
over cache-owning groups of (owner layers / tokens per entry) * entry bytes.

Parity: pinned to the byte counts printed on the fact sheet (tests/golden/
layout_bytes.txt): 288, 68, 528, 890 B/token, and the uniform-BF16 figures
3,200 / 3,240 B/token and 424,673,280 B per sequence at 131,072 tokens.
"""


def fp4_e4m3_16_entry_bytes(elements):
    """Bytes of one entry in the main-KV format: E2M1 data + one E4M3 per 16."""
    assert elements % 16 == 0
    return elements // 2 + elements // 16


def mxfp4_entry_bytes(elements):
    """Bytes of one entry in MXFP4: E2M1 data + one E8M0 per 32."""
    assert elements % 32 == 0
    return elements // 2 + elements // 32


def mxfp8_entry_bytes(elements):
    """Bytes of one entry in MXFP8 (E4M3 data + one E8M0 per 32)."""
    assert elements % 32 == 0
    return elements + elements // 32


def bf16_entry_bytes(elements):
    return 2 * elements


def global_bytes_per_token(groups):
    """Global (context-growing) cache bytes per token.

    groups: iterable of (owner_layers, tokens_per_entry, entry_bytes).
    Each owner layer stores one entry per tokens_per_entry tokens.
    Returns a float (exact for the pages' groups).
    """
    return sum(layers * entry / tpe for layers, tpe, entry in groups)


def bytes_at_context(groups, windows, tokens):
    """Retained cache bytes for one sequence of `tokens` tokens.

    groups: (owner_layers, tokens_per_entry, entry_bytes) for global caches,
    each holding floor(tokens / tokens_per_entry) entries per owner layer;
    windows: (layers, window, entry_bytes) for bounded caches, each holding
    min(tokens, window) entries per layer.
    """
    g = sum(layers * entry * (tokens // tpe) for layers, tpe, entry in groups)
    w = sum(layers * entry * min(tokens, win) for layers, win, entry in windows)
    return g + w
