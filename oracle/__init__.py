"""CPU oracle for the CSA2 decode/prefill hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
NumPy restatement of what the path computes: float64 wherever the sources do
not fix a precision, exact integer arithmetic where they do.  It shares no
code with the HIP library and imports nothing from it.  Only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never calls it.

Sources (cited by page title and section):
  [blog]  "DeepSeek-V4.1" technical blog, Introduction > DeepSeek-V4.1-Flash,
          paragraph "Compressed Sparse Attention 2 (CSA2)".
  [map]   "DeepSeek-V4.1-Flash" model techniques map, table "Checked in its
          code" (rows: indexer-selected sparse attention, learnable attention
          sink, partial RoPE, sliding-window attention) and the technique tree
          (KV cache management, inference quantization, unfiled).
  [facts] "DeepSeek-V4.1-Flash" architecture fact sheet: attention facts
          (token selection, sink, cross-layer KV sharing), the storage
          components of attn.kv_groups, and the KV-bytes calculations.
  [atlas] "DeepSeek-V4.1" training atlas, OPD stage card, "Architecture at
          this stage".
  [OCP]   OCP Microscaling Formats (MX) v1.0 specification (public standard)
          for the bit-level definitions of E2M1, E4M3 (FN) and E8M0.

Parity status per function is listed in each module header.
"""

from . import formats, layout, quant, indexer, topk, pool, attention  # noqa: F401
