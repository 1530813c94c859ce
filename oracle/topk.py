"""Exact Top-K token selection (oracle; test infrastructure).

[map] "Checked in its code", row "Indexer-selected sparse attention": the
attention of a query is restricted to the k highest-scoring cached entries of
the indexer; [facts] token selection: k = 512 (the measured workloads use
2048 and 256).

Readings (the pages give no tie rule, output order or short-context rule):
  * total order: score descending, then token index ascending, comparing
    scores as real numbers (so -0 and +0 tie);
  * keep the first min(K, visible) tokens of that order;
  * emit them sorted by token index ascending, padded with -1 to K; the
    optional scores are aligned with the emitted indices (-inf for padding).

Parity: pinned against a pure-Python sort on tiny inputs, and by the special
cases all-ties -> 0..K-1, K >= visible -> all visible tokens, K = 1 -> the
lowest-index maximum (tests/test_oracle_topk.py).
"""

import numpy as np


def topk_select(scores, n_visible, k, ids=None):
    """Select the top-k of scores[:n_visible] (ties -> lower id).

    ids: optional tie-break / output ids for each position (default 0..N-1),
    which must be ascending.  Returns (idx int32 [k], sel_scores float32 [k]).
    """
    scores = np.asarray(scores, dtype=np.float32)
    nv = max(0, min(int(n_visible), scores.shape[0]))
    if ids is None:
        ids = np.arange(scores.shape[0], dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    s = scores[:nv].astype(np.float64)
    order = np.lexsort((ids[:nv], -s))  # primary: -score ascending; secondary: id ascending
    take = order[: min(k, nv)]
    take = take[np.argsort(ids[take], kind="stable")]
    out = np.full(k, -1, dtype=np.int32)
    out_s = np.full(k, -np.inf, dtype=np.float32)
    out[: len(take)] = ids[take]
    out_s[: len(take)] = scores[take]
    return out, out_s
