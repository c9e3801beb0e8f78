"""Indexer logits: fp32-class MQA scores of query rows against pooled index keys.

Test infrastructure (see the package docstring).

[CPM, section 1]: each chunk's T query rows are scored against the whole
compressed prefix, output [T, max_seqlen_k] fp32, masked by the compressed
lengths. For one query row t, head h and pooled key j the score is the head's
dot product q[t,h] . k[j]; heads are combined as sum_h w[t,h] * ReLU(q[t,h] . k[j])
(per-head ReLU, per-head weights, summed), and keys past the row's compressed
length are masked to -inf.

Readings:

* Compressed length n_c(t) = floor(t / 4) + 1: the pooled block holding t is
  visible (the engine keeps a row for the pool in progress [#1732, "What this
  changes"]), so a top-k that takes every block equals dense attention.
* w[t,h] is a per-row, per-head fp32 weight with no further scale.
* Every product and sum is taken in fp64 here.
"""
from __future__ import annotations

import numpy as np


def n_compressed(t: int, pool_ratio: int = 4) -> int:
    return t // pool_ratio + 1


def indexer_logits(q: np.ndarray, w: np.ndarray, keys, positions, ld: int,
                   pool_ratio: int = 4) -> np.ndarray:
    """Logits [R, ld] (float64).

    q: [R, H, D] query values; w: [R, H] weights; keys: a sequence of R arrays,
    keys[r] holding at least min(n_c, ld) pooled keys [n, D] of row r's stream;
    positions: the absolute token position t of each row.
    Entries j >= n_c(t) are -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    R = q.shape[0]
    out = np.full((R, ld), -np.inf)
    for r in range(R):
        n = min(n_compressed(int(positions[r]), pool_ratio), ld)
        k = np.asarray(keys[r][:n], dtype=np.float64)        # [n, D]
        s = q[r] @ k.T                                        # [H, n]: per-head q . k
        out[r, :n] = (w[r][:, None] * np.maximum(s, 0.0)).sum(axis=0)
    return out
