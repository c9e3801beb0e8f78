"""Top-k pooled blocks of each row's logits.

Test infrastructure (see the package docstring).

[CPM, sections 1 and 2.3]: per row, select the k highest-scoring pooled blocks
among the row's own visible keys (rows are ragged: each has its own length),
e.g. the top-512. Section 2.3 states that taking the top-k of per-block top-k
candidates gives exactly the top-k of the whole row.

Readings: ties go to the lower block index; -0 equals +0; a row with fewer
visible blocks than k takes all of them and pads with -1; the output of a row is
its selected block ids in ascending order (the selection is a set).
"""
from __future__ import annotations

import numpy as np


def topk_row(vals: np.ndarray, n_valid: int, k: int) -> np.ndarray:
    v = np.asarray(vals[:n_valid], dtype=np.float64) + 0.0   # -0 -> +0
    idx = np.arange(v.size)
    order = np.lexsort((idx, -v))                            # by (-value, index)
    sel = np.sort(order[:min(k, v.size)])
    out = np.full(k, -1, dtype=np.int64)
    out[:sel.size] = sel
    return out


def topk_blocks(logits: np.ndarray, n_valid, k: int) -> np.ndarray:
    """[R, k] int64: ascending selected block ids, -1 padded."""
    logits = np.asarray(logits)
    R = logits.shape[0]
    return np.stack([topk_row(logits[r], int(n_valid[r]), k) for r in range(R)]) \
        if R else np.zeros((0, k), dtype=np.int64)
