"""Top-k pooled blocks of each row's logits.

Test infrastructure (see the package docstring).

[CPM, sections 1 and 2.3]: per row, select the k highest-scoring pooled blocks
among the row's own visible keys (rows are ragged: each has its own length),
e.g. the top-512. Section 2.3 states that taking the top-k of per-block top-k
candidates gives exactly the top-k of the whole row.

Readings: ties go to the lower block index; -0 equals +0; a row with fewer
visible blocks than k takes all of them and pads with -1; the output of a row is
its selected block ids in ascending order (the selection is a set).

Two-level candidate selection [CPM, section 1: the layer that publishes
candidate masks for the later low-ratio layers; section 2.3: its block pooling
over 8-key groups and top-2,048 groups, and the consumers' masking of
non-candidates before their own top-k]. The pages name the steps, not the
pooling operator or the masked value. Readings taken:

* a group of g consecutive keys (g = 8) scores the largest logit among its
  visible keys; the last group may be partial; a group with no visible key is
  not visible;
* candidates = the top-n_cand groups by that score (the rule above, on groups);
* a consumer row keeps the logits of keys in its candidate groups, sets the
  others to -inf (masked_fill_), and takes its top-k of the result with the rule
  above over its visible keys, so fewer than k candidate keys are completed by
  the lowest-index non-candidates.
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


def group_max(vals: np.ndarray, n_valid: int, g: int) -> np.ndarray:
    """Score of each visible group of g keys: the largest of its visible logits."""
    v = np.asarray(vals[:n_valid], dtype=np.float64)
    n_groups = -(-v.size // g)
    return np.array([v[j * g:(j + 1) * g].max() for j in range(n_groups)], dtype=np.float64)


def candidate_groups(logits: np.ndarray, n_valid, g: int, n_cand: int) -> np.ndarray:
    """[R, n_cand]: each row's top-n_cand groups of g keys, ascending, -1 padded."""
    logits = np.asarray(logits)
    out = []
    for r in range(logits.shape[0]):
        s = group_max(logits[r], int(n_valid[r]), g)
        out.append(topk_row(s, s.size, n_cand))
    return np.stack(out) if out else np.zeros((0, n_cand), dtype=np.int64)


def topk_in_candidates(logits: np.ndarray, n_valid, cand: np.ndarray, g: int, k: int) -> np.ndarray:
    """[R, k]: each row's top-k keys after the keys outside its candidate groups are
    set to -inf."""
    logits = np.asarray(logits)
    out = []
    for r in range(logits.shape[0]):
        nv = int(n_valid[r])
        keep = np.zeros(nv, dtype=bool)
        for c in np.asarray(cand[r]):
            if c >= 0:
                keep[c * g:(c + 1) * g] = True
        masked = np.where(keep, np.asarray(logits[r][:nv], dtype=np.float64), -np.inf)
        out.append(topk_row(masked, nv, k))
    return np.stack(out) if out else np.zeros((0, k), dtype=np.int64)
