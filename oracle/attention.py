"""Sparse absorbed-MLA attention over the selected latent rows.

Test infrastructure (see the package docstring).

The pages fix: a sparse row reads up to 2,048 latent rows (512 blocks x 4
tokens) of a layer, and its 32 heads' absorbed queries are 32 KiB (32 x 512
bf16) [#1313, "Step 2"]; the pass reads the selected token list from the pages
[#1142, "What stays as it is"; #1313, "Step 2", "What it is not"]. In absorbed
MLA a head's query is already multiplied into the latent space, so a head's
score for token s is q_h . [c_s ; r_s] over the 512 latent and 64 rope values,
and its output is the softmax-weighted sum of the latent rows c_s (the value
up-projection is applied after this step).

Readings:

* Token set of row t: S(t) = {s <= t : floor(s / 4) in blocks(t)}. The last
  visible block may hold tokens past t; they are masked.
* z_s = scale * q_h . [c_s ; r_s]; p = softmax over S(t); out_h = sum_s p_s c_s;
  lse_h = max z + ln sum exp(z - max z). The scale is a call argument.
* FP8 rows enter as c_s = decode(code) x row scale, exactly.
* An empty S(t) gives out = 0 and lse = -inf.
* Everything in fp64, in one pass (no chunking, no merge).

Dense pass [#1142, "What stays as it is", and the kernel list of its proposal,
where the same page-table kernels read the latent "for dense chunks and the
sparse gather"]: a row attends every token it can see, with no selection. The
pages give no formula for its extent; the reading taken: the pass covers the
first ``n_blocks`` pooled blocks (4 tokens each), so row t attends
S(t) = {s : s <= t and s < 4 n_blocks}. With n_blocks >= t // 4 + 1 that is
plain causal attention over tokens 0..t; the pages' 512-key chunks and their
merge order change the rounding only, never the definition.
"""
from __future__ import annotations

import numpy as np


def selected_tokens(blocks, t: int, pool_ratio: int = 4) -> np.ndarray:
    b = np.asarray([x for x in np.asarray(blocks).ravel() if x >= 0], dtype=np.int64)
    if b.size == 0:
        return b
    s = (b[:, None] * pool_ratio + np.arange(pool_ratio)[None, :]).ravel()
    return np.sort(s[s <= t])


def sparse_mla_row(q: np.ndarray, rows, blocks, t: int, scale: float, pool_ratio: int = 4):
    """One query row.

    q: [Hq, 576] query values; rows(tokens) -> (latent [n, 512], rope [n, 64])
    gives the stream's rows at those positions (as exact values); blocks: the
    row's selected pooled blocks (-1 entries ignored); t: the row's position.
    Returns (out [Hq, 512], lse [Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    S = selected_tokens(blocks, t, pool_ratio)
    Hq = q.shape[0]
    if S.size == 0:
        return np.zeros((Hq, 512)), np.full(Hq, -np.inf)
    lat, rope = rows(S)
    lat = np.asarray(lat, dtype=np.float64)
    K = np.concatenate([lat, np.asarray(rope, dtype=np.float64)], axis=1)   # [n, 576]
    z = scale * (q @ K.T)                                                    # [Hq, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e / l) @ lat                                                      # [Hq, 512]
    lse = (m + np.log(l)).ravel()
    return out, lse


def sparse_mla(q: np.ndarray, rows_of, blocks: np.ndarray, positions, scale: float,
               pool_ratio: int = 4):
    """All rows: rows_of(r, tokens) -> (latent, rope) of row r's stream."""
    R = q.shape[0]
    outs, lses = [], []
    for r in range(R):
        o, l = sparse_mla_row(q[r], lambda S, r=r: rows_of(r, S), blocks[r],
                              int(positions[r]), scale, pool_ratio)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def dense_tokens(t: int, n_blocks: int, pool_ratio: int = 4) -> np.ndarray:
    """Tokens of the dense pass for row t: 0 .. min(t, pool_ratio n_blocks - 1)."""
    return np.arange(max(0, min(t + 1, pool_ratio * n_blocks)), dtype=np.int64)


def dense_mla_row(q: np.ndarray, rows, t: int, n_blocks: int, scale: float, pool_ratio: int = 4):
    """One query row of the dense pass: softmax attention over dense_tokens(t, n_blocks).

    Same arguments and results as sparse_mla_row, with the extent n_blocks in
    place of a block list.
    """
    q = np.asarray(q, dtype=np.float64)
    S = dense_tokens(t, n_blocks, pool_ratio)
    if S.size == 0:
        return np.zeros((q.shape[0], 512)), np.full(q.shape[0], -np.inf)
    lat, rope = rows(S)
    lat = np.asarray(lat, dtype=np.float64)
    rope = np.asarray(rope, dtype=np.float64)
    # scores over the latent and rope parts, summed
    z = scale * (q[:, :512] @ lat.T + q[:, 512:] @ rope.T)      # [Hq, n]
    zmax = z.max(axis=1)
    w = np.exp(z - zmax[:, None])
    tot = w.sum(axis=1)
    return (w @ lat) / tot[:, None], zmax + np.log(tot)


def dense_mla(q: np.ndarray, rows_of, positions, n_blocks: int, scale: float, pool_ratio: int = 4):
    """All rows of the dense pass: rows_of(r, tokens) -> (latent, rope) of row r's stream."""
    outs, lses = [], []
    for r in range(q.shape[0]):
        o, l = dense_mla_row(q[r], lambda S, r=r: rows_of(r, S), int(positions[r]), n_blocks, scale, pool_ratio)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
