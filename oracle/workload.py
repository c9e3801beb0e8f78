"""The oracle evaluated on a synthetic workload (``synth.configs``).

Test infrastructure (see the package docstring). Inputs come only from the seeded
generator; the rows are the logical rows of each stream (no pool, no page table),
so a GPU result read through a page table is compared with what the rows
themselves define.
"""
from __future__ import annotations

import numpy as np

from synth import bf16_to_f64

from .attention import dense_mla, sparse_mla
from .fp8 import e4m3_decode
from .indexer import indexer_logits, n_compressed
from .topk import topk_blocks


def rows_reader(wl, c: int, b: int):
    """S -> (latent [n, 512], rope [n, 64]) exact values of stream b's rows in cache c."""
    def rows(S):
        S = np.asarray(S, dtype=np.int64)
        if wl.fp8:
            codes, scales, rope = wl.latent_fp8(c, b, S)
            lat = e4m3_decode(codes) * scales.astype(np.float64)[:, None]
            return lat, bf16_to_f64(rope)
        v = bf16_to_f64(wl.latent_bits(c, b, S))
        return v[:, :512], v[:, 512:]
    return rows


def keys_of(wl, c: int, b: int, n: int) -> np.ndarray:
    return bf16_to_f64(wl.pkey_bits(c, b, np.arange(n)))


def row_keys(wl, c: int, rows, ld: int):
    """Each row's pooled keys (one array per distinct stream, shared between its rows)."""
    keys, cache = [], {}
    for (b, t) in rows:
        n = min(n_compressed(t), ld)
        if cache.get(b, (None, 0))[1] < n:
            cache[b] = (keys_of(wl, c, b, n), n)
        keys.append(cache[b][0])
    return keys


def logits(wl, c: int, rows, ld: int, keys=None) -> np.ndarray:
    q = bf16_to_f64(wl.iq_bits(c, rows))
    w = wl.weights(c, rows).astype(np.float64)
    if keys is None:
        keys = row_keys(wl, c, rows, ld)
    return indexer_logits(q, w, keys, [t for _, t in rows], ld)


def n_valid(rows, ld: int) -> np.ndarray:
    return np.array([min(n_compressed(t), ld) for _, t in rows], dtype=np.int64)


def attention(wl, c: int, rows, blocks: np.ndarray, scale: float):
    q = bf16_to_f64(wl.q_bits(c, rows))
    readers = {b: rows_reader(wl, c, b) for b in {b for b, _ in rows}}
    return sparse_mla(q, lambda r, S: readers[rows[r][0]](S), blocks,
                      [t for _, t in rows], scale)


def dense_attention(wl, c: int, rows, n_blocks: int, scale: float):
    """The dense pass over the first n_blocks pooled blocks, for the given query rows."""
    q = bf16_to_f64(wl.q_bits(c, rows))
    readers = {b: rows_reader(wl, c, b) for b in {b for b, _ in rows}}
    return dense_mla(q, lambda r, S: readers[rows[r][0]](S), [t for _, t in rows], n_blocks, scale)


def step(wl, c: int, rows, ld: int, scale: float):
    """Indexer logits -> top-k blocks -> attention, for the given query rows."""
    l = logits(wl, c, rows, ld)
    nv = n_valid(rows, ld)
    blk = topk_blocks(l, nv, wl.k)
    out, lse = attention(wl, c, rows, blk, scale)
    return l, nv, blk, out, lse
