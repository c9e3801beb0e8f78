"""Synthetic workloads shaped like the pages' configurations.

Only shapes, seeds, page tables and generator indices live here: no step of the
method. Each value of a workload is a pure function of (seed, tag, index), so the
host (numpy) and the device fill kernel produce the same bits.

Index scheme (unique per tensor element):
  row id   rid(c, owner, t) = ((c * 64 + owner) << 32) | t
  latent   rid * 576 + d           (d < 512 latent, 512 <= d < 576 rope)
  pkey     rid(c, owner, j) * D_k + i
  q        (rid(c, b, t) * Hq + h) * 576 + d
  iq       (rid(c, b, t) * H + h) * D_k + i
  w        rid(c, b, t) * H + h
  fp8 code rid * 512 + d; fp8 scale rid
where ``owner`` is 0 for tokens of a shared prefix and the stream id otherwise.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import (TAG_IQ, TAG_LAT8, TAG_LATENT, TAG_PKEY, TAG_Q, TAG_SCALE8, TAG_W, bf16_values,
               e4m3_codes, f32_values, fp8_row_scales)

PAGE_ROWS = 512
POOL_RATIO = 4
LAT = 512
ROPE = 64
ROW = LAT + ROPE


def rid(c: int, owner, t) -> np.ndarray:
    return (((np.uint64(c) * np.uint64(64) + np.asarray(owner, dtype=np.uint64)) << np.uint64(32))
            | np.asarray(t, dtype=np.uint64))


@dataclass
class Workload:
    name: str
    seed: int
    n_caches: int
    n_streams: int
    lengths: list            # context length L_b of each stream (rows [0, L_b) exist)
    H: int                   # indexer heads
    Dk: int                  # indexer head dim / pooled key dim
    Hq: int                  # attention heads
    k: int                   # top-k blocks
    n_pages: int
    pt: np.ndarray           # [S, pt_stride] int32 page ids
    shared_tokens: int = 0   # tokens [0, shared) are one prefix held by every stream
    fp8: bool = False
    w_d: float = 1.0         # weights are N(0,1)/sqrt(w_d)
    rows: list = field(default_factory=list)   # query rows: (stream, position)
    description: str = ""

    @property
    def pt_stride(self) -> int:
        return self.pt.shape[1]

    # ---------------- owners ------------------------------------------------
    def owner(self, b: int, t) -> np.ndarray:
        t = np.asarray(t, dtype=np.int64)
        return np.where(t < self.shared_tokens, 0, b)

    def key_owner(self, b: int, j) -> np.ndarray:
        j = np.asarray(j, dtype=np.int64)
        return np.where((j + 1) * POOL_RATIO <= self.shared_tokens, 0, b)

    # ---------------- host values (numpy) -------------------------------------
    def latent_bits(self, c: int, b: int, tokens) -> np.ndarray:
        """bf16 bits [n, 576] of rows (latent then rope)."""
        tokens = np.asarray(tokens, dtype=np.int64)
        r = rid(c, self.owner(b, tokens), tokens)
        idx = r[:, None] * np.uint64(ROW) + np.arange(ROW, dtype=np.uint64)[None, :]
        return bf16_values(self.seed, TAG_LATENT, idx, ROW)

    def latent_fp8(self, c: int, b: int, tokens):
        """(codes [n, 512] uint8, scales [n] float32, rope bits [n, 64] uint16)."""
        tokens = np.asarray(tokens, dtype=np.int64)
        r = rid(c, self.owner(b, tokens), tokens)
        idx = r[:, None] * np.uint64(LAT) + np.arange(LAT, dtype=np.uint64)[None, :]
        codes = e4m3_codes(self.seed, TAG_LAT8, idx)
        scales = fp8_row_scales(self.seed, TAG_SCALE8, r)
        ridx = r[:, None] * np.uint64(ROW) + np.arange(LAT, ROW, dtype=np.uint64)[None, :]
        rope = bf16_values(self.seed, TAG_LATENT, ridx, ROW)
        return codes, scales, rope

    def pkey_bits(self, c: int, b: int, js) -> np.ndarray:
        js = np.asarray(js, dtype=np.int64)
        r = rid(c, self.key_owner(b, js), js)
        idx = r[:, None] * np.uint64(self.Dk) + np.arange(self.Dk, dtype=np.uint64)[None, :]
        return bf16_values(self.seed, TAG_PKEY, idx, self.Dk)

    def q_bits(self, c: int, rows) -> np.ndarray:
        """[R, Hq, 576] bf16 bits of attention queries."""
        out = []
        for (b, t) in rows:
            r = rid(c, b, t)
            idx = ((r * np.uint64(self.Hq) + np.arange(self.Hq, dtype=np.uint64))[:, None]
                   * np.uint64(ROW) + np.arange(ROW, dtype=np.uint64)[None, :])
            out.append(bf16_values(self.seed, TAG_Q, idx, ROW))
        return np.stack(out) if out else np.zeros((0, self.Hq, ROW), np.uint16)

    def iq_bits(self, c: int, rows) -> np.ndarray:
        out = []
        for (b, t) in rows:
            r = rid(c, b, t)
            idx = ((r * np.uint64(self.H) + np.arange(self.H, dtype=np.uint64))[:, None]
                   * np.uint64(self.Dk) + np.arange(self.Dk, dtype=np.uint64)[None, :])
            out.append(bf16_values(self.seed, TAG_IQ, idx, self.Dk))
        return np.stack(out) if out else np.zeros((0, self.H, self.Dk), np.uint16)

    def weights(self, c: int, rows) -> np.ndarray:
        out = []
        for (b, t) in rows:
            r = rid(c, b, t)
            idx = r * np.uint64(self.H) + np.arange(self.H, dtype=np.uint64)
            out.append(f32_values(self.seed, TAG_W, idx, self.w_d))
        return np.stack(out) if out else np.zeros((0, self.H), np.float32)

    def n_keys(self, b: int) -> int:
        """Pooled keys that exist for stream b: one per started block."""
        return (self.lengths[b] + POOL_RATIO - 1) // POOL_RATIO


def _shuffled_tables(rng, n_pages: int, per_stream: list, pt_stride: int) -> np.ndarray:
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((len(per_stream), pt_stride), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(per_stream):
        pt[b, :n] = perm[o:o + n]
        o += n
    assert o <= n_pages
    return pt


def _pages(L: int) -> int:
    return (L + PAGE_ROWS - 1) // PAGE_ROWS


def tiny(seed: int = 0) -> Workload:
    """1 layer; 2 streams of 2,048 tokens in 512-row pages scattered in a 16-page
    pool; keys of 64 bf16; 4 indexer heads; 8 attention heads; top-64. Query rows:
    one decode row per stream (position 2,047) and a prefill chunk of 256 rows,
    positions [1,792, 2,048) of stream 0."""
    rng = np.random.default_rng(seed)
    L = [2048, 2048]
    pt = _shuffled_tables(rng, 16, [4, 4], 4)
    rows = [(0, 2047), (1, 2047)] + [(0, t) for t in range(1792, 2048)]
    return Workload("tiny", seed, 1, 2, L, H=4, Dk=64, Hq=8, k=64, n_pages=16, pt=pt,
                    w_d=1.0, rows=rows,
                    description="2 streams x 2,048 tokens, 16-page pool, decode + T=256 chunk")


def decode_batch(seed: int = 0, n_streams: int = 8, L: int = 131072) -> Workload:
    """Decode batch: 8 streams x 131,072 tokens, 1 layer, pages shuffled in the
    pool; 16 indexer heads x 128; 32 attention heads; top-512 blocks."""
    rng = np.random.default_rng(seed)
    per = [_pages(L)] * n_streams
    n_pages = sum(per)
    pt = _shuffled_tables(rng, n_pages, per, per[0])
    rows = [(b, L - 1) for b in range(n_streams)]
    return Workload("decode_8x131072", seed, 1, n_streams, [L] * n_streams, H=16, Dk=128, Hq=32,
                    k=512, n_pages=n_pages, pt=pt, w_d=16.0, rows=rows,
                    description=f"{n_streams} streams x {L} tokens decode, shuffled pages")


def prefill_chunk(seed: int = 0, L: int = 100000, T: int = 2048, slack_pages: int = 60) -> Workload:
    """Prefill chunk T=2,048 rows [L-T, L) against a prefix of L=100,000 for one
    stream: logits [2,048, 25,000], top-512, 32 attention heads."""
    rng = np.random.default_rng(seed)
    n = _pages(L)
    pt = _shuffled_tables(rng, n + slack_pages, [n], n)
    rows = [(0, t) for t in range(L - T, L)]
    return Workload(f"prefill_{T}_at_{L}", seed, 1, 1, [L], H=16, Dk=128, Hq=32, k=512,
                    n_pages=n + slack_pages, pt=pt, w_d=16.0, rows=rows,
                    description=f"one stream, chunk rows [{L - T}, {L}), keys {L // 4}")


def shared_prefix_decode(seed: int = 0, n_streams: int = 8, n_caches: int = 12,
                         shared_pages: int = 2048) -> Workload:
    """Decode batch of 8 streams sharing a 1,048,576-token prefix by page reference
    (2,048 shared pages, the same ids in every table) plus one private tail page
    per stream with 1-511 tokens; 12 caches."""
    rng = np.random.default_rng(seed)
    shared = shared_pages * PAGE_ROWS
    tails = rng.integers(1, 512, size=n_streams)
    n_pages = shared_pages + n_streams
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.empty((n_streams, shared_pages + 1), dtype=np.int32)
    pt[:, :shared_pages] = perm[:shared_pages][None, :]
    pt[:, shared_pages] = perm[shared_pages:]
    L = [shared + int(x) for x in tails]
    rows = [(b, L[b] - 1) for b in range(n_streams)]
    return Workload("shared_prefix_decode_8x1M_12caches", seed, n_caches, n_streams, L, H=16,
                    Dk=128, Hq=32, k=512, n_pages=n_pages, pt=pt, shared_tokens=shared,
                    w_d=16.0, rows=rows,
                    description="8 streams share 2,048 pages (1,048,576 tokens) + 1 tail page each")


def adaptive_prefill(seed: int = 0, N: int = 390000, at: int = 262144) -> Workload:
    """390,000-token prompt in fp8 rows with per-row fp32 scales, prefilled in
    adaptive chunks; afterwards the first ``at`` rows are snapshot and one more
    2,048-token chunk is resumed. Stream 0 holds the run; stream 1 receives the
    snapshot (its own pages)."""
    rng = np.random.default_rng(seed)
    n_run = _pages(N)
    n_res = _pages(at + 2048)
    n_pages = n_run + n_res
    pt = _shuffled_tables(rng, n_pages, [n_run, n_res], max(n_run, n_res))
    return Workload("adaptive_prefill_390000_fp8", seed, 1, 2, [N, at + 2048], H=16, Dk=128,
                    Hq=32, k=512, n_pages=n_pages, pt=pt, fp8=True, w_d=16.0, rows=[],
                    description="fp8 rows, adaptive chunks, snapshot at 262,144 and resume")


def attention_scales():
    """Softmax scales used in parity runs: 1/sqrt(576) (flat softmax) and 24 (peaked)."""
    return [1.0 / math.sqrt(576.0), 24.0]
