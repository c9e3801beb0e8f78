"""Page geometry, the page-table address of a row, and a byte image of the pool.

Test infrastructure (see the package docstring).

The pages fix: 512-row pages [#1142, "GLM declares a kv_pool.Layout" and its
question 2]; kernels take a page table and "the elements between pages", and a
null table keeps contiguous rows [#1142, same section]; one page id spans all 12
caches (11 MLA layers + the MTP layer) [#1142, "What happens now"; #1313,
"Why"]; a latent row is 512 bf16 [#1142, "What happens now"]; one pooled index
key per 4 tokens [same]; FP8 rows keep their fp32 scales after the page's rows,
516 bytes a row and cache [#1313, "Proposal", step 1 item 3].

Readings (the pages are silent):

* Inside one cache's block of a page the planes are, in order: latent rows,
  (fp8 only) the rows' fp32 scales, the rows' 64 bf16 rope values, then the
  page's 512/4 = 128 pooled keys.
* A null page table maps stream b's page i to pool page ``b * pt_stride + i``:
  a window is its pages in order [#1313, "Proposal", step 1 item 3].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Geom:
    n_caches: int = 1
    page_rows: int = 512
    latent_dim: int = 512
    rope_dim: int = 64
    pool_ratio: int = 4
    index_dim: int = 128
    fp8: bool = False


@dataclass(frozen=True)
class BlockLayout:
    lat_row: int      # bytes of one latent row
    rope_row: int     # bytes of one rope row
    pkey_row: int     # bytes of one pooled key
    off_latent: int
    off_scale: int    # fp8 only (else equal to off_rope)
    off_rope: int
    off_pkey: int
    block: int        # bytes of one cache inside one page
    keys_per_page: int


def block_layout(g: Geom) -> BlockLayout:
    lat_row = g.latent_dim * (1 if g.fp8 else 2)
    rope_row = g.rope_dim * 2
    pkey_row = g.index_dim * 2
    kpp = g.page_rows // g.pool_ratio
    off_latent = 0
    off_scale = off_latent + g.page_rows * lat_row
    off_rope = off_scale + (g.page_rows * 4 if g.fp8 else 0)
    off_pkey = off_rope + g.page_rows * rope_row
    block = off_pkey + kpp * pkey_row
    return BlockLayout(lat_row, rope_row, pkey_row, off_latent, off_scale, off_rope,
                       off_pkey, block, kpp)


def page_bytes(g: Geom) -> int:
    return g.n_caches * block_layout(g).block


def page_id(pt: np.ndarray | None, pt_stride: int, b: int, i: int) -> int:
    """Pool page holding stream b's i-th page. [#1142, "GLM declares a kv_pool.Layout"]"""
    if pt is None:
        return b * pt_stride + i
    return int(pt[b][i])


class PoolImage:
    """A byte image of the pool, with the page-table address formula.

    Row t of stream b, cache c lives in page ``pt[b][t // page_rows]`` at slot
    ``t % page_rows``; pooled key j lives in page ``pt[b][j // keys_per_page]``
    at slot ``j % keys_per_page``.
    """

    def __init__(self, g: Geom, n_pages: int, fill: int | None = None):
        self.g = g
        self.L = block_layout(g)
        self.n_pages = n_pages
        self.page = page_bytes(g)
        self.buf = np.zeros(n_pages * self.page, dtype=np.uint8)
        if fill is not None:
            self.poison(fill)

    def poison(self, value16: int = 0x7FC0):
        """Fill every byte pair with a bf16 NaN pattern (a read-before-write shows as NaN).
        [#1142, "GLM declares a kv_pool.Layout": TF_KV_POISON fills taken pages with NaN]"""
        self.buf.view(np.uint16)[:] = value16

    # ---- addresses --------------------------------------------------------
    def _base(self, pt, pt_stride, b, page_index, cache):
        p = page_id(pt, pt_stride, b, page_index)
        if not (0 <= p < self.n_pages):
            raise IndexError(f"page id {p} outside the pool of {self.n_pages}")
        return p * self.page + cache * self.L.block

    def row_addr(self, pt, pt_stride, b, t, cache, plane):
        g, L = self.g, self.L
        base = self._base(pt, pt_stride, b, t // g.page_rows, cache)
        slot = t % g.page_rows
        if plane == "latent":
            return base + L.off_latent + slot * L.lat_row
        if plane == "scale":
            assert g.fp8
            return base + L.off_scale + slot * 4
        if plane == "rope":
            return base + L.off_rope + slot * L.rope_row
        raise ValueError(plane)

    def pkey_addr(self, pt, pt_stride, b, j, cache):
        L = self.L
        base = self._base(pt, pt_stride, b, j // L.keys_per_page, cache)
        return base + L.off_pkey + (j % L.keys_per_page) * L.pkey_row

    # ---- writes (a byte copy) ----------------------------------------------
    def write_row(self, pt, pt_stride, b, t, cache, latent: np.ndarray, rope: np.ndarray,
                  scale: np.float32 | None = None):
        """Copy one token's row bytes into its page slot.
        [#1142, "GLM declares a kv_pool.Layout": writes take the page table]"""
        lat = np.ascontiguousarray(latent).view(np.uint8).ravel()
        rp = np.ascontiguousarray(rope).view(np.uint8).ravel()
        assert lat.size == self.L.lat_row and rp.size == self.L.rope_row
        a = self.row_addr(pt, pt_stride, b, t, cache, "latent")
        self.buf[a:a + lat.size] = lat
        a = self.row_addr(pt, pt_stride, b, t, cache, "rope")
        self.buf[a:a + rp.size] = rp
        if self.g.fp8:
            s = np.asarray([scale], dtype=np.float32).view(np.uint8)
            a = self.row_addr(pt, pt_stride, b, t, cache, "scale")
            self.buf[a:a + 4] = s

    def write_pkey(self, pt, pt_stride, b, j, cache, key: np.ndarray):
        kb = np.ascontiguousarray(key).view(np.uint8).ravel()
        assert kb.size == self.L.pkey_row
        a = self.pkey_addr(pt, pt_stride, b, j, cache)
        self.buf[a:a + kb.size] = kb

    # ---- reads ---------------------------------------------------------------
    def read_row_bytes(self, pt, pt_stride, b, t, cache):
        a = self.row_addr(pt, pt_stride, b, t, cache, "latent")
        lat = self.buf[a:a + self.L.lat_row].copy()
        a = self.row_addr(pt, pt_stride, b, t, cache, "rope")
        rope = self.buf[a:a + self.L.rope_row].copy()
        scale = None
        if self.g.fp8:
            a = self.row_addr(pt, pt_stride, b, t, cache, "scale")
            scale = self.buf[a:a + 4].copy().view(np.float32)[0]
        return lat, rope, scale

    def read_pkey_bytes(self, pt, pt_stride, b, j, cache):
        a = self.pkey_addr(pt, pt_stride, b, j, cache)
        return self.buf[a:a + self.L.pkey_row].copy()


def snapshot_copy(src: PoolImage, src_pt, src_stride, dst: PoolImage, dst_pt, dst_stride,
                  src_streams, dst_streams, at: int):
    """Copy each cache's first ``at`` rows (every plane) and the pooled keys up to
    ``at`` from one paged view to another; nothing else changes.
    [#1142, "Proposal" piece 1: snap_bytes(at) and keepAs copy each cache's first
    at rows and the pooled keys up to at; rows past at are never read]

    Reading: ``at`` is a multiple of the pool ratio, and "the pooled keys up to
    at" are keys [0, at / pool_ratio).
    """
    g = src.g
    assert g == dst.g
    if at % g.pool_ratio != 0:
        raise ValueError("at must be a multiple of the pool ratio")
    for b_s, b_d in zip(src_streams, dst_streams):
        for c in range(g.n_caches):
            for t in range(at):
                lat, rope, sc = src.read_row_bytes(src_pt, src_stride, b_s, t, c)
                dst.write_row(dst_pt, dst_stride, b_d, t, c, lat, rope, sc)
            for j in range(at // g.pool_ratio):
                dst.write_pkey(dst_pt, dst_stride, b_d, j, c,
                               src.read_pkey_bytes(src_pt, src_stride, b_s, j, c))
