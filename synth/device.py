"""Device-side filling of synthetic workloads (the GPU twin of synth/__init__.py).

The fill kernels live in ``libtf_synth.so`` (built from ``synth.hip``) and draw
exactly the bits the numpy generator draws. Pools are populated through the
library's own ``tf_latent_write``, as an engine would fill them.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import (TAG_IQ, TAG_LAT8, TAG_LATENT, TAG_PKEY, TAG_Q, TAG_SCALE8, TAG_W, fp8_row_scale_base, stream_key,
               unit_scale)
from .configs import LAT, ROPE, ROW, rid

HERE = os.path.dirname(os.path.abspath(__file__))
SYNTH_LIB = os.path.join(HERE, "libtf_synth.so")
NAN16 = 0x7FC0
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SYNTH_LIB):
            raise RuntimeError(f"{SYNTH_LIB} is missing: build with `python -m attention_page_table_amd.build`")
        L = ctypes.CDLL(SYNTH_LIB)
        u64, vp = ctypes.c_uint64, ctypes.c_void_p
        L.tf_synth_bf16.argtypes = [vp, u64, u64, u64, u64, u64, ctypes.c_float, vp]
        L.tf_synth_f32.argtypes = [vp, u64, u64, u64, u64, u64, ctypes.c_float, vp]
        L.tf_synth_e4m3.argtypes = [vp, u64, u64, u64, u64, u64, vp]
        L.tf_synth_scale8.argtypes = [vp, u64, u64, u64, u64, ctypes.c_float, vp]
        for f in (L.tf_synth_bf16, L.tf_synth_f32, L.tf_synth_e4m3, L.tf_synth_scale8):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _st():
    return torch.cuda.current_stream().cuda_stream


def _ok(rc):
    if rc != 0:
        raise RuntimeError("synthetic fill kernel failed to launch")


def fill_bf16(out: torch.Tensor, n_rows: int, cols: int, seed: int, tag: int, base: int, stride: int, d: float):
    _ok(lib().tf_synth_bf16(out.data_ptr(), n_rows, cols, stream_key(seed, tag), int(base), int(stride),
                            float(unit_scale(d)), _st()))


def fill_f32(out, n_rows, cols, seed, tag, base, stride, d):
    _ok(lib().tf_synth_f32(out.data_ptr(), n_rows, cols, stream_key(seed, tag), int(base), int(stride),
                           float(unit_scale(d)), _st()))


def fill_e4m3(out, n_rows, cols, seed, tag, base, stride):
    _ok(lib().tf_synth_e4m3(out.data_ptr(), n_rows, cols, stream_key(seed, tag), int(base), int(stride), _st()))


def fill_scale8(out, n, seed, tag, base, stride=1):
    _ok(lib().tf_synth_scale8(out.data_ptr(), n, stream_key(seed, tag), int(base), int(stride),
                              float(fp8_row_scale_base()), _st()))


def _rid(c, owner, t) -> int:
    return int(rid(c, owner, t))


class Pool:
    """A workload's pool on the GPU: the byte pool, the page table and the plan."""

    def __init__(self, wl, plan, pool: torch.Tensor, pt: torch.Tensor):
        self.wl, self.plan, self.pool, self.pt = wl, plan, pool, pt

    def view(self, cache=0):
        import attention_page_table_amd as tf
        return tf.view(self.pool, self.pt, self.wl.pt_stride, self.wl.n_pages, cache)


def alloc_pool(wl, plan, poison=True) -> Pool:
    import attention_page_table_amd as tf
    tf.check_page_table(wl.pt, wl.n_pages)   # refuse a table naming pages outside the pool
    pool = torch.empty(wl.n_pages * plan.page_bytes, dtype=torch.uint8, device="cuda")
    if poison:
        pool.view(torch.int16).fill_(NAN16)
    pt = torch.from_numpy(np.ascontiguousarray(wl.pt)).cuda()
    return Pool(wl, plan, pool, pt)


def write_rows(P: Pool, c: int, b: int, t0: int, t1: int, owner: int | None = None, batch: int = 65536):
    """Write stream b's rows [t0, t1) and the pooled keys of the blocks they start,
    generated on the device, through tf_latent_write."""
    import attention_page_table_amd as tf
    wl = P.wl
    view = P.view(c)
    for s0 in range(t0, t1, batch):
        s1 = min(t1, s0 + batch)
        n = s1 - s0
        own = b if owner is None else owner
        r0 = _rid(c, own, s0)
        rope = torch.empty((n, ROPE), dtype=torch.bfloat16, device="cuda")
        fill_bf16(rope, n, ROPE, wl.seed, TAG_LATENT, r0 * ROW + LAT, ROW, ROW)
        if wl.fp8:
            lat = torch.empty((n, LAT), dtype=torch.uint8, device="cuda")
            fill_e4m3(lat, n, LAT, wl.seed, TAG_LAT8, r0 * LAT, LAT)
            sc = torch.empty(n, dtype=torch.float32, device="cuda")
            fill_scale8(sc, n, wl.seed, TAG_SCALE8, r0)
        else:
            lat = torch.empty((n, LAT), dtype=torch.bfloat16, device="cuda")
            fill_bf16(lat, n, LAT, wl.seed, TAG_LATENT, r0 * ROW, ROW, ROW)
            sc = None
        rs = torch.full((n,), b, dtype=torch.int32, device="cuda")
        rp = torch.arange(s0, s1, dtype=torch.int32, device="cuda")
        # pooled keys of the blocks that start in [s0, s1)
        j0, j1 = (s0 + 3) // 4, (s1 + 3) // 4
        nk = j1 - j0
        keys = torch.empty((max(nk, 1), wl.Dk), dtype=torch.bfloat16, device="cuda")
        if nk:
            fill_bf16(keys, nk, wl.Dk, wl.seed, TAG_PKEY, _rid(c, own, j0) * wl.Dk, wl.Dk, wl.Dk)
        ks = torch.full((nk,), b, dtype=torch.int32, device="cuda")
        ki = torch.arange(j0, j1, dtype=torch.int32, device="cuda")
        tf.latent_write(P.plan, view, rs, rp, lat, rope, row_scale=sc,
                        pkey_stream=ks if nk else None, pkey_idx=ki if nk else None, pkeys=keys if nk else None)


def populate(P: Pool, caches=None):
    """Write every stream's rows [0, L_b) (a shared prefix once, through stream 0)."""
    wl = P.wl
    for c in (range(wl.n_caches) if caches is None else caches):
        if wl.shared_tokens:
            write_rows(P, c, 0, 0, wl.shared_tokens, owner=0)
        for b in range(wl.n_streams):
            write_rows(P, c, b, wl.shared_tokens, wl.lengths[b])


def query_inputs(wl, c: int, rows):
    """Device tensors for the given (stream, position) rows: stream ids, positions,
    indexer queries [R,H,Dk] bf16, weights [R,H] fp32, attention queries [R,Hq,576] bf16."""
    R = len(rows)
    rs = torch.tensor([b for b, _ in rows], dtype=torch.int32, device="cuda")
    rp = torch.tensor([t for _, t in rows], dtype=torch.int32, device="cuda")
    iq = torch.empty((R, wl.H, wl.Dk), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((R, wl.H), dtype=torch.float32, device="cuda")
    q = torch.empty((R, wl.Hq, ROW), dtype=torch.bfloat16, device="cuda")
    # consecutive positions of one stream are consecutive generator rows: fill runs at once
    i = 0
    while i < R:
        b, t = rows[i]
        j = i
        while j + 1 < R and rows[j + 1] == (b, rows[j][1] + 1):
            j += 1
        n = j - i + 1
        r0 = _rid(c, b, t)
        fill_bf16(iq[i:], n * wl.H, wl.Dk, wl.seed, TAG_IQ, r0 * wl.H * wl.Dk, wl.Dk, wl.Dk)
        fill_f32(w[i:], n, wl.H, wl.seed, TAG_W, r0 * wl.H, wl.H, wl.w_d)
        fill_bf16(q[i:], n * wl.Hq, ROW, wl.seed, TAG_Q, r0 * wl.Hq * ROW, ROW, ROW)
        i = j + 1
    return rs, rp, iq, w, q
