"""GPU parity of exported paths that the workloads' own shapes do not reach: every
indexer instance (4, 8 and 16 heads x 64- and 128-dim keys) through each of its
kernel paths, the snapshot of a 12-cache pool (bf16 and fp8 rows), and page tables
that name pages outside the pool (writes skipped, reads NaN). Element by element
against the oracle, through the C ABI."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import attention_page_table_amd as tf
from oracle import Geom, PoolImage
from oracle import workload as ow
from oracle.layout import snapshot_copy
from synth import TAG_LATENT, TAG_PKEY, bf16_to_f64
from synth.configs import LAT, ROPE, ROW, shared_prefix_decode, tiny
from synth.device import NAN16, _rid, alloc_pool, fill_bf16, populate, query_inputs
from tests.gpu_common import check_attention, check_logits, host, logits_bound

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


_pools = {}


def _pool(Dk):
    """The tiny workload's streams with pooled keys of Dk values (one pool per width)."""
    if Dk not in _pools:
        wl = dataclasses.replace(tiny(0), Dk=Dk)
        plan = tf.kv_pool_plan(tf.geom(1, Dk))
        P = alloc_pool(wl, plan)
        populate(P)
        torch.cuda.synchronize()
        _pools[Dk] = (wl, plan, P)
    return _pools[Dk]


# rows that reach each indexer kernel path:
#   rows  - fewer than 64 rows: one wave per row (both streams, short and full prefixes);
#   tile  - 256 consecutive rows of one stream: the MFMA tile kernel;
#   mixed - 128 rows alternating between the streams: the tile kernel's per-row fallback.
INDEXER_ROWS = {
    "rows": [(0, 2047), (1, 2047), (0, 0), (1, 3), (1, 4), (0, 127), (0, 511), (1, 512), (0, 1000), (1, 1999)]
            + [(b, 1500 + 37 * i) for i in range(12) for b in (0, 1)],
    "tile": [(0, t) for t in range(1792, 2048)],
    "mixed": [(i % 2, 1024 + 7 * i) for i in range(128)],
}


@pytest.mark.parametrize("path", ["rows", "tile", "mixed"])
@pytest.mark.parametrize("H,Dk", [(4, 64), (8, 64), (16, 64), (4, 128), (8, 128), (16, 128)])
def test_indexer_every_instance(H, Dk, path):
    """Each (heads, key width) the ABI accepts, through the row kernel, the tile kernel
    (whose head sum follows the MFMAs for 128-dim keys and fewer than 16 heads, and is
    interleaved with them otherwise) and the tile kernel's per-row fallback."""
    _log(f"indexer: H={H} Dk={Dk}, {path} path")
    wl0, plan, P = _pool(Dk)
    wl = dataclasses.replace(wl0, H=H, w_d=float(H))
    rows = INDEXER_ROWS[path]
    rs, rp, iq, w, _ = query_inputs(wl, 0, rows)
    ld = 512
    logits = torch.empty((len(rows), ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(len(rows), dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, P.view(), rs, rp, iq, w, logits, n_valid=nv)
    torch.cuda.synchronize()
    ref = ow.logits(wl, 0, rows, ld)
    check_logits(host(logits), ref, logits_bound(wl, 0, rows, ld), f"H={H} Dk={Dk} {path}")
    assert np.array_equal(host(nv), ow.n_valid(rows, ld))



@pytest.mark.parametrize("n_rows,Dk", [(8, 128), (9, 128), (8, 64)])
def test_indexer_shared_prefix_rows(n_rows, Dk):
    """Rows of streams that hold the same prefix pages ([#1732] "What this changes"):
    a row group of four such streams scores each page once for all four rows (ranges
    of several pages); every logit is the oracle's. Eight rows make two such groups;
    nine add a group of one row, scored one row at a time. Rows 1, 3 and 6 stop
    inside the prefix, so the shared path masks per row; the last key range
    holds the last shared page and the streams' private tail pages, which the four
    rows score one at a time. Keys of 64 and 128 values."""
    wl = dataclasses.replace(shared_prefix_decode(0, n_streams=9, n_caches=1, shared_pages=601), Dk=Dk)
    _log(f"indexer: shared prefix, {wl.n_pages} pages, {n_rows} rows, Dk={Dk}")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    L = wl.lengths
    rows = [(0, L[0] - 1), (1, 200000), (2, L[2] - 1), (3, 77777), (4, L[4] - 1), (5, L[5] - 1), (6, 250000),
            (7, L[7] - 1), (8, L[8] - 1)][:n_rows]
    rs, rp, iq, w, _ = query_inputs(wl, 0, rows)
    ld = max(t // 4 + 1 for _, t in rows)
    logits = torch.empty((len(rows), ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(len(rows), dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, P.view(), rs, rp, iq, w, logits, n_valid=nv)
    torch.cuda.synchronize()
    ns = wl.shared_tokens // 4
    shared = ow.keys_of(wl, 0, 0, ns)
    keys = []
    for b, t in rows:
        n = t // 4 + 1
        keys.append(shared[:n] if n <= ns else
                    np.concatenate([shared, bf16_to_f64(wl.pkey_bits(0, b, np.arange(ns, n)))]))
    ref = ow.logits(wl, 0, rows, ld, keys=keys)
    check_logits(host(logits), ref, logits_bound(wl, 0, rows, ld, keys=keys), "shared prefix")
    assert np.array_equal(host(nv), ow.n_valid(rows, ld))


def test_indexer_shared_prefix_bad_pages():
    """A shared range in which one page id is outside the pool and one is -1 in every
    stream's table (the four rows still agree on every page): the keys of those two
    pages score NaN within each row's compressed length, as on the per-row path, and
    every other logit is the oracle's."""
    wl0 = shared_prefix_decode(0, n_streams=8, n_caches=1, shared_pages=601)
    plan = tf.kv_pool_plan(tf.geom(1, wl0.Dk))
    P = alloc_pool(wl0, plan)
    populate(P)
    pt = wl0.pt.copy()
    pt[:, 100] = wl0.n_pages + 3
    pt[:, 101] = -1
    _log("indexer: shared prefix with pages outside the pool")
    view = tf.view(P.pool, torch.from_numpy(pt).cuda(), wl0.pt_stride, wl0.n_pages)
    rows = wl0.rows
    rs, rp, iq, w, _ = query_inputs(wl0, 0, rows)
    ld = max(t // 4 + 1 for _, t in rows)
    logits = torch.empty((len(rows), ld), dtype=torch.float32, device="cuda")
    tf.indexer_logits(plan, view, rs, rp, iq, w, logits)
    torch.cuda.synchronize()
    got = host(logits).astype(np.float64)
    ns = wl0.shared_tokens // 4
    shared = ow.keys_of(wl0, 0, 0, ns)
    keys = [np.concatenate([shared, bf16_to_f64(wl0.pkey_bits(0, b, np.arange(ns, t // 4 + 1)))]) for b, t in rows]
    ref = ow.logits(wl0, 0, rows, ld, keys=keys)
    nan = np.zeros_like(ref, dtype=bool)
    nan[:, 100 * 128:102 * 128] = True
    assert np.array_equal(np.isnan(got), nan)
    ok = ~nan
    A = logits_bound(wl0, 0, rows, ld, keys=keys)
    check_logits(np.where(ok, got, 0.0), np.where(ok, ref, 0.0), np.where(ok, A, 0.0), "shared prefix, bad pages")

def _oracle_image_all_caches(wl, fp8):
    """The oracle's byte image of a pool holding every stream's rows and keys in every cache."""
    g = Geom(n_caches=wl.n_caches, index_dim=wl.Dk, fp8=fp8)
    img = PoolImage(g, wl.n_pages, fill=NAN16)
    for c in range(wl.n_caches):
        for b in range(wl.n_streams):
            L = wl.lengths[b]
            if fp8:
                codes, sc, rope = wl.latent_fp8(c, b, np.arange(L))
                for t in range(L):
                    img.write_row(wl.pt, wl.pt_stride, b, t, c, codes[t], rope[t], sc[t])
            else:
                bits = wl.latent_bits(c, b, np.arange(L))
                for t in range(L):
                    img.write_row(wl.pt, wl.pt_stride, b, t, c, bits[t, :LAT], bits[t, LAT:])
            kb = wl.pkey_bits(c, b, np.arange(wl.n_keys(b)))
            for j in range(wl.n_keys(b)):
                img.write_pkey(wl.pt, wl.pt_stride, b, j, c, kb[j])
    return img


@pytest.mark.parametrize("fp8", [False, True])
def test_snapshot_twelve_caches(fp8):
    """The snapshot copies rows [0, at) of every plane of all 12 caches, and keys
    [0, at / 4), for two stream pairs in one call; at = 1,540 leaves a partial last
    page. Byte for byte against the oracle's snapshot of its own pool image; the
    destination's other bytes keep their poison."""
    _log(f"snapshot: 12 caches, {'fp8' if fp8 else 'bf16'} rows, at 1,540, two stream pairs")
    rng = np.random.default_rng(12)
    pt = rng.permutation(8).astype(np.int32).reshape(2, 4)
    wl = dataclasses.replace(tiny(3), name="tiny_12_caches", n_caches=12, n_pages=8, pt=pt,
                             lengths=[2048, 1700], fp8=fp8, rows=[])
    plan = tf.kv_pool_plan(tf.geom(12, wl.Dk, fp8=fp8))
    P = alloc_pool(wl, plan)
    populate(P)
    torch.cuda.synchronize()
    img = _oracle_image_all_caches(wl, fp8)
    assert np.array_equal(host(P.pool), img.buf), "populated 12-cache pool differs from the oracle's image"
    at = 1540
    dpt = np.array([[5, 2, 7, 0], [1, 6, 3, 4]], dtype=np.int32)
    dst = torch.empty(8 * plan.page_bytes, dtype=torch.uint8, device="cuda")
    dst.view(torch.int16).fill_(NAN16)
    src_s = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    dst_s = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    tf.snapshot_copy(plan, P.view(), tf.view(dst, torch.from_numpy(dpt).cuda(), 4, 8, pt_host=dpt), src_s, dst_s, at)
    torch.cuda.synchronize()
    dimg = PoolImage(img.g, 8, fill=NAN16)
    snapshot_copy(img, wl.pt, wl.pt_stride, dimg, dpt, 4, [1, 0], [0, 1], at)
    got = host(dst)
    if not np.array_equal(got, dimg.buf):
        bad = np.flatnonzero(got != dimg.buf)
        raise AssertionError(f"{bad.size} bytes differ, first at {bad[:8]} (page bytes {plan.page_bytes})")


# ---- page tables naming pages outside the pool ----------------------------------------
# Stream 1 of the tiny pool with its page index 2 naming page 23 (past the 16-page pool)
# and page index 3 naming -1 (no page): tokens [1024, 2048) and keys [256, 512) of that
# stream are unreadable and unwritable; its pages 0 and 1 are as before.

def _bad_table(wl):
    pt = wl.pt.copy()
    pt[1, 2] = wl.n_pages + 7
    pt[1, 3] = -1
    return pt


def test_bad_page_ids_writes_skipped():
    """Rows and keys whose page the table cannot name are not written; every other
    byte of the pool is as the oracle's image with only the nameable rows written."""
    _log("bad page ids: writes through a table naming pages outside the pool")
    wl, plan, P = _pool(64)
    pt_bad = _bad_table(wl)
    pool = P.pool.clone()
    view = tf.view(pool, torch.from_numpy(pt_bad).cuda(), wl.pt_stride, wl.n_pages)
    # new values (another seed) for stream 1's rows 900..1199 and keys 200..299:
    # rows < 1024 and keys < 256 live in named pages, the rest do not
    wl2 = dataclasses.replace(wl, seed=wl.seed + 41)
    t0, t1, j0, j1 = 900, 1200, 200, 300
    n, nk = t1 - t0, j1 - j0
    lat = torch.empty((n, LAT), dtype=torch.bfloat16, device="cuda")
    rope = torch.empty((n, ROPE), dtype=torch.bfloat16, device="cuda")
    r0 = _rid(0, 1, t0)
    fill_bf16(lat, n, LAT, wl2.seed, TAG_LATENT, r0 * ROW, ROW, ROW)
    fill_bf16(rope, n, ROPE, wl2.seed, TAG_LATENT, r0 * ROW + LAT, ROW, ROW)
    keys = torch.empty((nk, wl.Dk), dtype=torch.bfloat16, device="cuda")
    fill_bf16(keys, nk, wl.Dk, wl2.seed, TAG_PKEY, _rid(0, 1, j0) * wl.Dk, wl.Dk, wl.Dk)
    rs = torch.full((n,), 1, dtype=torch.int32, device="cuda")
    rp = torch.arange(t0, t1, dtype=torch.int32, device="cuda")
    ks = torch.full((nk,), 1, dtype=torch.int32, device="cuda")
    kj = torch.arange(j0, j1, dtype=torch.int32, device="cuda")
    tf.latent_write(plan, view, rs, rp, lat, rope, pkey_stream=ks, pkey_idx=kj, pkeys=keys)
    torch.cuda.synchronize()
    img = PoolImage(Geom(n_caches=1, index_dim=wl.Dk), wl.n_pages)
    img.buf[:] = host(P.pool)                                  # the pool before the write
    bits = wl2.latent_bits(0, 1, np.arange(t0, t1))
    for i, t in enumerate(range(t0, t1)):
        if t < 1024:
            img.write_row(wl.pt, wl.pt_stride, 1, t, 0, bits[i, :LAT], bits[i, LAT:])
    kb = wl2.pkey_bits(0, 1, np.arange(j0, j1))
    for i, j in enumerate(range(j0, j1)):
        if j < 256:
            img.write_pkey(wl.pt, wl.pt_stride, 1, j, 0, kb[i])
    got = host(pool)
    if not np.array_equal(got, img.buf):
        raise AssertionError(_where_bytes_differ(got, img, wl.pt))


def _where_bytes_differ(got, img, pt):
    """Which pages, planes and slots hold the differing bytes (for the failure message)."""
    bad = np.flatnonzero(got != img.buf)
    L = img.L
    inv = {int(p): (b, i) for b, row in enumerate(pt) for i, p in enumerate(row) if p >= 0}
    out = {}
    for off in bad[:: max(1, bad.size // 64)]:
        page, r = divmod(int(off), img.page)
        if r < L.off_scale:
            plane, slot = "latent", r // L.lat_row
        elif r < L.off_rope:
            plane, slot = "scale", (r - L.off_scale) // 4
        elif r < L.off_pkey:
            plane, slot = "rope", (r - L.off_rope) // L.rope_row
        else:
            plane, slot = "pkey", (r - L.off_pkey) // L.pkey_row
        key = (page, inv.get(page), plane)
        out.setdefault(key, set()).add(slot)
    return f"{bad.size} bytes differ: " + "; ".join(
        f"page {k[0]} (stream, index {k[1]}) {k[2]} slots {min(v)}..{max(v)}" for k, v in sorted(out.items()))


@pytest.mark.parametrize("path", ["rows", "tile"])
def test_bad_page_ids_logits_nan(path):
    """Keys the table cannot name score NaN (within the row's compressed length); every
    other logit is the oracle's, and keys past the length stay -inf."""
    _log(f"bad page ids: indexer logits ({path} path)")
    wl, plan, P = _pool(64)
    pt_bad = _bad_table(wl)
    view = tf.view(P.pool, torch.from_numpy(pt_bad).cuda(), wl.pt_stride, wl.n_pages)
    rows = [(1, 2047), (1, 1100), (1, 300), (0, 2047)] if path == "rows" else [(1, t) for t in range(1800, 2048)]
    rs, rp, iq, w, _ = query_inputs(wl, 0, rows)
    ld = 512
    logits = torch.empty((len(rows), ld), dtype=torch.float32, device="cuda")
    tf.indexer_logits(plan, view, rs, rp, iq, w, logits)
    torch.cuda.synchronize()
    got = host(logits).astype(np.float64)
    ref = ow.logits(wl, 0, rows, ld)
    nan = np.zeros_like(ref, dtype=bool)
    for r, (b, t) in enumerate(rows):
        if b == 1:
            nan[r, 256:t // 4 + 1] = True
    assert np.array_equal(np.isnan(got), nan)
    ok = ~nan
    A = logits_bound(wl, 0, rows, ld)
    check_logits(np.where(ok, got, 0.0), np.where(ok, ref, 0.0), np.where(ok, A, 0.0), f"bad ids {path}")


@pytest.mark.parametrize("n_rows", [3, 160])
def test_bad_page_ids_attention_nan(n_rows):
    """A row that selects a token the table cannot name gives NaN for every head (and
    its log-sum-exp); rows whose selection stays in named pages match the oracle. Few
    rows take the decode kernel, many the 32-head kernel; the dense pass likewise."""
    _log(f"bad page ids: attention over {n_rows} rows (sparse and dense)")
    wl0, plan, P = _pool(64)
    wl = dataclasses.replace(wl0, Hq=32)
    pt_bad = _bad_table(wl)
    view = tf.view(P.pool, torch.from_numpy(pt_bad).cuda(), wl.pt_stride, wl.n_pages)
    if n_rows == 3:
        rows = [(1, 2047), (1, 1000), (0, 2047)]
    else:
        rows = [(1, 900 + 2 * i) for i in range(n_rows)]   # positions 900 .. 1218
    R = len(rows)
    k = 64
    blk = np.full((R, k), -1, dtype=np.int32)
    for r, (b, t) in enumerate(rows):
        vis = t // 4 + 1
        blk[r] = np.round(np.linspace(0, vis - 1, k)).astype(np.int32) if vis >= k else -1
        if vis < k:
            blk[r, :vis] = np.arange(vis)
    blk = np.sort(blk, axis=1)
    rs, rp, _, _, q = query_inputs(wl, 0, rows)
    scale = 1.0 / math.sqrt(576.0)
    for dense in (False, True):
        out = torch.empty((R, 32, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((R, 32), dtype=torch.float32, device="cuda")
        if dense:
            tf.dense_mla_attn(plan, view, rs, rp, q, scale, 512, out, lse)
        else:
            tf.sparse_mla_attn(plan, view, rs, rp, q, scale, torch.from_numpy(blk).cuda(), out, lse)
        torch.cuda.synchronize()
        o, l = host(out), host(lse)
        sel = blk if not dense else np.tile(np.arange(512, dtype=np.int32), (R, 1))
        bad = np.array([b == 1 and any(4 * x <= t and 4 * x >= 1024 for x in s if x >= 0)
                        for (b, t), s in zip(rows, sel)])
        assert bad.any() and (~bad).any()
        assert np.all(np.isnan(o[bad])) and np.all(np.isnan(l[bad]))
        good = np.flatnonzero(~bad)
        grows = [rows[i] for i in good]
        if dense:
            ro, rl = ow.dense_attention(wl, 0, grows, 512, scale)
        else:
            ro, rl = ow.attention(wl, 0, grows, blk[good], scale)
        check_attention(o[good], l[good], ro, rl, f"bad ids, dense={dense}")
