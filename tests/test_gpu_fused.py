"""GPU parity of the fused indexer + top-k (tf_indexer_topk_fused), which writes no
logits: its blocks and n_valid equal those of tf_indexer_logits followed by
tf_topk_blocks, bit for bit, through the C ABI.

Two streams of 40,000 and 36,000 tokens (10,000 and 9,000 pooled keys, so the page
sample and the filtered pass run) reach every kernel path: the row kernel (fewer than
64 rows; with ld = 300,000, since calls of fewer than 64 rows of at most 262,144 keys
are scored whole), the tile kernel (256 rows of one stream) and its per-row fallback
(rows alternating between the streams). Rows that see at most k keys, a row before its
stream's start and ragged lengths are included; so are inputs that overflow the
candidate regions and take the re-scoring path: rows whose logits all tie (zero
queries) and keys scaled up in all but every third page, so that a page sample sees
mostly small logits. k = 1024 takes the workgroup selection (about 2,048 candidates a
row); k = 2048, short rows (at most max(4,096, 8k) keys) and few rows at ld = 10,000
take the direct path, whose top-k runs its blocked mode on few rows. Sampled rows are
also checked against the oracle's logits."""
import dataclasses

import numpy as np
import pytest
import torch

import attention_page_table_amd as tf
from oracle import workload as ow
from synth.configs import Workload, tiny
from synth.device import alloc_pool, populate, query_inputs
from tests.gpu_common import check_attention, check_topk_against_oracle, host

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _medium(H, Dk):
    """Two streams of 40,000 and 36,000 tokens in shuffled 512-row pages (79 and 71 of a
    160-page pool), H indexer heads of Dk."""
    rng = np.random.default_rng(5)
    perm = rng.permutation(160).astype(np.int32)
    pt = np.full((2, 79), -1, dtype=np.int32)
    pt[0, :79] = perm[:79]
    pt[1, :71] = perm[79:150]
    return Workload("medium", 0, 1, 2, [40000, 36000], H=H, Dk=Dk, Hq=8, k=512, n_pages=160, pt=pt,
                    w_d=float(H), rows=[], description="2 streams x 40,000 / 36,000 tokens")


_pools = {}


def _pool(Dk):
    if Dk not in _pools:
        wl = _medium(16, Dk)
        plan = tf.kv_pool_plan(tf.geom(1, Dk))
        P = alloc_pool(wl, plan)
        populate(P)
        torch.cuda.synchronize()
        _pools[Dk] = (wl, plan, P)
    return _pools[Dk]


ROWS = {
    "rows": [(0, 39999), (1, 35999), (0, 0), (1, 3), (0, 2047), (0, 2048), (1, 8191), (0, 16383), (1, 20000),
             (0, 30001), (1, 35000), (0, 39000), (1, -1)],
    "tile": [(0, t) for t in range(39744, 40000)],
    "mixed": [(i % 2, 20000 + 61 * i) for i in range(128)],
}
ROWS["rows_direct"] = ROWS["rows"]
# the logits' row length per case: 13 rows take the filtered row kernel only past
# 262,144 keys (keys past a row's visible count are -inf)
LD = {"rows": 300000, "rows_direct": 10000, "tile": 10000, "mixed": 10000}


def _reference(plan, P, rs, rp, iq, w, ld, k):
    R = rs.numel()
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, P.view(), rs, rp, iq, w, logits, n_valid=nv)
    ref = torch.empty((R, k), dtype=torch.int32, device="cuda")
    tf.topk_blocks(logits, nv, k, ref)
    return ref, nv


def _fused(plan, P, rs, rp, iq, w, ld, k, ws=None):
    R = rs.numel()
    got = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    nv = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    tf.indexer_topk_fused(plan, P.view(), rs, rp, iq, w, ld, k, got, n_valid=nv, ws=ws)
    return got, nv


@pytest.mark.parametrize("path", ["rows", "rows_direct", "tile", "mixed"])
@pytest.mark.parametrize("H,Dk,k", [(16, 128, 512), (16, 128, 64), (16, 128, 1024), (16, 128, 2048), (8, 128, 512),
                                    (4, 64, 512), (16, 64, 200)])
def test_fused_equals_unblocked(H, Dk, k, path):
    _log(f"fused indexer + top-k: H={H} Dk={Dk} k={k}, {path} rows")
    wl0, plan, P = _pool(Dk)
    wl = dataclasses.replace(wl0, H=H, w_d=float(H))
    rows = ROWS[path]
    ld = LD[path]
    rs, rp, iq, w, _ = query_inputs(wl, 0, [(b, max(t, 0)) for b, t in rows])
    if path.startswith("rows"):
        rp[-1] = -1
    ref, nv = _reference(plan, P, rs, rp, iq, w, ld, k)
    got, nv2 = _fused(plan, P, rs, rp, iq, w, ld, k)
    torch.cuda.synchronize()
    assert torch.equal(nv2, nv)
    assert torch.equal(got, ref)


def test_fused_against_oracle():
    """20 rows (decode rows and every 37th tile row) at ld = 10,000: the direct path
    against the oracle's logits (the filtered paths are checked bit for bit against the
    unblocked pair, which is checked against the oracle)."""
    _log("fused indexer + top-k: oracle on decode and tile rows")
    wl, plan, P = _pool(128)
    rows = ROWS["rows"][:-1] + ROWS["tile"][::37]
    ld = 10000
    rs, rp, iq, w, _ = query_inputs(wl, 0, rows)
    got, nv = _fused(plan, P, rs, rp, iq, w, ld, wl.k)
    torch.cuda.synchronize()
    assert np.array_equal(host(nv), ow.n_valid(rows, ld))
    ref_l = ow.logits(wl, 0, rows, ld)
    check_topk_against_oracle(host(got), ref_l, host(nv), wl.k)


@pytest.mark.parametrize("path", ["rows", "tile"])
def test_fused_tied_rows_take_the_rescoring_path(path):
    """Zero queries: every visible logit is 0, every key passes the threshold and the
    regions overflow; the re-scoring path selects the k lowest-index keys, as the
    unblocked path does. Other rows of the call keep the candidate path."""
    _log(f"fused indexer + top-k: tied rows ({path})")
    wl, plan, P = _pool(128)
    rows = ROWS[path]
    ld = LD[path]
    rs, rp, iq, w, _ = query_inputs(wl, 0, [(b, max(t, 0)) for b, t in rows])
    if path == "rows":
        rp[-1] = -1
    iq[::3] = 0
    ref, nv = _reference(plan, P, rs, rp, iq, w, ld, wl.k)
    got, nv2 = _fused(plan, P, rs, rp, iq, w, ld, wl.k)
    torch.cuda.synchronize()
    assert torch.equal(nv2, nv)
    assert torch.equal(got, ref)
    blk, n = host(got), host(nv)
    for r in range(0, len(rows), 3):
        m = min(n[r], wl.k)
        assert np.array_equal(blk[r, :m], np.arange(m)) and np.all(blk[r, m:] == -1)


def test_fused_keys_large_outside_the_sample():
    """Keys of stream 0 scaled by 4 (exponent + 2) in every page but each third: a page
    sample that sees mostly unscaled keys sets a low threshold, regions overflow, and
    the rows take the re-scoring path; the blocks still equal the unblocked path's."""
    _log("fused indexer + top-k: keys scaled outside every third page")
    wl = _medium(16, 128)
    plan = tf.kv_pool_plan(tf.geom(1, 128))
    P = alloc_pool(wl, plan)
    populate(P)
    torch.cuda.synchronize()
    pool16 = P.pool.view(torch.int16)
    for i in range(79):
        if i % 3 == 0:
            continue
        page = int(wl.pt[0, i])
        o = (page * plan.page_bytes + plan.off_pkey) // 2
        seg = pool16[o:o + 128 * plan.pkey_row_bytes // 2]
        exp = (seg >> 7) & 0xFF
        seg.copy_(torch.where((exp > 0) & (exp < 0xFD), seg + 0x100, seg))
    for path in ("rows", "tile"):
        rows, ld = ROWS[path], LD[path]
        rs, rp, iq, w, _ = query_inputs(wl, 0, [(b, max(t, 0)) for b, t in rows])
        if path == "rows":
            rp[-1] = -1
        ref, nv = _reference(plan, P, rs, rp, iq, w, ld, wl.k)
        got, nv2 = _fused(plan, P, rs, rp, iq, w, ld, wl.k)
        torch.cuda.synchronize()
        assert torch.equal(nv2, nv)
        assert torch.equal(got, ref)


@pytest.mark.parametrize("k", [64, 200])
def test_fused_short_rows_direct(k):
    """At most 4,096 keys: the rows are scored whole into the workspace and selected
    there (tiny workload: 512 keys, decode rows and the 256-row chunk)."""
    _log(f"fused indexer + top-k: short rows, k={k}")
    wl = tiny(0)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    rows = wl.rows + [(1, 0), (1, 200), (0, 1000)]
    rs, rp, iq, w, _ = query_inputs(wl, 0, rows)
    ld = 512
    ref, nv = _reference(plan, P, rs, rp, iq, w, ld, k)
    got, nv2 = _fused(plan, P, rs, rp, iq, w, ld, k)
    torch.cuda.synchronize()
    assert torch.equal(nv2, nv)
    assert torch.equal(got, ref)


def test_fused_reused_workspace_without_n_valid():
    """One workspace for two calls in a row, the second on fewer rows; no n_valid."""
    _log("fused indexer + top-k: reused workspace, no n_valid")
    wl, plan, P = _pool(128)
    ld, k = 10000, 512
    ws = torch.empty(tf.indexer_topk_fused_workspace_bytes(256, ld, k, 16), dtype=torch.uint8, device="cuda")
    for rows in (ROWS["tile"], ROWS["tile"][:100], ROWS["rows"][:-1]):
        rs, rp, iq, w, _ = query_inputs(wl, 0, rows)
        ref, _ = _reference(plan, P, rs, rp, iq, w, ld, k)
        got = torch.empty((len(rows), k), dtype=torch.int32, device="cuda")
        tf.indexer_topk_fused(plan, P.view(), rs, rp, iq, w, ld, k, got, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


@pytest.mark.parametrize("k", [1024, 2048])
def test_decode_attention_long_block_lists(k):
    """Decode rows (fewer than 128) with up to 2,048 selected blocks (8,192 tokens): the
    decode attention kernel runs up to 64 splits a row and the merge combines them in
    batches; against the oracle on the GPU's own blocks."""
    _log(f"decode attention: k={k}, 32 heads, merge over up to {k // 32} splits")
    wl0, plan, P = _pool(128)
    wl = dataclasses.replace(wl0, Hq=32)
    rows = [(0, 39999), (1, 35999), (0, 20000), (1, 9000), (0, 4000)]
    ld = 10000
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    blocks, nv = _reference(plan, P, rs, rp, iq, w, ld, k)
    out = torch.empty((len(rows), 32, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((len(rows), 32), dtype=torch.float32, device="cuda")
    scale = 1.0 / np.sqrt(576.0)
    tf.sparse_mla_attn(plan, P.view(), rs, rp, q, scale, blocks, out, lse)
    torch.cuda.synchronize()
    ro, rl = ow.attention(wl, 0, rows, host(blocks), scale)
    check_attention(host(out), host(lse), ro, rl, f"k={k}")
