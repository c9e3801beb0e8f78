"""GPU parity on the tiny workload (2 streams x 2,048 tokens, 16-page pool, 8 heads,
top-64): every step through the C ABI, element by element against the oracle.
Sizes span several tiles and ragged tails; edge cases included."""
import math

import numpy as np
import pytest
import torch

import attention_page_table_amd as tf
from oracle import PoolImage, Geom, topk_blocks, quantize_rows
from oracle import workload as ow
from oracle.layout import snapshot_copy
from synth import TAG_LATENT, bf16_values, e4m3_codes, fp8_row_scales, TAG_LAT8, TAG_SCALE8
from synth.configs import tiny, ROW, rid
from synth.device import alloc_pool, populate, query_inputs, fill_bf16, fill_e4m3, fill_scale8, NAN16
from tests.gpu_common import (bf16_host, check_attention, check_logits, check_topk_against_oracle, host,
                              logits_bound, topk_on_values)

pytestmark = pytest.mark.gpu
SCALES = [1.0 / math.sqrt(576.0), 24.0]


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def tiny_pool():
    wl = tiny(0)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    torch.cuda.synchronize()
    return wl, plan, P


def oracle_image(wl, fp8=False):
    g = Geom(n_caches=wl.n_caches, index_dim=wl.Dk, fp8=fp8)
    img = PoolImage(g, wl.n_pages, fill=NAN16)
    for b in range(wl.n_streams):
        L = wl.lengths[b]
        if fp8:
            codes, sc, rope = wl.latent_fp8(0, b, np.arange(L))
            for t in range(L):
                img.write_row(wl.pt, wl.pt_stride, b, t, 0, codes[t], rope[t], sc[t])
        else:
            bits = wl.latent_bits(0, b, np.arange(L))
            for t in range(L):
                img.write_row(wl.pt, wl.pt_stride, b, t, 0, bits[t, :512], bits[t, 512:])
        kb = wl.pkey_bits(0, b, np.arange(wl.n_keys(b)))
        for j in range(wl.n_keys(b)):
            img.write_pkey(wl.pt, wl.pt_stride, b, j, 0, kb[j])
    return img


def test_device_generator_matches_host():
    _log("generator: bf16, e4m3 and scale fills against numpy")
    n = 100_003
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    fill_bf16(out, n // 7, 7, 3, TAG_LATENT, 12345, 11, 576)
    m = (n // 7) * 7
    idx = 12345 + (np.arange(m) // 7) * 11 + np.arange(m) % 7
    assert np.array_equal(host(out.view(torch.int16))[:m].view(np.uint16), bf16_values(3, TAG_LATENT, idx, 576))
    o8 = torch.empty(m, dtype=torch.uint8, device="cuda")
    fill_e4m3(o8, n // 7, 7, 3, TAG_LAT8, 12345, 11)
    assert np.array_equal(host(o8), e4m3_codes(3, TAG_LAT8, idx))
    sc = torch.empty(1000, dtype=torch.float32, device="cuda")
    fill_scale8(sc, 1000, 3, TAG_SCALE8, 77)
    assert np.array_equal(host(sc), fp8_row_scales(3, TAG_SCALE8, 77 + np.arange(1000)))


def test_write_bytes_exact(tiny_pool):
    _log("write: pool bytes against the oracle's pool image (tiny)")
    wl, plan, P = tiny_pool
    img = oracle_image(wl)
    assert np.array_equal(host(P.pool), img.buf)


def test_snapshot_bytes_exact(tiny_pool):
    _log("snapshot: first at rows into fresh pages (tiny)")
    wl, plan, P = tiny_pool
    at = 1540  # not a page multiple: a partial last page
    dst = torch.empty(4 * plan.page_bytes, dtype=torch.uint8, device="cuda")
    dst.view(torch.int16).fill_(NAN16)
    dpt = torch.tensor([[2, 0, 3, 1]], dtype=torch.int32, device="cuda")
    src_s = torch.tensor([1], dtype=torch.int32, device="cuda")
    dst_s = torch.tensor([0], dtype=torch.int32, device="cuda")
    tf.snapshot_copy(plan, P.view(), tf.view(dst, dpt, 4, 4), src_s, dst_s, at)
    torch.cuda.synchronize()
    img = oracle_image(wl)
    dimg = PoolImage(img.g, 4, fill=NAN16)
    snapshot_copy(img, wl.pt, wl.pt_stride, dimg, host(dpt), 4, [1], [0], at)
    assert np.array_equal(host(dst), dimg.buf)
    with pytest.raises(tf.TFError):
        tf.snapshot_copy(plan, P.view(), tf.view(dst, dpt, 4, 4), src_s, dst_s, 6)


def run_step(wl, plan, view, rows, ld, scale, k=None):
    k = k or wl.k
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    R = len(rows)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, view, rs, rp, iq, w, logits, n_valid=nv)
    blocks = torch.empty((R, k), dtype=torch.int32, device="cuda")
    tf.topk_blocks(logits, nv, k, blocks)
    out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
    tf.sparse_mla_attn(plan, view, rs, rp, q, scale, blocks, out, lse)
    torch.cuda.synchronize()
    return host(logits), host(nv), host(blocks), host(out), host(lse)


@pytest.mark.parametrize("hq", [8, 32])
@pytest.mark.parametrize("scale", SCALES)
def test_full_step_against_oracle(tiny_pool, scale, hq):
    _log(f"step: indexer -> top-k -> attention, tiny, {hq} heads, scale {scale:.4f}")
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, hq)
    rows = wl.rows
    ld = 512
    lg, nv, blk, out, lse = run_step(wl, plan, P.view(), rows, ld, scale)
    ref_l = ow.logits(wl, 0, rows, ld)
    check_logits(lg, ref_l, logits_bound(wl, 0, rows, ld), "tiny")
    assert np.array_equal(nv, ow.n_valid(rows, ld))
    # top-k on the GPU's own logits is exact
    assert np.array_equal(blk, topk_on_values(lg, nv, wl.k))
    check_topk_against_oracle(blk, ref_l, nv, wl.k)
    ro, rl = ow.attention(wl, 0, rows, blk, scale)
    check_attention(out, lse, ro, rl, "tiny")


def _with_heads(wl, hq):
    import copy
    w2 = copy.copy(wl)
    w2.Hq = hq
    return w2


@pytest.mark.parametrize("hq", [8, 32])
def test_decode_rows_split_paths(tiny_pool, hq):
    _log(f"decode rows only (split block lists, merge kernel), tiny, {hq} heads")
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, hq)
    rows = [(0, 2047), (1, 2047), (1, 1000), (0, 3)]
    lg, nv, blk, out, lse = run_step(wl, plan, P.view(), rows, 512, 24.0)
    ro, rl = ow.attention(wl, 0, rows, blk, 24.0)
    check_attention(out, lse, ro, rl, "decode split")


@pytest.mark.parametrize("scale", SCALES)
def test_prefill_rows_split_and_sparse_tiles(tiny_pool, scale):
    """Many rows with 32 heads (one workgroup per row and split, all heads together):
    154 rows split each block list in two (partials and the merge kernel); rows near
    the start of a stream have fewer visible blocks than k, so whole tiles hold no
    attended token."""
    _log(f"prefill rows: 32 heads, split block lists, sparse tiles, scale {scale:.4f}")
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, 32)
    rows = [(0, t) for t in range(1792, 1792 + 150)] + [(1, 3), (1, 40), (0, 511), (1, 2047)]
    lg, nv, blk, out, lse = run_step(wl, plan, P.view(), rows, 512, scale)
    assert np.array_equal(blk, topk_on_values(lg, nv, wl.k))
    ro, rl = ow.attention(wl, 0, rows, blk, scale)
    check_attention(out, lse, ro, rl, "prefill rows")


def test_paged_equals_contiguous_bitwise(tiny_pool):
    _log("paged == contiguous window, bit for bit (tiny)")
    wl, plan, P = tiny_pool
    contig = torch.empty(8 * plan.page_bytes, dtype=torch.uint8, device="cuda")
    contig.view(torch.int16).fill_(NAN16)
    # copy each stream's pages into window order with the snapshot (rows [0, 2048))
    s = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    tf.snapshot_copy(plan, P.view(), tf.view(contig, None, 4, 8), s, s, 2048)
    a = run_step(wl, plan, P.view(), wl.rows, 512, 24.0)
    b = run_step(wl, plan, tf.view(contig, None, 4, 8), wl.rows, 512, 24.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_shuffled_pages_same_bits():
    _log("another page permutation gives the same bits (tiny)")
    wl1 = tiny(0)
    wl2 = tiny(0)
    rng = np.random.default_rng(99)
    perm = rng.permutation(16).astype(np.int32)
    wl2.pt = perm[:8].reshape(2, 4)
    outs = []
    for wl in (wl1, wl2):
        plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
        P = alloc_pool(wl, plan)
        populate(P)
        outs.append(run_step(wl, plan, P.view(), wl.rows, 512, 24.0))
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


def test_decode_row_equals_chunk_last_row(tiny_pool):
    _log("decode row == last row of the prefill chunk (tiny)")
    wl, plan, P = tiny_pool
    dec = run_step(wl, plan, P.view(), [(0, 2047)], 512, 24.0)
    chunk = run_step(wl, plan, P.view(), [(0, t) for t in range(1792, 2048)], 512, 24.0)
    assert np.array_equal(dec[0][0], chunk[0][-1])
    assert np.array_equal(dec[2][0], chunk[2][-1])
    check_attention(dec[3], dec[4], chunk[3][-1:], chunk[4][-1:], "decode vs chunk")


def test_topk_takes_all_and_dense_equivalence(tiny_pool):
    _log("top-k >= visible blocks: attention equals dense causal attention (tiny)")
    wl, plan, P = tiny_pool
    rows = [(0, 0), (0, 3), (0, 4), (1, 37), (1, 255), (0, 511)]   # n_c = 1, 1, 2, 10, 64, 128
    ld = 128
    lg, nv, blk, out, lse = run_step(wl, plan, P.view(), rows, ld, 24.0, k=128)
    for r, (b, t) in enumerate(rows):
        nc = t // 4 + 1
        assert blk[r, :nc].tolist() == list(range(nc)) and np.all(blk[r, nc:] == -1)
    from oracle.attention import sparse_mla_row
    from synth import bf16_to_f64
    q = bf16_to_f64(wl.q_bits(0, rows))
    for r, (b, t) in enumerate(rows):
        o, l = sparse_mla_row(q[r], ow.rows_reader(wl, 0, b), list(range(t // 4 + 1)), t, 24.0)
        check_attention(out[r:r + 1], lse[r:r + 1], o[None], l[None], f"dense row {r}")


def test_topk_edge_cases():
    _log("top-k: ties, signed zeros, ragged rows, k > n_valid, single and blocked modes")
    rng = np.random.default_rng(5)
    for ld, R, k in [(300, 5, 64), (5000, 3, 512), (40000, 4, 512), (4096, 600, 100), (20000, 600, 512)]:
        v = np.round(rng.standard_normal((R, ld)), 1).astype(np.float32)    # many ties
        v[0, :50] = -0.0
        v[0, 50:100] = 0.0
        nv = rng.integers(1, ld + 1, size=R).astype(np.int32)
        nv[0] = ld
        nv[-1] = min(ld, k - 1) if k > 1 else 1                               # fewer than k visible
        lg = torch.from_numpy(v).cuda()
        nvt = torch.from_numpy(nv).cuda()
        blk = torch.empty((R, k), dtype=torch.int32, device="cuda")
        tf.topk_blocks(lg, nvt, k, blk)
        torch.cuda.synchronize()
        assert np.array_equal(host(blk), topk_on_values(v, nv, k)), (ld, R, k)
    # all equal values
    lg = torch.zeros((2, 10000), dtype=torch.float32, device="cuda")
    blk = torch.empty((2, 512), dtype=torch.int32, device="cuda")
    tf.topk_blocks(lg, None, 512, blk)
    torch.cuda.synchronize()
    assert np.array_equal(host(blk), np.tile(np.arange(512), (2, 1)))


def test_topk_sampled_threshold_paths():
    """Rows of 16 and 32 keys per thread cut their keys down with a threshold from
    per-group maxima (1, 2 or 4 samples per thread as k grows) before the exact
    selection; ragged rows, few visible samples, heavy ties (the whole-row fallback)
    and continuous values all give the exact top-k; rows of 24 and 28 keys per thread
    (16,385 .. 28,672 keys) included. Rows of 8 keys per thread (up to 8,192 keys)
    select on the whole row."""
    _log("top-k: sampled thresholds, k up to 2048, fallbacks")
    rng = np.random.default_rng(13)
    for ld, k, ties in [(20000, 512, False), (20000, 1000, False), (30000, 1500, False), (32768, 2048, False),
                        (10000, 700, False), (20000, 512, True), (32768, 2048, True),
                        (8192, 512, False), (6000, 1000, False), (8000, 2000, False), (8192, 2048, False),
                        (8192, 512, True), (24576, 2048, False), (25000, 512, False), (28672, 1500, True)]:
        R = 130                                                    # >= 128 rows: one workgroup per row
        v = rng.standard_normal((R, ld)).astype(np.float32)
        if ties:
            v = np.round(v, 1).astype(np.float32)
        nv = rng.integers(k + 1, ld + 1, size=R).astype(np.int32)
        nv[0] = ld
        nv[1] = k + 1                                              # fewer valid samples than k
        nv[2] = k
        nv[3] = 1
        lg = torch.from_numpy(v).cuda()
        nvt = torch.from_numpy(nv).cuda()
        blk = torch.empty((R, k), dtype=torch.int32, device="cuda")
        tf.topk_blocks(lg, nvt, k, blk)
        torch.cuda.synchronize()
        assert np.array_equal(host(blk), topk_on_values(v, nv, k)), (ld, k, ties)


def test_topk_blocked_workspace_reuse_and_graph_replay():
    """Long rows merge per-block candidates through the workspace: a reused workspace,
    a workspace of arbitrary bytes and replays of a captured call all give the exact
    top-k."""
    _log("top-k blocked mode: workspace reuse, arbitrary workspace bytes, graph replays")
    rng = np.random.default_rng(9)
    R, ld, k = 5, 33000, 512
    nv = np.array([ld, 30000, 4097, 513, 20000], dtype=np.int32)
    vals = [rng.standard_normal((R, ld)).astype(np.float32) for _ in range(3)]
    want = [topk_on_values(v, nv, k) for v in vals]
    nvt = torch.from_numpy(nv).cuda()
    need = tf.topk_workspace_bytes(R, ld, k)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    lg = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    blk = torch.empty((R, k), dtype=torch.int32, device="cuda")
    for i in range(6):                                   # the same workspace, call after call
        lg.copy_(torch.from_numpy(vals[i % 3]))
        tf.topk_blocks(lg, nvt, k, blk, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(blk), want[i % 3]), f"reuse {i}"
    junk = torch.from_numpy(rng.integers(0, 256, size=need, dtype=np.uint8)).cuda()
    tf.topk_blocks(lg, nvt, k, blk, ws=junk)
    torch.cuda.synchronize()
    assert np.array_equal(host(blk), want[5 % 3]), "arbitrary workspace bytes"
    # one captured launch (one epoch) replayed with eager calls on the same workspace between
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tf.topk_blocks(lg, nvt, k, blk, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(6):
        lg.copy_(torch.from_numpy(vals[i % 3]))
        blk.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(blk), want[i % 3]), f"replay {i}"
        if i % 2 == 1:                                   # eager work between replays
            tf.topk_blocks(lg, nvt, k, blk, ws=ws)
            torch.cuda.synchronize()
            assert np.array_equal(host(blk), want[i % 3]), f"eager after replay {i}"


def test_empty_and_degenerate(tiny_pool):
    _log("degenerate calls: zero rows, blocks all -1")
    wl, plan, P = tiny_pool
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    tf.latent_write(plan, P.view(), e, e, torch.empty((0, 512), dtype=torch.bfloat16, device="cuda"),
                    torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    rs, rp, iq, w, q = query_inputs(wl, 0, [(0, 100), (1, 2047)])
    blocks = torch.full((2, 64), -1, dtype=torch.int32, device="cuda")
    out = torch.full((2, wl.Hq, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.zeros((2, wl.Hq), dtype=torch.float32, device="cuda")
    tf.sparse_mla_attn(plan, P.view(), rs, rp, q, 1.0, blocks, out, lse)
    torch.cuda.synchronize()
    assert np.all(host(out) == 0) and np.all(np.isneginf(host(lse)))


@pytest.mark.parametrize("scale", SCALES)
def test_fp8_rows(scale):
    _log(f"fp8 rows: write bytes and attention with in-kernel dequant (tiny, scale {scale:.4f})")
    wl = tiny(1)
    wl.fp8 = True
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk, fp8=True))
    P = alloc_pool(wl, plan)
    populate(P)
    torch.cuda.synchronize()
    img = oracle_image(wl, fp8=True)
    assert np.array_equal(host(P.pool), img.buf)
    lg, nv, blk, out, lse = run_step(wl, plan, P.view(), wl.rows, 512, scale)
    ro, rl = ow.attention(wl, 0, wl.rows, blk, scale)
    check_attention(out, lse, ro, rl, "fp8 tiny")


def _bf16_rows(x: np.ndarray):
    """float32 values rounded to bf16: the device tensor and the same values as float32."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.cuda(), t.to(torch.float32).numpy(), t.view(torch.int16).numpy().view(np.uint16)


def test_latent_write_quantize():
    _log("quantizing write: e4m3 codes, row scales, rope and keys against the oracle, byte for byte")
    wl = tiny(2)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk, fp8=True))
    P = alloc_pool(wl, plan)
    rng = np.random.default_rng(11)
    # 384 distinct rows of both streams, the pages' first and last slots among them
    pos = [(b, t) for b in range(2) for t in (0, 511, 512, 1023, 1536, 2047)]
    rest = rng.choice(2 * 2048, 384, replace=False)
    for v in rest:
        if len(pos) == 384:
            break
        bt = (int(v) // 2048, int(v) % 2048)
        if bt not in pos:
            pos.append(bt)
    R = len(pos)
    x = (rng.standard_normal((R, 512)) / 24.0).astype(np.float32)
    x[0] = 0.0                                      # an all-zero row
    x[1] = rng.uniform(-6e-5, 6e-5, 512)            # one large value: the rest code as subnormals
    x[1, 300] = 3.0
    x[2, ::2] = -0.0                                # signed zeros
    x[3] = -np.abs(x[3])
    x[3, 5] = -1.0                                  # the maximum is negative
    x[4] = np.float32(1.0) + np.arange(512, dtype=np.float32) / 64.0   # many codes on ties after scaling
    lat, xf, _ = _bf16_rows(x)
    rope, _, rope_bits = _bf16_rows(rng.standard_normal((R, 64)) / 24.0)
    rs = torch.tensor([b for b, _ in pos], dtype=torch.int32, device="cuda")
    rp = torch.tensor([t for _, t in pos], dtype=torch.int32, device="cuda")
    keys = [(b, j) for b in range(2) for j in (0, 127, 128, 511)] + [(0, 300), (1, 5)]
    kv, _, key_bits = _bf16_rows(rng.standard_normal((len(keys), wl.Dk)) / 8.0)
    ks = torch.tensor([b for b, _ in keys], dtype=torch.int32, device="cuda")
    kj = torch.tensor([j for _, j in keys], dtype=torch.int32, device="cuda")
    tf.latent_write_quantize(plan, P.view(), rs, rp, lat, rope, ks, kj, kv)
    torch.cuda.synchronize()
    codes, scale = quantize_rows(xf)
    img = PoolImage(Geom(n_caches=1, index_dim=wl.Dk, fp8=True), wl.n_pages, fill=NAN16)
    for i, (b, t) in enumerate(pos):
        img.write_row(wl.pt, wl.pt_stride, b, t, 0, codes[i], rope_bits[i], scale[i])
    for i, (b, j) in enumerate(keys):
        img.write_pkey(wl.pt, wl.pt_stride, b, j, 0, key_bits[i])
    got = host(P.pool)
    if not np.array_equal(got, img.buf):
        bad = np.flatnonzero(got != img.buf)
        raise AssertionError(f"{bad.size} bytes differ, first at {bad[:8]}")
    assert scale[0] == 0 and np.sum((codes[1] & 0x78) == 0) > 400
    # the plan's bf16 twin refuses the call
    plan16 = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    with pytest.raises(tf.TFError):
        tf.latent_write_quantize(plan16, P.view(), rs, rp, lat, rope)


@pytest.mark.parametrize("scale", SCALES)
def test_attention_running_max_jumps(tiny_pool, scale):
    """Queries aimed at one token in each of four later tiles, so that a head's scores
    on them sit at 5, 11, 14 and 40 (log2 units): the running max of the online
    softmax jumps mid-row, sometimes by more than 2^8 (O rescaled) and sometimes by
    less (the tile taken against a max that lags its own). 256 rows, 32 heads, chosen
    blocks; against the oracle."""
    _log(f"attention: running-max jumps mid-row, 32 heads, scale {scale:.4f}")
    from oracle import sparse_mla
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, 32)
    rows = [(0, t) for t in range(1792, 2048)]
    R = len(rows)
    rs, rp, _, _, q = query_inputs(wl, 0, rows)
    # 64 distinct blocks per row, spread over the visible ones, ascending
    blk = np.stack([np.round(np.linspace(0, t // 4, wl.k)).astype(np.int32) for _, t in rows])
    assert all(len(np.unique(b)) == wl.k for b in blk)
    reader = ow.rows_reader(wl, 0, 0)
    qf = q.to(torch.float32).cpu().numpy().astype(np.float64)
    targets_log2 = np.array([5.0, 11.0, 14.0, 40.0])
    c = targets_log2 / (scale * np.log2(np.e))                 # q . k on each target token
    for r in range(R):
        toks = [4 * int(blk[r][j]) for j in (15, 31, 47, 63)]   # tiles 7, 15, 23, 31 of the row
        lat, rope = reader(toks)
        kv = np.concatenate([lat, rope], axis=1)               # [4, 576]
        aim = (c[:, None] * kv / (kv * kv).sum(axis=1, keepdims=True)).sum(axis=0)
        qf[r, 0::2] += aim                                     # half the heads
    qd = torch.from_numpy(qf.astype(np.float32)).to(torch.bfloat16).cuda()
    qexact = qd.to(torch.float32).cpu().numpy().astype(np.float64)
    blocks = torch.from_numpy(blk).cuda()
    out = torch.empty((R, 32, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, 32), dtype=torch.float32, device="cuda")
    tf.sparse_mla_attn(plan, P.view(), rs, rp, qd, scale, blocks, out, lse)
    torch.cuda.synchronize()
    ro, rl = sparse_mla(qexact, lambda r, S: reader(S), blk, [t for _, t in rows], scale)
    # the jumps are there: on aimed heads the last target outscores the first by far
    lat, rope = reader([4 * int(blk[0][15]), 4 * int(blk[0][63])])
    z = scale * np.log2(np.e) * (qexact[0] @ np.concatenate([lat, rope], axis=1).T)
    assert np.all(z[0::2, 1] - z[0::2, 0] > 20)
    check_attention(host(out), host(lse), ro, rl, "running-max jumps")


@pytest.mark.parametrize("hq,nrows", [(24, 152), (20, 4)])
def test_attention_partial_head_group(tiny_pool, hq, nrows):
    """A head count that fills neither 16 nor 32: the last head group runs with its
    missing heads masked (never written). 24 heads on many rows (one group of 32),
    20 heads on decode rows (two groups of 16)."""
    _log(f"attention: {hq} heads over {nrows} rows (a partial head group)")
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, hq)
    rows = [(0, t) for t in range(1792, 1792 + nrows - 2)] + [(1, 2047), (1, 700)]
    lg, nv, blk, out, lse = run_step(wl, plan, P.view(), rows, 512, 24.0)
    assert out.shape == (nrows, hq, 512)
    ro, rl = ow.attention(wl, 0, rows, blk, 24.0)
    check_attention(out, lse, ro, rl, f"{hq} heads")


# ---- the dense pass (no indexer, no top-k) -------------------------------------------

def run_dense(wl, plan, view, rows, n_blocks, scale):
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    R = len(rows)
    out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
    tf.dense_mla_attn(plan, view, rs, rp, q, scale, n_blocks, out, lse)
    torch.cuda.synchronize()
    return host(out), host(lse)


# decode rows (few rows: the 128-token kernel, splits past a row's position cut to
# one masked slot), and a chunk with early positions (many rows: the 32-head sliced
# kernel or the 16-head kernel)
DENSE_ROWS = {
    "decode": [(0, 2047), (1, 2047), (1, 0), (0, 130), (1, 1029)],
    "chunk": [(0, t) for t in range(1792, 2048)] + [(1, t) for t in (0, 1, 2, 3, 4, 63, 511, 512, 1500)],
}


@pytest.mark.parametrize("hq", [8, 32])
@pytest.mark.parametrize("kind", ["decode", "chunk"])
@pytest.mark.parametrize("n_blocks", [512, 300, 1024, 2048])
def test_dense_against_oracle(tiny_pool, hq, kind, n_blocks):
    """Every visible token within the first n_blocks blocks: 512 covers each row's
    causal range exactly, 300 cuts the later rows at token 1,199, 1024 and 2048 run
    past the streams (2048: two 4,096-token splits for the chunk, the second all
    masked, merged)."""
    _log(f"dense pass: {kind} rows, {hq} heads, n_blocks {n_blocks} (tiny)")
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, hq)
    rows = DENSE_ROWS[kind]
    scale = 24.0 if n_blocks != 300 else SCALES[0]
    out, lse = run_dense(wl, plan, P.view(), rows, n_blocks, scale)
    ro, rl = ow.dense_attention(wl, 0, rows, n_blocks, scale)
    check_attention(out, lse, ro, rl, f"dense {kind}")


@pytest.mark.parametrize("kind", ["decode", "chunk"])
@pytest.mark.parametrize("n_blocks", [512, 200, 1024, 2048])
def test_dense_equals_sparse_on_every_block_bitwise(tiny_pool, kind, n_blocks):
    """The dense pass is the sparse pass with blocks 0 .. n_blocks - 1 selected: same
    bits (the slots it cuts hold masked tokens only). At 1,024 and 2,048 blocks the
    sparse pass's workgroups own 4,096-token lists (one split, or two merged) whose
    tokens past the streams are masked."""
    _log(f"dense == sparse over blocks 0..{n_blocks - 1}, bit for bit ({kind})")
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, 32)
    rows = DENSE_ROWS[kind]
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    R = len(rows)
    blocks = torch.arange(n_blocks, dtype=torch.int32, device="cuda").repeat(R, 1).contiguous()
    outs = []
    for dense in (True, False):
        out = torch.full((R, 32, 512), 7.0, dtype=torch.float32, device="cuda")
        lse = torch.full((R, 32), 7.0, dtype=torch.float32, device="cuda")
        if dense:
            tf.dense_mla_attn(plan, P.view(), rs, rp, q, 24.0, n_blocks, out, lse)
        else:
            tf.sparse_mla_attn(plan, P.view(), rs, rp, q, 24.0, blocks, out, lse)
        torch.cuda.synchronize()
        outs.append((host(out), host(lse)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_dense_bits_do_not_depend_on_pages(tiny_pool):
    """The same streams in a contiguous window (null table) give the same bits."""
    _log("dense pass: paged == contiguous window, bit for bit (tiny)")
    wl, plan, P = tiny_pool
    wl = _with_heads(wl, 32)
    contig = torch.empty(8 * plan.page_bytes, dtype=torch.uint8, device="cuda")
    contig.view(torch.int16).fill_(NAN16)
    s = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    tf.snapshot_copy(plan, P.view(), tf.view(contig, None, 4, 8), s, s, 2048)
    for kind in ("decode", "chunk"):
        a = run_dense(wl, plan, P.view(), DENSE_ROWS[kind], 512, 24.0)
        b = run_dense(wl, plan, tf.view(contig, None, 4, 8), DENSE_ROWS[kind], 512, 24.0)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


@pytest.mark.parametrize("hq,rows_kind,n_blocks", [(8, "mixed", 512), (32, "mixed", 512),
                                                  (32, "chunk", 1024), (32, "chunk", 2048)])
def test_dense_fp8_rows(hq, rows_kind, n_blocks):
    """fp8 rows through the dense pass. With 32 heads over the 265 chunk rows the
    32-head fp8 kernel runs; at 1,024 blocks a workgroup owns one 4,096-token list,
    at 2,048 two splits are merged."""
    _log(f"dense pass over fp8 rows, {hq} heads, {rows_kind} rows, n_blocks {n_blocks} (tiny)")
    wl = tiny(1)
    wl.fp8 = True
    wl = _with_heads(wl, hq)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk, fp8=True))
    P = alloc_pool(wl, plan)
    populate(P)
    torch.cuda.synchronize()
    rows = DENSE_ROWS["decode"] + DENSE_ROWS["chunk"][::4] if rows_kind == "mixed" else DENSE_ROWS["chunk"]
    out, lse = run_dense(wl, plan, P.view(), rows, n_blocks, 24.0)
    ro, rl = ow.dense_attention(wl, 0, rows, n_blocks, 24.0)
    check_attention(out, lse, ro, rl, "dense fp8")


@pytest.mark.parametrize("k", [1024, 2048])
def test_sparse_fp8_long_block_lists(k):
    """The sparse pass over fp8 rows with 1,024 and 2,048 selected blocks on 265 rows and
    32 heads (the 32-head fp8 kernel, 4,096-token workgroup lists): every visible
    block of a row is selected, in a shuffled order padded with blocks past the row
    and -1 entries; against the oracle on the same lists."""
    _log(f"sparse pass over fp8 rows, k {k}, 265 rows, 32 heads (tiny)")
    from oracle import sparse_mla
    wl = tiny(1)
    wl.fp8 = True
    wl = _with_heads(wl, 32)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk, fp8=True))
    P = alloc_pool(wl, plan)
    populate(P)
    rows = DENSE_ROWS["chunk"]
    R = len(rows)
    rng = np.random.default_rng(k)
    blk = np.full((R, k), -1, dtype=np.int32)
    for r, (_, t) in enumerate(rows):
        vis = np.arange(t // 4 + 1)
        extra = np.arange(t // 4 + 1, t // 4 + 1 + (k - vis.size) // 2)   # past the row: masked
        lst = np.concatenate([vis, extra]).astype(np.int32)
        rng.shuffle(lst)
        blk[r, :lst.size] = lst
    rs, rp, _, _, q = query_inputs(wl, 0, rows)
    out = torch.empty((R, 32, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, 32), dtype=torch.float32, device="cuda")
    tf.sparse_mla_attn(plan, P.view(), rs, rp, q, 24.0, torch.from_numpy(blk).cuda(), out, lse)
    torch.cuda.synchronize()
    ro, rl = ow.attention(wl, 0, rows, blk, 24.0)
    check_attention(host(out), host(lse), ro, rl, f"sparse fp8 k={k}")


# ---- key-blocked indexer + top-k -----------------------------------------------------

@pytest.mark.parametrize("key_block,k", [(128, 64), (256, 64), (384, 64), (128, 200), (512, 64)])
def test_indexer_topk_blocked_equals_unblocked(tiny_pool, key_block, k):
    """Scoring one key block at a time and merging the blocks' top-k gives the blocks
    the whole logits buffer gives, bit for bit: decode rows, the chunk, and rows that
    see fewer than k blocks (early positions, a row before the stream's start).
    Block sizes that divide the 512 keys, one that leaves a ragged last block (384),
    k above the block size (each block passes all its keys on), one block."""
    _log(f"indexer + top-k by key blocks of {key_block}, k = {k} (tiny)")
    wl, plan, P = tiny_pool
    rows = wl.rows + [(1, 0), (1, 3), (1, 200), (0, 1000), (1, -1)]
    ld = 512
    rs, rp, iq, w, q = query_inputs(wl, 0, [(b, max(t, 0)) for b, t in rows])
    rp[-1] = -1
    R = len(rows)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, P.view(), rs, rp, iq, w, logits, n_valid=nv)
    ref = torch.empty((R, k), dtype=torch.int32, device="cuda")
    tf.topk_blocks(logits, nv, k, ref)
    got = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    nv2 = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    tf.indexer_topk(plan, P.view(), rs, rp, iq, w, ld, k, key_block, got, n_valid=nv2)
    torch.cuda.synchronize()
    assert np.array_equal(host(nv2), host(nv))
    assert np.array_equal(host(got), host(ref))
    blk = host(got)
    assert np.all(blk[-1] == -1)
    # and against the oracle's logits (the checks of the unblocked path)
    ref_l = ow.logits(wl, 0, [(b, max(t, 0)) for b, t in rows[:-1]], ld)
    check_topk_against_oracle(blk[:-1], ref_l, host(nv)[:-1], k)


def test_indexer_topk_blocked_without_n_valid_and_reused_workspace(tiny_pool):
    """No n_valid output (the library keeps n_c in the workspace); one workspace for two
    calls in a row, the second on fewer rows."""
    _log("indexer + top-k by key blocks: workspace n_c, reused workspace (tiny)")
    wl, plan, P = tiny_pool
    ld, k, B = 512, 64, 128
    ws = torch.empty(tf.indexer_topk_workspace_bytes(len(wl.rows), ld, k, B), dtype=torch.uint8, device="cuda")
    for rows in (wl.rows, wl.rows[:40]):
        rs, rp, iq, w, q = query_inputs(wl, 0, rows)
        R = len(rows)
        logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
        nv = torch.empty(R, dtype=torch.int32, device="cuda")
        tf.indexer_logits(plan, P.view(), rs, rp, iq, w, logits, n_valid=nv)
        ref = torch.empty((R, k), dtype=torch.int32, device="cuda")
        tf.topk_blocks(logits, nv, k, ref)
        got = torch.empty((R, k), dtype=torch.int32, device="cuda")
        tf.indexer_topk(plan, P.view(), rs, rp, iq, w, ld, k, B, got, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(got), host(ref))


# ---- two-level candidate selection ---------------------------------------------------

@pytest.mark.parametrize("group,n_cand,k", [(8, 64, 40), (8, 2048, 512), (3, 50, 60), (1, 100, 100), (8, 5, 64)])
def test_candidate_selection_against_oracle(group, n_cand, k):
    """Groups of 8 (quads), 3 (no quads) and 1 (plain top-k), ragged rows whose last group
    is partial, a row before the stream's start, tied values; consumers with more
    candidate keys than k and with fewer (n_cand 5 x 8 keys < 64: completed by the
    lowest-index others); one workgroup per row (3,000 or 20,000 keys) and, on a few
    long rows, the per-block kernels. Exact against the oracle on the same fp32
    values."""
    from oracle import candidate_groups as o_cand, topk_in_candidates as o_topk
    _log(f"candidate selection: groups of {group}, {n_cand} candidates, top-{k}")
    rng = np.random.default_rng(group * 1000 + n_cand)
    R, ld = 140, 20000 if n_cand == 2048 else 3000
    v = rng.standard_normal((R, ld)).astype(np.float32)
    v[::3] = np.round(v[::3], 1)                               # heavy ties on every third row
    nv = rng.integers(1, ld + 1, size=R).astype(np.int32)
    nv[0], nv[1], nv[2], nv[3] = ld, ld - 1, 0, 7
    lg = torch.from_numpy(v).cuda()
    nvt = torch.from_numpy(nv).cuda()
    cand = torch.full((R, n_cand), -7, dtype=torch.int32, device="cuda")
    tf.candidate_groups(lg, nvt, group, n_cand, cand)
    blk = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    lg2 = lg.clone()
    tf.topk_in_candidates(lg2, nvt, cand, group, k, blk)
    torch.cuda.synchronize()
    assert torch.equal(lg, torch.from_numpy(v).cuda())        # both calls only read the logits
    assert torch.equal(lg2, lg)
    ref_c = o_cand(v, nv, group, n_cand)
    assert np.array_equal(host(cand), ref_c)
    assert np.array_equal(host(blk), o_topk(v, nv, ref_c, group, k))


@pytest.mark.parametrize("group,n_cand,k", [(8, 2048, 512), (3, 700, 300)])
def test_candidate_selection_long_rows(group, n_cand, k):
    """A few long rows (40,000 keys): the consumer's top-k runs per key block (masked
    stage 1, then the merge), and groups straddle the blocks when the group does not
    divide them (groups of 3)."""
    from oracle import candidate_groups as o_cand, topk_in_candidates as o_topk
    _log(f"candidate selection on long rows: groups of {group}, {n_cand} candidates, top-{k}")
    rng = np.random.default_rng(group + n_cand)
    R, ld = 6, 40000
    v = rng.standard_normal((R, ld)).astype(np.float32)
    v[1] = np.round(v[1], 1)
    nv = np.array([ld, ld - 5, 33000, 4097, 9000, 12], dtype=np.int32)
    lg = torch.from_numpy(v).cuda()
    nvt = torch.from_numpy(nv).cuda()
    cand = torch.empty((R, n_cand), dtype=torch.int32, device="cuda")
    tf.candidate_groups(lg, nvt, group, n_cand, cand)
    blk = torch.empty((R, k), dtype=torch.int32, device="cuda")
    tf.topk_in_candidates(lg, nvt, cand, group, k, blk)
    torch.cuda.synchronize()
    ref_c = o_cand(v, nv, group, n_cand)
    assert np.array_equal(host(cand), ref_c)
    assert np.array_equal(host(blk), o_topk(v, nv, ref_c, group, k))
