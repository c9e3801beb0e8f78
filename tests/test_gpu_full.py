"""GPU parity at the workloads' full sizes, in the launch configuration the bench
times: every row where the oracle computes it in seconds, sampled rows otherwise,
and properties that hold at any size (top-k exact on the GPU's own logits; resumed
== fresh bit for bit; unwritten rows never read)."""
import math

import numpy as np
import pytest
import torch

import attention_page_table_amd as tf
from oracle import topk_blocks as oracle_topk
from oracle import workload as ow
from oracle.attention import sparse_mla_row
from oracle.indexer import indexer_logits
from synth import bf16_to_f64
from synth.configs import adaptive_prefill, decode_batch, prefill_chunk, shared_prefix_decode
from synth.device import NAN16, alloc_pool, populate, query_inputs, write_rows
from tests.gpu_common import (check_attention, check_logits, check_topk_against_oracle, host, logits_bound,
                              topk_on_values)

pytestmark = pytest.mark.gpu
SCALES = [1.0 / math.sqrt(576.0), 24.0]


def _log(msg):
    print(msg, flush=True)


def gpu_step(plan, view, wl, c, rows, ld, scales, q_rows=None, stream_override=None):
    """indexer -> top-k -> attention for the given rows; returns host copies."""
    rs, rp, iq, w, q = query_inputs(wl, c, q_rows or rows)
    if stream_override is not None:
        rs = torch.full_like(rs, stream_override)
    R = len(rows)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, view, rs, rp, iq, w, logits, n_valid=nv)
    blocks = torch.empty((R, wl.k), dtype=torch.int32, device="cuda")
    tf.topk_blocks(logits, nv, wl.k, blocks)
    outs = []
    for sc in scales:
        out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
        tf.sparse_mla_attn(plan, view, rs, rp, q, sc, blocks, out, lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return logits, host(nv), host(blocks), outs


def fused_blocks(plan, view, wl, c, rows, ld):
    """tf_indexer_topk_fused on the same rows: (blocks, n_valid) host copies."""
    rs, rp, iq, w, _ = query_inputs(wl, c, rows)
    R = len(rows)
    blocks = torch.full((R, wl.k), -7, dtype=torch.int32, device="cuda")
    nv = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    tf.indexer_topk_fused(plan, view, rs, rp, iq, w, ld, wl.k, blocks, n_valid=nv)
    torch.cuda.synchronize()
    return host(blocks), host(nv)


def test_decode_batch_full():
    """8 streams x 131,072 tokens, shuffled pages: every row against the oracle."""
    wl = decode_batch(0)
    _log(f"decode batch: populating {wl.n_pages} pages")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    rows, ld = wl.rows, 32768
    lg_t, nv, blk, outs = gpu_step(plan, P.view(), wl, 0, rows, ld, SCALES)
    lg = host(lg_t)
    _log("decode batch: fused indexer + top-k equals the unblocked path")
    fb, fnv = fused_blocks(plan, P.view(), wl, 0, rows, ld)
    assert np.array_equal(fnv, nv) and np.array_equal(fb, blk)
    _log("decode batch: oracle logits")
    ref = ow.logits(wl, 0, rows, ld)
    check_logits(lg, ref, logits_bound(wl, 0, rows, ld), "decode batch")
    assert np.array_equal(blk, topk_on_values(lg, nv, wl.k))
    check_topk_against_oracle(blk, ref, nv, wl.k)
    for sc, (out, lse) in zip(SCALES, outs):
        _log(f"decode batch: oracle attention, scale {sc:.4f}")
        ro, rl = ow.attention(wl, 0, rows, blk, sc)
        check_attention(host(out), host(lse), ro, rl, f"decode batch scale {sc}")


def test_prefill_chunk_full():
    """T = 2,048 rows against L = 100,000: logits and attention on sampled rows, top-k
    exact on every row's GPU logits."""
    wl = prefill_chunk(0)
    _log("prefill chunk: populating")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    rows, ld = wl.rows, 25000
    lg_t, nv, blk, outs = gpu_step(plan, P.view(), wl, 0, rows, ld, SCALES)
    lg = host(lg_t)
    _log("prefill chunk: exact top-k of every row's logits")
    assert np.array_equal(blk, topk_on_values(lg, nv, wl.k))
    _log("prefill chunk: fused indexer + top-k equals the unblocked path")
    fb, fnv = fused_blocks(plan, P.view(), wl, 0, rows, ld)
    assert np.array_equal(fnv, nv) and np.array_equal(fb, blk)
    rng = np.random.default_rng(7)
    sample = sorted(set([0, 1, 511, 1024, 2046, 2047] + rng.choice(2048, 10, replace=False).tolist()))
    srows = [rows[i] for i in sample]
    _log(f"prefill chunk: oracle on {len(sample)} sampled rows")
    ref = ow.logits(wl, 0, srows, ld)
    check_logits(lg[sample], ref, logits_bound(wl, 0, srows, ld), "prefill sampled")
    check_topk_against_oracle(blk[sample], ref, nv[sample], wl.k)
    for sc, (out, lse) in zip(SCALES, outs):
        ro, rl = ow.attention(wl, 0, srows, blk[sample], sc)
        check_attention(host(out)[sample], host(lse)[sample], ro, rl, f"prefill scale {sc}")


def test_shared_prefix_decode_12_caches():
    """8 streams sharing 2,048 pages (1,048,576 tokens) plus a private tail page each, 12
    caches: every cache runs (odd caches with the logits rows padded to 16 bytes, the
    bench's layout); caches 0, 5 and 11 are checked row by row."""
    wl = shared_prefix_decode(0)
    plan = tf.kv_pool_plan(tf.geom(wl.n_caches, wl.Dk))
    _log(f"shared prefix: pool {wl.n_pages} pages x {plan.page_bytes} B")
    P = alloc_pool(wl, plan)
    populate(P)
    rows = wl.rows
    ld0 = max(t // 4 + 1 for _, t in rows)
    for c in range(wl.n_caches):
        # odd caches: the logits rows padded to 16 bytes, as the bench lays them out (top-k's
        # 16-byte loads); even caches: the rows' own length (its 4-byte loads)
        ld = (ld0 + 3) // 4 * 4 if c % 2 else ld0
        lg_t, nv, blk, outs = gpu_step(plan, P.view(c), wl, c, rows, ld, [24.0])
        lg = host(lg_t)
        assert np.array_equal(blk, topk_on_values(lg, nv, wl.k)), f"cache {c}"
        fb, fnv = fused_blocks(plan, P.view(c), wl, c, rows, ld)
        assert np.array_equal(fnv, nv) and np.array_equal(fb, blk), f"fused, cache {c}"
        if c not in (0, 5, 11):
            continue
        _log(f"shared prefix: oracle, cache {c}")
        shared = ow.keys_of(wl, c, 0, wl.shared_tokens // 4)      # one copy of the shared keys
        keys = []
        for b, t in rows:
            n = t // 4 + 1
            tail = bf16_to_f64(wl.pkey_bits(c, b, np.arange(wl.shared_tokens // 4, n)))
            keys.append(np.concatenate([shared, tail]))
        ref = ow.logits(wl, c, rows, ld, keys=keys)
        check_logits(lg, ref, logits_bound(wl, c, rows, ld, keys=keys), f"cache {c}")
        check_topk_against_oracle(blk, ref, nv, wl.k)
        ro, rl = ow.attention(wl, c, rows, blk, 24.0)
        out, lse = outs[0]
        check_attention(host(out), host(lse), ro, rl, f"cache {c}")


def test_adaptive_prefill_fp8_snapshot_resume():
    """390,000-token prompt in fp8 rows, chunk(L) = clamp(round_down_256(2e8 / L), 256, 2048);
    sampled rows of several chunks against the oracle, and the fused indexer + top-k's
    blocks equal to the pair's on every 29th chunk; then the first 262,144 rows are
    snapshot into fresh pages, one 2,048-token chunk is resumed there, and it equals
    the same rows of the fresh run bit for bit."""
    wl = adaptive_prefill(0)
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk, fp8=True))
    P = alloc_pool(wl, plan)
    N = wl.lengths[0]
    view = P.view()
    L = 0
    n_chunks = 0
    checks = []
    rng = np.random.default_rng(11)
    _log("adaptive prefill: running the chunk schedule")
    while L < N:
        T = tf.prefill_chunk(L, N - L)
        write_rows(P, 0, 0, L, L + T)
        rows = [(0, t) for t in range(L, L + T)]
        ld = (L + T - 1) // 4 + 1
        lg_t, nv, blk, outs = gpu_step(plan, view, wl, 0, rows, ld, [24.0])
        if n_chunks % 29 == 0 or n_chunks in (47, 48, 463):   # every chunk size, short and long prefixes
            fb, fnv = fused_blocks(plan, view, wl, 0, rows, ld)
            assert np.array_equal(fnv, nv) and np.array_equal(fb, blk), f"fused, chunk at {L}"
        if n_chunks in (0, 1, 47, 48, 100, 200, 463) or L + T == N:
            sel = sorted(set([0, T - 1] + rng.choice(T, 2, replace=False).tolist()))
            checks.append((L, T, ld, [rows[i] for i in sel], host(lg_t)[sel], nv[sel], blk[sel],
                           host(outs[0][0])[sel], host(outs[0][1])[sel]))
        assert not torch.isnan(outs[0][0]).any(), f"NaN in chunk at {L}"
        L += T
        n_chunks += 1
    assert n_chunks == 464
    all_keys = ow.keys_of(wl, 0, 0, (N - 1) // 4 + 1)      # stream 0's keys, generated once
    for (L0, T, ld, srows, lg, nv, blk, out, lse) in checks:
        _log(f"adaptive prefill: oracle on chunk [{L0}, {L0 + T})")
        keys = [all_keys] * len(srows)
        ref = ow.logits(wl, 0, srows, ld, keys=keys)
        check_logits(lg, ref, logits_bound(wl, 0, srows, ld, keys=keys), f"chunk {L0}")
        assert np.array_equal(blk, topk_on_values(lg, nv, wl.k))
        check_topk_against_oracle(blk, ref, nv, wl.k)
        ro, rl = ow.attention(wl, 0, srows, blk, 24.0)
        check_attention(out, lse, ro, rl, f"chunk {L0}")

    at = 262144
    _log("adaptive prefill: snapshot of the first 262,144 rows, resume one chunk")
    src = torch.tensor([0], dtype=torch.int32, device="cuda")
    dst = torch.tensor([1], dtype=torch.int32, device="cuda")
    tf.snapshot_copy(plan, view, view, src, dst, at)
    torch.cuda.synchronize()
    # snapshot bytes: every copied page block equals its source; stream 1's rows past at are poison
    pool = host(P.pool)
    pb = plan.page_bytes
    pt = wl.pt
    for i in [0, 1, 255, 511]:
        a = pool[pt[0, i] * pb:(pt[0, i] + 1) * pb]
        b = pool[pt[1, i] * pb:(pt[1, i] + 1) * pb]
        assert np.array_equal(a, b), f"page {i}"
    tail = pool[pt[1, 512] * pb:(pt[1, 512] + 1) * pb].view(np.uint16)
    assert np.all(tail == NAN16)
    # resume: rows [at, at + 2048) of stream 1 from the same generator rows as stream 0
    write_rows(P, 0, 1, at, at + 2048, owner=0)
    rows = [(0, t) for t in range(at, at + 2048)]
    ld = (at + 2047) // 4 + 1
    fresh = gpu_step(plan, view, wl, 0, rows, ld, [24.0])
    resumed = gpu_step(plan, view, wl, 0, rows, ld, [24.0], stream_override=1)
    assert torch.equal(fresh[0], resumed[0])
    assert np.array_equal(fresh[2], resumed[2])
    assert torch.equal(fresh[3][0][0], resumed[3][0][0])
    assert torch.equal(fresh[3][0][1], resumed[3][0][1])
    # no poisoned byte reached the outputs
    assert not torch.isnan(resumed[3][0][0]).any()


def test_quantizing_write_chunk_full():
    _log("quantizing write: a 2,048-row chunk and its 512 keys into fp8 pages, every byte against the oracle")
    from oracle import PoolImage, Geom, quantize_rows
    pw = prefill_chunk(0)
    plan8 = tf.kv_pool_plan(tf.geom(1, pw.Dk, fp8=True))
    T = len(pw.rows)
    t0 = pw.rows[0][1]
    p0, p1 = t0 // 512, (t0 + T - 1) // 512 + 1
    pool = torch.empty((p1 - p0) * plan8.page_bytes, dtype=torch.uint8, device="cuda")
    pool.view(torch.int16).fill_(NAN16)
    pt_h = np.full((1, p1), -1, dtype=np.int32)
    pt_h[0, p0:p1] = np.random.default_rng(4).permutation(p1 - p0)
    pt = torch.from_numpy(pt_h).cuda()
    rng = np.random.default_rng(8)
    x = torch.from_numpy((rng.standard_normal((T, 512)) / 24.0).astype(np.float32)).to(torch.bfloat16)
    rope = torch.from_numpy((rng.standard_normal((T, 64)) / 24.0).astype(np.float32)).to(torch.bfloat16)
    j0, j1 = (t0 + 3) // 4, (t0 + T + 3) // 4
    keys = torch.from_numpy((rng.standard_normal((j1 - j0, pw.Dk)) / 8.0).astype(np.float32)).to(torch.bfloat16)
    rs = torch.zeros(T, dtype=torch.int32, device="cuda")
    rp = torch.arange(t0, t0 + T, dtype=torch.int32, device="cuda")
    ks = torch.zeros(j1 - j0, dtype=torch.int32, device="cuda")
    kj = torch.arange(j0, j1, dtype=torch.int32, device="cuda")
    tf.latent_write_quantize(plan8, tf.view(pool, pt, p1, p1 - p0), rs, rp, x.cuda(), rope.cuda(), ks, kj,
                             keys.cuda())
    torch.cuda.synchronize()
    codes, scale = quantize_rows(x.to(torch.float32).numpy())
    img = PoolImage(Geom(n_caches=1, index_dim=pw.Dk, fp8=True), p1 - p0, fill=NAN16)
    rope_bits = rope.view(torch.int16).numpy().view(np.uint16)
    key_bits = keys.view(torch.int16).numpy().view(np.uint16)
    for i in range(T):
        img.write_row(pt_h, p1, 0, t0 + i, 0, codes[i], rope_bits[i], scale[i])
    for i in range(j1 - j0):
        img.write_pkey(pt_h, p1, 0, j0 + i, 0, key_bits[i])
    got = host(pool)
    assert np.array_equal(got, img.buf), f"{np.count_nonzero(got != img.buf)} bytes differ"


def test_dense_chunk_full():
    """The dense pass over a 2,048-row chunk at L = 4,096 (rows [2,048, 4,096), each
    row's whole causal range: n_blocks = 1,024), in the launch configuration the bench
    times: sampled rows against the oracle at both scales, and every row equal, bit
    for bit, to the sparse pass with blocks 0 .. 1,023 selected."""
    wl = prefill_chunk(0, L=4096, T=2048, slack_pages=4)
    _log("dense chunk: populating")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    rows, nb = wl.rows, 1024
    R = len(rows)
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    blocks = torch.arange(nb, dtype=torch.int32, device="cuda").repeat(R, 1).contiguous()
    rng = np.random.default_rng(8)
    sample = sorted(set([0, 1, 1023, 2046, 2047] + rng.choice(2048, 8, replace=False).tolist()))
    srows = [rows[i] for i in sample]
    for sc in SCALES:
        out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
        tf.dense_mla_attn(plan, P.view(), rs, rp, q, sc, nb, out, lse)
        out2 = torch.empty_like(out)
        lse2 = torch.empty_like(lse)
        tf.sparse_mla_attn(plan, P.view(), rs, rp, q, sc, blocks, out2, lse2)
        torch.cuda.synchronize()
        _log(f"dense chunk: dense == sparse over every block, scale {sc:.4f}")
        assert torch.equal(out, out2) and torch.equal(lse, lse2)
        _log(f"dense chunk: oracle on {len(sample)} sampled rows")
        ro, rl = ow.dense_attention(wl, 0, srows, nb, sc)
        check_attention(host(out)[sample], host(lse)[sample], ro, rl, f"dense chunk scale {sc}")


def test_indexer_topk_blocked_chunk_full():
    """T = 2,048 rows against L = 100,000 (25,000 keys) in key blocks of 8,192, as the
    bench times it: the same blocks as the whole logits buffer and tf_topk_blocks, bit
    for bit, with 67 MB of block logits in place of 205 MB; sampled rows against the
    oracle."""
    wl = prefill_chunk(0)
    _log("blocked indexer + top-k: populating")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    rows, ld, k, B = wl.rows, 25000, wl.k, 8192
    R = len(rows)
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, P.view(), rs, rp, iq, w, logits, n_valid=nv)
    ref = torch.empty((R, k), dtype=torch.int32, device="cuda")
    tf.topk_blocks(logits, nv, k, ref)
    got = torch.empty((R, k), dtype=torch.int32, device="cuda")
    nv2 = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_topk(plan, P.view(), rs, rp, iq, w, ld, k, B, got, n_valid=nv2)
    torch.cuda.synchronize()
    _log("blocked indexer + top-k: equal to the unblocked path")
    assert torch.equal(nv, nv2)
    assert torch.equal(got, ref)
    rng = np.random.default_rng(9)
    sample = sorted(set([0, 2047] + rng.choice(2048, 6, replace=False).tolist()))
    srows = [rows[i] for i in sample]
    _log(f"blocked indexer + top-k: oracle on {len(sample)} sampled rows")
    ref_l = ow.logits(wl, 0, srows, ld)
    check_topk_against_oracle(host(got)[sample], ref_l, host(nv)[sample], k)


def test_decode_step_graph_replays():
    """The whole decode step (write, indexer, top-k, attention over 8 x 131,072 tokens)
    captured as one HIP graph: replays with three different input sets copied in
    between, and eager steps between replays, each replay equal bit for bit to the
    eager step on the same inputs. No call of the step records a memset or allocates."""
    from synth import TAG_LATENT, TAG_PKEY
    from synth.configs import LAT, ROPE, ROW
    from synth.device import _rid, fill_bf16
    wl = decode_batch(0)
    _log("decode graph: populating")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    view = P.view()
    R, ld, scale = 8, 32768, 1.0 / math.sqrt(576.0)
    sets = []
    for back in (1, 2, 3):                                  # rows at L-1, L-2, L-3
        rows = [(b, wl.lengths[b] - back) for b in range(R)]
        rs, rp, iq, w, q = query_inputs(wl, 0, rows)
        lat = torch.empty((R, LAT), dtype=torch.bfloat16, device="cuda")
        rope = torch.empty((R, ROPE), dtype=torch.bfloat16, device="cuda")
        key = torch.empty((R, wl.Dk), dtype=torch.bfloat16, device="cuda")
        for i, (b, t) in enumerate(rows):
            r0 = _rid(0, b, t)
            fill_bf16(lat[i:], 1, LAT, wl.seed, TAG_LATENT, r0 * ROW, ROW, ROW)
            fill_bf16(rope[i:], 1, ROPE, wl.seed, TAG_LATENT, r0 * ROW + LAT, ROW, ROW)
            fill_bf16(key[i:], 1, wl.Dk, wl.seed, TAG_PKEY, _rid(0, b, t // 4) * wl.Dk, wl.Dk, wl.Dk)
        kidx = torch.tensor([t // 4 for _, t in rows], dtype=torch.int32, device="cuda")
        sets.append((rs, rp, iq, w, q, lat, rope, key, kidx))
    # the step's tensors: inputs copied in from a set, outputs read after each run
    cur = [x.clone() for x in sets[0]]
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    blocks = torch.empty((R, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
    tws = torch.empty(max(1, tf.topk_workspace_bytes(R, ld, wl.k)), dtype=torch.uint8, device="cuda")
    aws = torch.empty(max(1, tf.attn_workspace_bytes(R, wl.Hq, wl.k)), dtype=torch.uint8, device="cuda")

    def step():
        rs, rp, iq, w, q, lat, rope, key, kidx = cur
        tf.latent_write(plan, view, rs, rp, lat, rope, pkey_stream=rs, pkey_idx=kidx, pkeys=key)
        tf.indexer_logits(plan, view, rs, rp, iq, w, logits, n_valid=nv)
        tf.topk_blocks(logits, nv, wl.k, blocks, ws=tws)
        tf.sparse_mla_attn(plan, view, rs, rp, q, scale, blocks, out, lse, ws=aws)

    def load(i):
        for dst, src in zip(cur, sets[i]):
            dst.copy_(src)

    def results():
        torch.cuda.synchronize()
        return [x.clone() for x in (logits, nv, blocks, out, lse)]

    want = []
    for i in range(3):
        load(i)
        step()
        want.append(results())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for n in range(9):
        i = n % 3
        load(i)
        out.fill_(7.0)
        blocks.fill_(-7)
        g.replay()
        got = results()
        _log(f"decode graph: replay {n} (inputs {i})")
        for a, b in zip(got, want[i]):
            assert torch.equal(a, b), f"replay {n}"
        if n % 2 == 1:                                      # eager work between replays
            load((i + 1) % 3)
            step()
            for a, b in zip(results(), want[(i + 1) % 3]):
                assert torch.equal(a, b), f"eager after replay {n}"


def test_candidate_selection_chunk_full():
    """Two-level selection on the prefill chunk's own logits (2,048 rows x 25,000 keys,
    as the bench times it): top-2,048 groups of 8 keys, then top-512 inside them;
    sampled rows exact against the oracle on the same fp32 values, and the logits
    left unchanged."""
    from oracle import candidate_groups as o_cand, topk_in_candidates as o_topk
    wl = prefill_chunk(0)
    _log("candidate selection, full chunk: populating")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    rows, ld = wl.rows, 25000
    R = len(rows)
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, P.view(), rs, rp, iq, w, logits, n_valid=nv)
    before = logits.clone()
    cand = torch.empty((R, 2048), dtype=torch.int32, device="cuda")
    tf.candidate_groups(logits, nv, 8, 2048, cand)
    blk = torch.empty((R, wl.k), dtype=torch.int32, device="cuda")
    tf.topk_in_candidates(logits, nv, cand, 8, wl.k, blk)
    torch.cuda.synchronize()
    assert torch.equal(logits, before)
    rng = np.random.default_rng(11)
    sample = sorted(set([0, 2047] + rng.choice(2048, 10, replace=False).tolist()))
    _log(f"candidate selection, full chunk: oracle on {len(sample)} sampled rows")
    lg = host(logits)[sample]
    nvs = host(nv)[sample]
    ref_c = o_cand(lg, nvs, 8, 2048)
    assert np.array_equal(host(cand)[sample], ref_c)
    assert np.array_equal(host(blk)[sample], o_topk(lg, nvs, ref_c, 8, wl.k))
