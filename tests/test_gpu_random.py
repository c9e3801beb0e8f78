"""GPU parity over seeded random shapes: each case draws 1-4 streams with ragged
lengths (from a single token to several pages), a shuffled page table with slack
pages and unused slots, bf16 or fp8 rows, indexer heads and width, attention heads
(including ones that fill no whole head group), k and the query rows: decode-like
(one row per stream, at its last position), a chunk (consecutive positions of one
stream, 64 rows or more, so the tile kernels run) or a scatter (any stream, any
position, including position 0). Through the C ABI, each case checks:
* n_valid and the logits against the oracle (the logit tolerance);
* the top-k bit for bit against an exact top-k of the GPU's own logits, and within
  the gap rule of the oracle's top-k;
* attention against the oracle run on the GPU's block sets;
* the fused indexer + top-k equal to the pair, bit for bit.
The cases are drawn from fixed seeds; the logits' row length ld has random slack
past the longest row's keys."""
import math

import numpy as np
import pytest
import torch

import attention_page_table_amd as tf
from oracle import workload as ow
from synth.configs import PAGE_ROWS, Workload
from synth.device import alloc_pool, populate, query_inputs
from tests.gpu_common import (check_attention, check_logits, check_topk_against_oracle, host, logits_bound,
                              topk_on_values)

pytestmark = pytest.mark.gpu
CASES = 15
SCALES = [1.0 / math.sqrt(576.0), 24.0]


def _log(msg):
    print(msg, flush=True)


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    S = int(rng.integers(1, 5))
    lengths = [int(rng.choice([1, 3, 4, 5, 511, 512, 513, 2047, 2048, 3001, 4096, 5555])) for _ in range(S)]
    per = [(L + PAGE_ROWS - 1) // PAGE_ROWS for L in lengths]
    stride = max(per) + int(rng.integers(0, 3))       # unused table slots read -1
    n_pages = sum(per) + int(rng.integers(0, 4))      # slack pages no table names
    perm = rng.permutation(n_pages).astype(np.int32)
    pt = np.full((S, stride), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(per):
        pt[b, :n] = perm[o:o + n]
        o += n
    H = int(rng.choice([4, 8, 16]))
    Dk = int(rng.choice([64, 128]))
    Hq = int(rng.choice([8, 16, 20, 32]))
    k = int(rng.choice([1, 7, 64, 200, 512]))
    kind = ["decode", "chunk", "scatter"][seed % 3]
    if kind == "decode":
        rows = [(b, lengths[b] - 1) for b in range(S)]
    elif kind == "chunk":
        b = int(np.argmax(lengths))
        T = min(lengths[b], int(rng.choice([64, 80, 130])))
        rows = [(b, t) for t in range(lengths[b] - T, lengths[b])]
    else:
        n = int(rng.choice([3, 63, 64, 90]))
        rows = []
        for _ in range(n):
            b = int(rng.integers(0, S))
            rows.append((b, int(rng.choice([0, lengths[b] - 1, int(rng.integers(0, lengths[b]))]))))
    fp8 = bool(rng.integers(0, 3) == 0)
    wl = Workload(f"random_{seed}", seed, 1, S, lengths, H=H, Dk=Dk, Hq=Hq, k=k, n_pages=n_pages, pt=pt,
                  fp8=fp8, w_d=float(H), rows=rows, description=f"seeded random case {seed} ({kind})")
    ld = max(t // 4 + 1 for _, t in rows) + int(rng.integers(0, 40))
    scale = SCALES[seed % 2]
    return wl, kind, ld, scale


@pytest.mark.parametrize("seed", range(CASES))
def test_random_step(seed):
    wl, kind, ld, scale = _case(seed)
    rows = wl.rows
    R = len(rows)
    _log(f"random case {seed}: {kind}, {wl.n_streams} streams {wl.lengths}, {R} rows, H={wl.H} Dk={wl.Dk} "
         f"Hq={wl.Hq} k={wl.k} ld={ld} {'fp8' if wl.fp8 else 'bf16'}")
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk, fp8=wl.fp8))
    P = alloc_pool(wl, plan)
    populate(P)
    view = P.view()
    rs, rp, iq, w, q = query_inputs(wl, 0, rows)
    logits = torch.empty((R, ld), dtype=torch.float32, device="cuda")
    nv = torch.empty(R, dtype=torch.int32, device="cuda")
    tf.indexer_logits(plan, view, rs, rp, iq, w, logits, n_valid=nv)
    blocks = torch.empty((R, wl.k), dtype=torch.int32, device="cuda")
    tf.topk_blocks(logits, nv, wl.k, blocks)
    out = torch.empty((R, wl.Hq, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, wl.Hq), dtype=torch.float32, device="cuda")
    tf.sparse_mla_attn(plan, view, rs, rp, q, scale, blocks, out, lse)
    fb = torch.full((R, wl.k), -7, dtype=torch.int32, device="cuda")
    fnv = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    tf.indexer_topk_fused(plan, view, rs, rp, iq, w, ld, wl.k, fb, n_valid=fnv)
    torch.cuda.synchronize()
    lg, n_v, blk = host(logits), host(nv), host(blocks)
    assert np.array_equal(n_v, ow.n_valid(rows, ld))
    ref_l = ow.logits(wl, 0, rows, ld)
    check_logits(lg, ref_l, logits_bound(wl, 0, rows, ld), f"case {seed}")
    assert np.array_equal(blk, topk_on_values(lg, n_v, wl.k))
    check_topk_against_oracle(blk, ref_l, n_v, wl.k)
    ro, rl = ow.attention(wl, 0, rows, blk, scale)
    check_attention(host(out), host(lse), ro, rl, f"case {seed}")
    assert torch.equal(fnv, nv) and torch.equal(fb, blocks), f"case {seed}: fused differs from the pair"
