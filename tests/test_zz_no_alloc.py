"""The allocation-free sparse pass (tf_sparse_mla_attn_noalloc) against the sparse pass
with a caller's workspace, through the C ABI: bit for bit, on two calls in a row (the
second smaller), decode rows whose block lists are split over workgroups and merged
(the split partials are what the fixed scratch holds)."""
import math

import numpy as np
import pytest
import torch

import attention_page_table_amd as tf
from synth.configs import tiny
from synth.device import alloc_pool, populate, query_inputs

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _rows_and_blocks(wl, rows, k, seed):
    rng = np.random.default_rng(seed)
    blk = np.full((len(rows), k), -1, dtype=np.int32)
    for r, (_, t) in enumerate(rows):
        n = min(k, t // 4 + 1)
        blk[r, :n] = np.sort(rng.choice(t // 4 + 1, n, replace=False))
    return torch.from_numpy(blk).cuda()


def test_noalloc_equals_workspace_call_twice():
    import copy
    wl = copy.copy(tiny(0))
    wl.Hq = 32
    plan = tf.kv_pool_plan(tf.geom(1, wl.Dk))
    P = alloc_pool(wl, plan)
    populate(P)
    cases = [
        # decode rows, 512 blocks each: the block lists split over workgroups, then merged
        ([(0, 2047), (1, 2047), (1, 1500), (0, 1030), (1, 64), (0, 2000)], 512, 24.0),
        # a smaller second call: fewer rows, fewer blocks
        ([(1, 2047), (0, 900)], 96, 1.0 / math.sqrt(576.0)),
    ]
    for i, (rows, k, scale) in enumerate(cases):
        _log(f"no-alloc sparse pass, call {i + 1}: {len(rows)} rows, k {k}")
        need = tf.attn_workspace_bytes(len(rows), wl.Hq, k)
        assert 0 < need <= tf.sparse_mla_attn_noalloc_max_bytes()
        rs, rp, _, _, q = query_inputs(wl, 0, rows)
        blocks = _rows_and_blocks(wl, rows, k, seed=i)
        R = len(rows)
        ref_o = torch.full((R, wl.Hq, 512), 7.0, dtype=torch.float32, device="cuda")
        ref_l = torch.full((R, wl.Hq), 7.0, dtype=torch.float32, device="cuda")
        tf.sparse_mla_attn(plan, P.view(), rs, rp, q, scale, blocks, ref_o, ref_l)
        got_o = torch.full_like(ref_o, -7.0)
        got_l = torch.full_like(ref_l, -7.0)
        tf.sparse_mla_attn_noalloc(plan, P.view(), rs, rp, q, scale, blocks, got_o, got_l)
        torch.cuda.synchronize()
        assert not torch.isnan(ref_o).any()
        assert torch.equal(got_o, ref_o), f"call {i + 1}: outputs differ"
        assert torch.equal(got_l, ref_l), f"call {i + 1}: log-sum-exp differs"
