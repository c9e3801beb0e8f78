"""The C-ABI library on the host (no GPU): it loads, exports every entry point that
include/tf.h declares, its host-only plan and chunk rule agree with the oracle, and
argument validation refuses bad calls before any launch."""
import ctypes
import os
import re

import pytest

import attention_page_table_amd as tf
import oracle
from oracle.plan import ONE_WINDOW_FIRST, WINDOWS_FIRST, PlanNoMem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tf.h")
MiB, GiB = 1 << 20, 1 << 30


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tf_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    L = tf.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tf.SIGNATURES), "binding and header list different entry points"


@pytest.mark.parametrize("n_caches,index_dim,fp8,rope", [(1, 64, False, 64), (12, 128, False, 64),
                                                         (12, 128, True, 64), (12, 128, False, 0),
                                                         (3, 128, True, 0)])
def test_layout_matches_oracle(n_caches, index_dim, fp8, rope):
    p = tf.kv_pool_plan(tf.geom(n_caches, index_dim, fp8, rope_dim=rope))
    g = oracle.Geom(n_caches=n_caches, index_dim=index_dim, fp8=fp8, rope_dim=rope)
    L = oracle.block_layout(g)
    assert (p.off_latent, p.off_scale, p.off_rope, p.off_pkey) == (L.off_latent, L.off_scale, L.off_rope, L.off_pkey)
    assert p.cache_block_bytes == L.block and p.page_bytes == oracle.page_bytes(g)
    assert p.bytes_per_token == oracle.bytes_per_token(g)
    assert (p.lat_row_bytes, p.rope_row_bytes, p.pkey_row_bytes) == (L.lat_row, L.rope_row, L.pkey_row)


def test_pages_figures_through_the_abi():
    p = tf.kv_pool_plan(tf.geom(12, 128, rope_dim=0))
    assert p.bytes_per_token_pages == 13056
    b = tf.tf_budget(int(15.2 * GiB), 1048576, 1, 176 * MiB, 16 * GiB, 8, tf.TF_PLAN_ONE_WINDOW_FIRST)
    q = tf.kv_pool_plan(tf.geom(12, 128, rope_dim=0), b)
    assert (q.window_pages, q.total_pages) == (2049, 2056)


@pytest.mark.parametrize("policy", [ONE_WINDOW_FIRST, WINDOWS_FIRST])
def test_budget_matches_oracle(policy):
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        nc = int(rng.integers(1, 13))
        g = oracle.Geom(n_caches=nc, index_dim=128, rope_dim=int(rng.choice([0, 64])), fp8=bool(rng.integers(2)))
        room = int(rng.integers(1, 200)) * GiB + int(rng.integers(0, GiB))
        win = int(rng.integers(1, 2_000_000))
        look = int(rng.integers(0, 3))
        fixed = int(rng.integers(0, 400)) * MiB
        cap = int(rng.integers(0, 32)) * GiB
        lanes = int(rng.integers(1, 17))
        b = tf.tf_budget(room, win, look, fixed, cap, lanes, policy)
        try:
            want = oracle.kv_pool_plan(g, room, win, look, fixed, cap, lanes, policy)
        except PlanNoMem:
            with pytest.raises(tf.TFError) as e:
                tf.kv_pool_plan(tf.geom(nc, 128, g.fp8, g.rope_dim), b)
            assert e.value.status == tf.TF_E_NOMEM and "room" in str(e.value)
            continue
        got = tf.kv_pool_plan(tf.geom(nc, 128, g.fp8, g.rope_dim), b)
        assert (got.window_pages, got.n_windows, got.stream_pages, got.total_pages, got.cache_bytes,
                got.fixed_bytes) == (want.window_pages, want.n_windows, want.stream_pages, want.total_pages,
                                     want.cache_bytes, want.fixed_bytes)


def test_chunk_rule_matches_oracle():
    for L in list(range(0, 3000, 7)) + list(range(90_000, 900_000, 997)):
        assert tf.prefill_chunk(L, 10**9) == oracle.chunk_size(L)
    assert tf.prefill_chunk(389_888, 112) == 112
    assert tf.prefill_chunk(5, 0) == 0
    s, L = [], 0
    while L < 390_000:
        c = tf.prefill_chunk(L, 390_000 - L)
        s.append((L, c))
        L += c
    assert s == oracle.chunk_schedule(390_000)


def _status(fn, *args):
    return fn(*args)


def test_validation_refuses_before_launch():
    L = tf.lib()
    p = tf.kv_pool_plan(tf.geom(1, 64))
    fake = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
    v = tf.tf_kv_view(fake, None, 4, 4, 16, 0)
    # at not a multiple of 4
    assert L.tf_snapshot_copy(ctypes.byref(p), v, v, 1, fake, fake, 6, None) == tf.TF_E_INVAL
    assert "multiple of 4" in L.tf_last_error().decode()
    # at beyond the tables
    assert L.tf_snapshot_copy(ctypes.byref(p), v, v, 1, fake, fake, 4 * 512 + 4, None) == tf.TF_E_RANGE
    # cache outside the plan
    bad = tf.tf_kv_view(fake, None, 4, 4, 16, 3)
    assert L.tf_indexer_logits(ctypes.byref(p), bad, 1, fake, fake, fake, fake, 4, fake, 16, None,
                               None) == tf.TF_E_RANGE
    # heads the indexer is not built for
    assert L.tf_indexer_logits(ctypes.byref(p), v, 1, fake, fake, fake, fake, 5, fake, 16, None,
                               None) == tf.TF_E_UNSUPPORTED
    # k out of range, missing workspace
    assert L.tf_topk_blocks(fake, 100, 1, None, 0, fake, None, 0, None) == tf.TF_E_RANGE
    assert L.tf_topk_blocks(fake, 1 << 20, 1, None, 512, fake, None, 0, None) == tf.TF_E_INVAL
    assert "workspace" in L.tf_last_error().decode()
    assert L.tf_sparse_mla_attn(ctypes.byref(p), v, 8, fake, fake, fake, 33, 1.0, fake, 64, fake, None, None, 0,
                                None) == tf.TF_E_UNSUPPORTED
    assert L.tf_sparse_mla_attn(ctypes.byref(p), v, 8, fake, fake, fake, 32, -1.0, fake, 64, fake, None, None, 0,
                                None) == tf.TF_E_INVAL
    # the dense pass: extent out of range (longer contexts take the sparse path),
    # heads, missing query; no rows is a no-op
    assert L.tf_dense_mla_attn(ctypes.byref(p), v, 8, fake, fake, fake, 32, 1.0, 2049, fake, None, None, 0,
                               None) == tf.TF_E_RANGE
    assert "tf_sparse_mla_attn" in L.tf_last_error().decode()
    assert L.tf_dense_mla_attn(ctypes.byref(p), v, 8, fake, fake, fake, 32, 1.0, 0, fake, None, None, 0,
                               None) == tf.TF_E_RANGE
    assert L.tf_dense_mla_attn(ctypes.byref(p), v, 8, fake, fake, fake, 40, 1.0, 64, fake, None, None, 0,
                               None) == tf.TF_E_UNSUPPORTED
    assert L.tf_dense_mla_attn(ctypes.byref(p), v, 8, fake, fake, None, 32, 1.0, 64, fake, None, None, 0,
                               None) == tf.TF_E_INVAL
    assert L.tf_dense_mla_attn(ctypes.byref(p), v, 8, fake, fake, fake, 32, 0.0, 64, fake, None, None, 0,
                               None) == tf.TF_E_INVAL
    assert L.tf_dense_mla_attn(ctypes.byref(p), v, 8, fake, fake, fake, 32, 1.0, 1024, fake, None, None, 0,
                               None) == tf.TF_E_INVAL
    assert "workspace" in L.tf_last_error().decode()
    assert L.tf_dense_mla_attn(ctypes.byref(p), v, 0, None, None, None, 32, 1.0, 64, None, None, None, 0,
                               None) == tf.TF_OK
    # the key-blocked indexer + top-k: block size, merge capacity, workspace, heads
    assert L.tf_indexer_topk(ctypes.byref(p), v, 8, fake, fake, fake, fake, 4, 4096, 64, 200, fake, None, fake,
                             1 << 30, None) == tf.TF_E_INVAL
    assert "multiple of 128" in L.tf_last_error().decode()
    assert L.tf_indexer_topk(ctypes.byref(p), v, 8, fake, fake, fake, fake, 4, 1 << 20, 2048, 128, fake, None,
                             fake, 1 << 30, None) == tf.TF_E_RANGE
    assert "raise key_block" in L.tf_last_error().decode()
    assert L.tf_indexer_topk(ctypes.byref(p), v, 8, fake, fake, fake, fake, 4, 4096, 64, 1024, fake, None, fake,
                             16, None) == tf.TF_E_INVAL
    assert "workspace" in L.tf_last_error().decode()
    assert L.tf_indexer_topk(ctypes.byref(p), v, 8, fake, fake, fake, fake, 6, 4096, 64, 1024, fake, None, fake,
                             1 << 30, None) == tf.TF_E_UNSUPPORTED
    assert L.tf_indexer_topk(ctypes.byref(p), v, 0, None, None, None, None, 4, 4096, 64, 1024, None, None, None,
                             0, None) == tf.TF_OK
    # one block of logits, 4 blocks x 64 candidates x 8 bytes, n_c: per row
    assert tf.indexer_topk_workspace_bytes(8, 4096, 64, 1024) == 8 * 1024 * 4 + 8 * 4 * 64 * 8 + 32
    # the fused indexer + top-k: k, heads, workspace size and its 256-byte alignment
    assert L.tf_indexer_topk_fused(ctypes.byref(p), v, 8, fake, fake, fake, fake, 4, 4096, 4096, fake, None, fake,
                                   1 << 30, None) == tf.TF_E_RANGE
    assert L.tf_indexer_topk_fused(ctypes.byref(p), v, 8, fake, fake, fake, fake, 6, 4096, 64, fake, None, fake,
                                   1 << 30, None) == tf.TF_E_UNSUPPORTED
    assert L.tf_indexer_topk_fused(ctypes.byref(p), v, 8, fake, fake, fake, fake, 4, 25000, 512, fake, None, fake,
                                   1024, None) == tf.TF_E_INVAL
    assert "workspace" in L.tf_last_error().decode()
    assert L.tf_indexer_topk_fused(ctypes.byref(p), v, 8, fake, fake, fake, fake, 4, 25000, 512, fake, None,
                                   ctypes.c_void_p(0x1010), 1 << 30, None) == tf.TF_E_INVAL
    assert L.tf_indexer_topk_fused(ctypes.byref(p), v, 0, None, None, None, None, 4, 25000, 512, None, None, None,
                                   0, None) == tf.TF_OK
    # rows of at most 4,096 keys: their logits and n_c; longer rows: the sample (an
    # sixteenth of the pages, at least 16 pages), thresholds, n_c and the candidate regions,
    # less than the logits (a third of them at 2,048 rows x 25,000 keys)
    assert tf.indexer_topk_fused_workspace_bytes(8, 4096, 64, 4) == 8 * 4096 * 4 + 256
    # few rows of more than 4,096 keys scored whole: the top-k's blocked mode has its own
    # workspace inside
    assert tf.indexer_topk_fused_workspace_bytes(13, 10000, 2048, 16) >= 13 * 10000 * 4 + tf.topk_workspace_bytes(
        13, 10000, 2048) > 13 * 10000 * 4
    # fewer than 64 rows of at most 262,144 keys are scored whole too; more rows, or
    # longer ones, take the sample and the filtered pass
    assert tf.indexer_topk_fused_workspace_bytes(8, 25000, 512, 16) >= 8 * 25000 * 4
    assert tf.indexer_topk_fused_workspace_bytes(8, 300000, 512, 16) < 8 * 300000 * 4
    assert tf.indexer_topk_fused_workspace_bytes(64, 25000, 512, 16) < 64 * 25000 * 4
    assert tf.indexer_topk_fused_workspace_bytes(2048, 25000, 512, 16) < 2048 * 25000 * 4 / 3
    # two-level candidate selection: group size, candidate count, bitmap capacity, workspace
    assert L.tf_candidate_groups(fake, 25000, 8, None, 0, 2048, fake, fake, 1 << 30, None) == tf.TF_E_RANGE
    assert L.tf_candidate_groups(fake, 25000, 8, None, 8, 4096, fake, fake, 1 << 30, None) == tf.TF_E_RANGE
    assert L.tf_candidate_groups(fake, 25000, 8, None, 8, 2048, fake, fake, 16, None) == tf.TF_E_INVAL
    assert "workspace" in L.tf_last_error().decode()
    assert L.tf_candidate_groups(fake, 25000, 0, None, 8, 2048, None, None, 0, None) == tf.TF_OK
    assert L.tf_topk_in_candidates(fake, 25000, 8, None, fake, 0, 8, 512, fake, fake, 1 << 30,
                                   None) == tf.TF_E_RANGE
    assert L.tf_topk_in_candidates(fake, 25000, 8, None, fake, 2048, 65, 512, fake, fake, 1 << 30,
                                   None) == tf.TF_E_RANGE
    assert L.tf_topk_in_candidates(fake, 25000, 8, None, None, 2048, 8, 512, fake, fake, 1 << 30,
                                   None) == tf.TF_E_INVAL
    # null plan, null pool
    assert L.tf_latent_write(None, v, 1, fake, fake, fake, None, fake, 0, None, None, None, None) == tf.TF_E_INVAL
    nv = tf.tf_kv_view(None, None, 4, 4, 16, 0)
    assert L.tf_latent_write(ctypes.byref(p), nv, 1, fake, fake, fake, None, fake, 0, None, None, None,
                             None) == tf.TF_E_INVAL
    # the quantizing write needs an fp8 plan, and its latent rows
    assert L.tf_latent_write_quantize(ctypes.byref(p), v, 1, fake, fake, fake, fake, 0, None, None, None,
                                      None) == tf.TF_E_INVAL
    assert "TF_LAT_FP8E4M3_ROWSCALE" in L.tf_last_error().decode()
    p8 = tf.kv_pool_plan(tf.geom(1, 64, True))
    assert L.tf_latent_write_quantize(ctypes.byref(p8), v, 1, fake, fake, None, fake, 0, None, None, None,
                                      None) == tf.TF_E_INVAL
    assert "latent" in L.tf_last_error().decode()
    assert L.tf_latent_write_quantize(ctypes.byref(p8), v, 0, None, None, None, None, 0, None, None, None,
                                      None) == tf.TF_OK
    # bad geometry
    with pytest.raises(tf.TFError) as e:
        tf.kv_pool_plan(tf.geom(1, 96))
    assert e.value.status == tf.TF_E_UNSUPPORTED
    # a successful call clears the message
    assert L.tf_topk_blocks(fake, 100, 0, None, 4, fake, None, 0, None) == tf.TF_OK
    assert L.tf_last_error().decode() == ""


def test_page_table_check_refuses_ids_outside_the_pool():
    """A host copy of a page table is refused before any launch when it names a page
    outside [0, n_pages); -1 (no page yet) is accepted."""
    import numpy as np
    L = tf.lib()
    pt = np.array([[3, 0, -1, 2], [1, 4, 5, 6]], dtype=np.int32)
    tf.check_page_table(pt, 7)
    assert L.tf_last_error().decode() == ""
    with pytest.raises(tf.TFError) as e:
        tf.check_page_table(pt, 6)                         # page 6 is past a 6-page pool
    assert e.value.status == tf.TF_E_RANGE
    assert "stream 1 page index 3 names page 6" in str(e.value)
    bad = pt.copy()
    bad[0, 1] = -2
    with pytest.raises(tf.TFError) as e:
        tf.check_page_table(bad, 7)
    assert e.value.status == tf.TF_E_RANGE and "stream 0 page index 1" in str(e.value)
    assert L.tf_check_page_table(None, 1, 1, 1) == tf.TF_E_INVAL
    assert L.tf_check_page_table(pt.ctypes.data, 2, 4, 0) == tf.TF_E_INVAL
    # the binding's view checks a host copy when one is given
    with pytest.raises(tf.TFError):
        tf.view(None, None, 4, 6, pt_host=pt)


def test_noalloc_sparse_pass_refuses_beyond_its_scratch():
    """The allocation-free sparse pass refuses, before any launch, a call whose split
    partials exceed its fixed scratch (no pointer is dereferenced)."""
    L = tf.lib()
    p = tf.kv_pool_plan(tf.geom(1, 64))
    fake = ctypes.c_void_p(0x1000)
    v = tf.tf_kv_view(fake, None, 4, 4, 16, 0)
    cap = tf.sparse_mla_attn_noalloc_max_bytes()
    assert cap == 32 << 20
    assert tf.attn_workspace_bytes(4096, 16, 2048) > cap
    assert L.tf_sparse_mla_attn_noalloc(ctypes.byref(p), v, 4096, fake, fake, fake, 16, 1.0, fake, 2048, fake, None,
                                        None) == tf.TF_E_RANGE
    assert "fixed scratch" in L.tf_last_error().decode()
    assert L.tf_sparse_mla_attn_noalloc(ctypes.byref(p), v, 8, fake, fake, fake, 33, 1.0, fake, 64, fake, None,
                                        None) == tf.TF_E_UNSUPPORTED
    assert L.tf_sparse_mla_attn_noalloc(ctypes.byref(p), v, 0, None, None, None, 32, 1.0, None, 64, None, None,
                                        None) == tf.TF_OK
