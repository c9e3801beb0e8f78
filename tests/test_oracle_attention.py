"""Pins of the oracle's sparse absorbed-MLA attention: dense attention when every block
is selected (a textbook definition in pure Python), closed forms, the absorbed-MLA
identity against plain multi-head attention, the causal mask inside the last block."""
import math

import numpy as np

from oracle import dense_mla, dense_mla_row, dense_tokens, selected_tokens, sparse_mla_row
from oracle.fp8 import e4m3_decode


def rows_from(lat, rope):
    return lambda S: (lat[S], rope[S])


def dense_textbook(q, lat, rope, t, scale):
    """Causal softmax attention of one query over tokens 0..t, in pure Python."""
    Hq = len(q)
    out, lses = [], []
    for h in range(Hq):
        z = []
        for s in range(t + 1):
            key = list(lat[s]) + list(rope[s])
            z.append(scale * math.fsum(float(a) * float(b) for a, b in zip(q[h], key)))
        m = max(z)
        e = [math.exp(x - m) for x in z]
        tot = math.fsum(e)
        o = [math.fsum(e[s] / tot * float(lat[s][d]) for s in range(t + 1)) for d in range(len(lat[0]))]
        out.append(o)
        lses.append(m + math.log(tot))
    return np.array(out), np.array(lses)


def test_all_blocks_equal_dense():
    rng = np.random.default_rng(0)
    lat = rng.standard_normal((16, 512)) / 24
    rope = rng.standard_normal((16, 64)) / 24
    q = rng.standard_normal((2, 576)) / 24
    for t in (0, 5, 13, 15):
        for scale in (1 / 24, 24.0):
            blocks = list(range(t // 4 + 1)) + [-1, -1]
            o, l = sparse_mla_row(q, rows_from(lat, rope), blocks, t, scale)
            od, ld = dense_textbook(q, lat, rope, t, scale)
            assert np.allclose(o, od, rtol=1e-12, atol=1e-15)
            assert np.allclose(l, ld, rtol=1e-12)


def test_one_token_context_returns_its_row():
    rng = np.random.default_rng(1)
    lat = rng.standard_normal((4, 512))
    rope = rng.standard_normal((4, 64))
    q = rng.standard_normal((3, 576))
    o, l = sparse_mla_row(q, rows_from(lat, rope), [0], 0, 1.7)
    assert np.array_equal(o, np.repeat(lat[:1], 3, axis=0))
    assert np.allclose(l, 1.7 * (q @ np.concatenate([lat[0], rope[0]])))


def test_zero_query_gives_mean_of_selected_rows():
    rng = np.random.default_rng(2)
    lat = rng.standard_normal((64, 512))
    rope = rng.standard_normal((64, 64))
    blocks = [2, 7, 11]
    t = 45                               # block 11 holds 44..47: 46 and 47 are masked
    o, l = sparse_mla_row(np.zeros((2, 576)), rows_from(lat, rope), blocks, t, 5.0)
    S = [8, 9, 10, 11, 28, 29, 30, 31, 44, 45]
    assert selected_tokens(blocks, t).tolist() == S
    assert np.allclose(o, lat[S].mean(axis=0)[None, :], rtol=1e-13)
    assert np.allclose(l, math.log(len(S)))


def test_block_order_and_padding_do_not_matter():
    rng = np.random.default_rng(3)
    lat = rng.standard_normal((100, 512))
    rope = rng.standard_normal((100, 64))
    q = rng.standard_normal((4, 576)) / 10
    a = sparse_mla_row(q, rows_from(lat, rope), [3, 9, 20, -1], 99, 0.3)
    b = sparse_mla_row(q, rows_from(lat, rope), [-1, 20, 3, 9], 99, 0.3)
    assert np.allclose(a[0], b[0], rtol=1e-13) and np.allclose(a[1], b[1], rtol=1e-13)


def test_empty_selection():
    o, l = sparse_mla_row(np.ones((2, 576)), lambda S: None, [-1, -1], 10, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_absorbed_identity_against_plain_mha():
    """Absorbed MLA (query folded through W_UK, output through W_UV afterwards) equals
    plain multi-head attention with per-head keys W_UK c_s (+ shared rope) and values W_UV c_s."""
    rng = np.random.default_rng(4)
    Hq, dn, dv, n = 3, 24, 20, 40
    lat = rng.standard_normal((n, 512)) / 20
    rope = rng.standard_normal((n, 64)) / 20
    W_UK = rng.standard_normal((Hq, dn, 512)) / 20
    W_UV = rng.standard_normal((Hq, dv, 512)) / 20
    q_nope = rng.standard_normal((Hq, dn))
    q_rope = rng.standard_normal((Hq, 64))
    scale, t = 0.9, n - 1
    blocks = list(range(n // 4))
    # plain MHA over all tokens 0..t
    ref = np.zeros((Hq, dv))
    for h in range(Hq):
        K = lat @ W_UK[h].T                      # [n, dn]
        V = lat @ W_UV[h].T                      # [n, dv]
        z = scale * (K @ q_nope[h] + rope @ q_rope[h])
        p = np.exp(z - z.max())
        p /= p.sum()
        ref[h] = p @ V
    q_abs = np.concatenate([np.einsum("hdk,hd->hk", W_UK, q_nope), q_rope], axis=1)
    o, _ = sparse_mla_row(q_abs, rows_from(lat, rope), blocks, t, scale)
    got = np.einsum("hvk,hk->hv", W_UV, o)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-14)


def test_scale_enters_the_exponent():
    rng = np.random.default_rng(5)
    lat = rng.standard_normal((8, 512))
    rope = rng.standard_normal((8, 64))
    q = rng.standard_normal((1, 576))
    # two tokens: p1 / p0 = exp(scale * (z1 - z0))
    o, _ = sparse_mla_row(q, rows_from(lat, rope), [0], 1, 0.25)
    K = np.concatenate([lat[:2], rope[:2]], axis=1)
    z = 0.25 * (K @ q[0])
    p1 = 1 / (1 + math.exp(z[0] - z[1]))
    assert np.allclose(o[0], (1 - p1) * lat[0] + p1 * lat[1], rtol=1e-12)


def test_e4m3_decode_all_codes_against_torch():
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


# ---- dense pass: causal attention over the first n_blocks pooled blocks ----------------

def test_dense_equals_textbook_causal_attention():
    rng = np.random.default_rng(10)
    lat = rng.standard_normal((24, 512)) / 24
    rope = rng.standard_normal((24, 64)) / 24
    q = rng.standard_normal((2, 576)) / 24
    for t, n_blocks in ((0, 1), (6, 2), (6, 6), (13, 4), (23, 6), (23, 3), (17, 1)):
        last = min(t, 4 * n_blocks - 1)           # the extent cuts the causal range
        for scale in (1 / 24, 24.0):
            o, l = dense_mla_row(q, rows_from(lat, rope), t, n_blocks, scale)
            od, ld = dense_textbook(q, lat, rope, last, scale)
            assert np.allclose(o, od, rtol=1e-12, atol=1e-15), (t, n_blocks, scale)
            assert np.allclose(l, ld, rtol=1e-12), (t, n_blocks, scale)


def test_dense_equals_sparse_with_the_same_blocks_selected():
    rng = np.random.default_rng(11)
    lat = rng.standard_normal((40, 512))
    rope = rng.standard_normal((40, 64))
    q = rng.standard_normal((3, 576)) / 24
    for t, n_blocks in ((39, 10), (39, 4), (21, 8), (2, 1)):
        o, l = dense_mla_row(q, rows_from(lat, rope), t, n_blocks, 2.0)
        os_, ls = sparse_mla_row(q, rows_from(lat, rope), list(range(n_blocks)), t, 2.0)
        assert np.allclose(o, os_, rtol=1e-12, atol=1e-14)
        assert np.allclose(l, ls, rtol=1e-12)


def test_dense_closed_forms():
    rng = np.random.default_rng(12)
    lat = rng.standard_normal((32, 512))
    rope = rng.standard_normal((32, 64))
    q = rng.standard_normal((2, 576))
    # one visible token: its own row, lse = its score
    o, l = dense_mla_row(q, rows_from(lat, rope), 0, 5, 0.3)
    assert np.array_equal(o, np.repeat(lat[:1], 2, axis=0))
    assert np.allclose(l, 0.3 * (q @ np.concatenate([lat[0], rope[0]])))
    # zero query: the mean of the visible rows, lse = ln(count)
    for t, n_blocks, count in ((30, 8, 31), (30, 3, 12)):
        o, l = dense_mla_row(np.zeros((2, 576)), rows_from(lat, rope), t, n_blocks, 7.0)
        assert np.allclose(o, lat[:count].mean(axis=0)[None, :], rtol=1e-13)
        assert np.allclose(l, math.log(count))
    # a row before the stream's start sees nothing
    o, l = dense_mla_row(q, rows_from(lat, rope), -1, 4, 1.0)
    assert not o.any() and np.all(l == -np.inf)
    assert dense_tokens(9, 2).tolist() == list(range(8))
    assert dense_tokens(9, 3).tolist() == list(range(10))


def test_dense_rows_follow_their_own_streams_and_positions():
    rng = np.random.default_rng(13)
    lat = rng.standard_normal((2, 20, 512))
    rope = rng.standard_normal((2, 20, 64))
    q = rng.standard_normal((3, 2, 576)) / 24
    streams, pos = [1, 0, 1], [19, 7, 3]
    o, l = dense_mla(q, lambda r, S: (lat[streams[r]][S], rope[streams[r]][S]), pos, 5, 1.5)
    for r in range(3):
        od, ld = dense_textbook(q[r], lat[streams[r]], rope[streams[r]], pos[r], 1.5)
        assert np.allclose(o[r], od, rtol=1e-12, atol=1e-15)
        assert np.allclose(l[r], ld, rtol=1e-12)
