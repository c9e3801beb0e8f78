"""Pins of the oracle's indexer logits: closed forms, special cases, and an exact
rational brute force on tiny inputs (chunked-prefill-memory section 1)."""
from fractions import Fraction

import numpy as np

from oracle import indexer_logits, n_compressed


def test_compressed_length():
    # the pooled block holding t is visible: t = 0..3 -> 1 key, t = 4 -> 2 keys
    assert [n_compressed(t) for t in range(9)] == [1, 1, 1, 1, 2, 2, 2, 2, 3]
    assert n_compressed(131071) == 32768
    assert n_compressed(99999) == 25000


def test_one_head_self_key_is_squared_norm():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 16))
    keys = [np.concatenate([q[0], rng.standard_normal((3, 16))])]
    l = indexer_logits(q, np.ones((1, 1)), keys, [15], ld=4)
    assert np.isclose(l[0, 0], float(q[0, 0] @ q[0, 0]), rtol=1e-15)


def test_all_nonpositive_scores_give_zero():
    rng = np.random.default_rng(2)
    q = np.abs(rng.standard_normal((1, 3, 8)))
    keys = [-np.abs(rng.standard_normal((5, 8)))]
    l = indexer_logits(q, rng.standard_normal((1, 3)), keys, [19], ld=5)
    assert np.all(l == 0.0)


def test_relu_is_per_head_before_weighting():
    # head 0 scores +0.5, head 1 scores -0.3: the sum is 0.5, not 0.2 and not relu(0.2)
    q = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    keys = [np.array([[0.5, -0.3]])]
    l = indexer_logits(q, np.array([[1.0, 1.0]]), keys, [0], ld=1)
    assert l[0, 0] == 0.5
    # negative weight on the positive head gives a negative logit
    l = indexer_logits(q, np.array([[-2.0, 7.0]]), keys, [0], ld=1)
    assert l[0, 0] == -1.0


def test_mask_by_compressed_length():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 2, 4))
    keys = [rng.standard_normal((8, 4))] * 3
    l = indexer_logits(q, np.ones((3, 2)), keys, [3, 4, 30], ld=8)
    assert np.isfinite(l[0, 0]) and np.all(np.isneginf(l[0, 1:]))
    assert np.all(np.isfinite(l[1, :2])) and np.all(np.isneginf(l[1, 2:]))
    assert np.all(np.isfinite(l[2, :8]))


def test_exact_rational_brute_force():
    """Small-integer inputs with H != D != n, computed exactly with Fractions in pure
    Python loops: catches a transposed operand, a wrong head index or a dropped term."""
    rng = np.random.default_rng(4)
    R, H, D, n = 3, 3, 5, 7
    q = rng.integers(-3, 4, size=(R, H, D))
    w = rng.integers(-2, 3, size=(R, H))
    keys = [rng.integers(-3, 4, size=(n, D)) for _ in range(R)]
    pos = [27, 9, 13]
    ld = 8
    got = indexer_logits(q.astype(float), w.astype(float), [k.astype(float) for k in keys], pos, ld)
    for r in range(R):
        nc = pos[r] // 4 + 1
        for j in range(ld):
            if j >= min(nc, n):
                if j >= nc:
                    assert np.isneginf(got[r, j])
                continue
            total = Fraction(0)
            for h in range(H):
                dot = sum(Fraction(int(q[r, h, i])) * int(keys[r][j, i]) for i in range(D))
                total += int(w[r, h]) * max(dot, Fraction(0))
            assert got[r, j] == float(total)


def test_row_batches_equal_single_pass():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((10, 4, 16))
    w = rng.standard_normal((10, 4))
    keys = [rng.standard_normal((40, 16))] * 10
    pos = list(range(100, 110))
    one = indexer_logits(q, w, keys, pos, 40)
    two = np.concatenate([indexer_logits(q[:4], w[:4], keys[:4], pos[:4], 40),
                          indexer_logits(q[4:], w[4:], keys[4:], pos[4:], 40)])
    assert np.array_equal(one, two)
