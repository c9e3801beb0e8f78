"""Pins of the oracle's top-k: brute force by a stable sort on tiny rows, the blocked
merge identity of chunked-prefill-memory section 2.3, ties, signed zeros, ragged rows."""
import numpy as np

from oracle import topk_blocks
from oracle.topk import topk_row


def brute(vals, n, k):
    # pure Python: every index, sorted by (value desc, index asc)
    cand = sorted(range(n), key=lambda j: (-(float(vals[j]) + 0.0), j))[:k]
    return sorted(cand) + [-1] * (k - len(cand))


def test_brute_force_small_rows_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 45))
        vals = rng.integers(-4, 5, size=n).astype(float)   # many ties
        assert list(topk_row(vals, n, k)) == brute(vals, n, k), (trial, n, k)


def test_ties_go_to_lower_index():
    assert list(topk_row(np.ones(10), 10, 3)) == [0, 1, 2]
    v = np.array([5.0, 1.0, 5.0, 5.0, 0.0])
    assert list(topk_row(v, 5, 2)) == [0, 2]


def test_signed_zero_is_one_value():
    v = np.array([-0.0, 0.0, -0.0, 0.0, -1.0])
    assert list(topk_row(v, 5, 2)) == [0, 1]
    assert list(topk_row(np.array([0.0, -0.0]), 2, 1)) == [0]


def test_ragged_rows_pad_with_minus_one():
    v = np.array([[3.0, 1.0, 2.0, 9.0, 9.0], [1.0, 2.0, 3.0, 4.0, 5.0]])
    out = topk_blocks(v, [3, 5], 4)
    assert out[0].tolist() == [0, 1, 2, -1]       # entries past n_valid are never read
    assert out[1].tolist() == [1, 2, 3, 4]


def test_output_ascending_and_is_the_largest():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(1000)
    s = topk_row(v, 1000, 64)
    assert np.all(np.diff(s) > 0)
    thr = np.sort(v)[-64]
    assert set(s.tolist()) == set(np.nonzero(v >= thr)[0].tolist())


def test_blocked_merge_identity():
    """topk(union) == topk(union of per-block topk), exactly, for several key-block sizes."""
    rng = np.random.default_rng(2)
    for n, k, B in [(5000, 512, 1024), (25000, 512, 4096), (3000, 64, 100), (2000, 512, 32768)]:
        v = np.round(rng.standard_normal(n), 2)            # ties across blocks
        cand = []
        for b0 in range(0, n, B):
            sel = topk_row(v[b0:b0 + B], min(B, n - b0), k)
            cand.extend((sel[sel >= 0] + b0).tolist())
        cand = np.array(sorted(cand))
        sub = topk_row(v[cand], cand.size, k)
        merged = cand[sub[sub >= 0]]
        direct = topk_row(v, n, k)
        assert np.array_equal(np.sort(merged), direct[direct >= 0])
