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


# ---- two-level candidate selection: groups of g keys, top-n_cand groups, then top-k ----

from oracle import candidate_groups, topk_in_candidates  # noqa: E402


def test_candidates_worked_example():
    # 19 visible keys in groups of 8: {0..7}, {8..15}, {16..18} (key 19 is not visible)
    v = np.array([0, 1, 2, 3, 4, 5, 6, 7,  9, 0, 0, 0, 0, 0, 0, 0,  8, 8, 1, 99], dtype=float)
    # group scores 7, 9, 8 -> the best group is 1, the best two are 1 and 2
    assert candidate_groups(v[None], [19], 8, 1).tolist() == [[1]]
    assert candidate_groups(v[None], [19], 8, 2).tolist() == [[1, 2]]
    assert candidate_groups(v[None], [19], 8, 5).tolist() == [[0, 1, 2, -1, -1]]
    # inside groups 1 and 2 the top three keys are 8 (9), 16 and 17 (8 each)
    assert topk_in_candidates(v[None], [19], [[1, 2]], 8, 3).tolist() == [[8, 16, 17]]
    # only group 1 kept: its key 8 (9), then its zeros by index (9, 10)
    assert topk_in_candidates(v[None], [19], [[1, -1]], 8, 3).tolist() == [[8, 9, 10]]
    # more keys wanted than the candidates hold: the -inf keys follow by index
    assert topk_in_candidates(v[None], [19], [[2]], 8, 5).tolist() == [[0, 1, 16, 17, 18]]


def test_group_of_one_is_plain_topk():
    rng = np.random.default_rng(5)
    v = rng.integers(-3, 4, size=(6, 50)).astype(float)
    nv = [50, 49, 17, 1, 30, 8]
    for k in (1, 5, 20, 60):
        assert np.array_equal(candidate_groups(v, nv, 1, k), topk_blocks(v, nv, k))


def test_all_groups_candidates_is_plain_topk():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((5, 64))
    nv = [64, 63, 9, 40, 1]
    cand = candidate_groups(v, nv, 8, 8)                 # every group of every row
    for k in (1, 7, 30):
        assert np.array_equal(topk_in_candidates(v, nv, cand, 8, k), topk_blocks(v, nv, k))


def test_candidates_brute_force_with_ties():
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(1, 60))
        g = int(rng.choice([1, 2, 3, 8]))
        nc = int(rng.integers(1, 10))
        k = int(rng.integers(1, 20))
        vals = rng.integers(-3, 4, size=n).astype(float)
        scores = [max(float(vals[j]) for j in range(s, min(s + g, n))) for s in range(0, n, g)]
        cand = brute(scores, len(scores), nc)
        assert candidate_groups(vals[None], [n], g, nc)[0].tolist() == cand, trial
        masked = [float(vals[j]) if j // g in cand else -np.inf for j in range(n)]
        assert topk_in_candidates(vals[None], [n], [cand], g, k)[0].tolist() == brute(masked, n, k), trial
