"""Shared helpers of the GPU parity tests: tolerances and host copies.

The tolerances are the ones the method's target states:
* page mapping, writes, snapshots, top-k on the same logits: bit-exact;
* logits: |g - r| <= 1e-4 |r| + 1e-5 A, A = sum_h |w_h| sum_i |q_hi k_ji|: the
  1e-4 relative bound, with an absolute floor where signed weights cancel to ~0;
* top-k against the oracle's own logits: equal sets wherever the k-th and
  (k+1)-th logits differ by more than 1e-3 relative; any differing block lies
  within 1e-3 relative of the k-th value;
* attention: relative L2 <= 1e-3 over each row's heads x 512 values and
  max-abs <= 5e-3, against the oracle run on the GPU's own block sets.
"""
from __future__ import annotations

import numpy as np
import torch

from synth import bf16_to_f64


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return bf16_to_f64(host(t.view(torch.int16)).view(np.uint16))


def logits_bound(wl, c, rows, ld, keys=None):
    """A[r, j] of the logit tolerance (fp64)."""
    from oracle import workload as ow
    q = np.abs(bf16_to_f64(wl.iq_bits(c, rows)))
    w = np.abs(wl.weights(c, rows).astype(np.float64))
    if keys is None:
        keys = ow.row_keys(wl, c, rows, ld)
    out = np.zeros((len(rows), ld))
    for r, (b, t) in enumerate(rows):
        n = min(t // 4 + 1, ld)
        k = np.abs(keys[r][:n])
        out[r, :n] = w[r] @ (q[r] @ k.T)
    return out


def check_logits(got, ref, A, rows_label=""):
    got = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"mask differs {rows_label}"
    assert not np.isnan(got).any(), f"NaN in logits {rows_label}"
    err = np.abs(got[fin] - ref[fin])
    bound = 1e-4 * np.abs(ref[fin]) + 1e-5 * A[fin]
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} logits out of tolerance {rows_label}; worst {np.max(err - bound):.3e}"


def topk_on_values(vals: np.ndarray, n_valid: np.ndarray, k: int) -> np.ndarray:
    """Exact top-k (value desc, index asc; -0 == +0) of the given fp32 rows, ascending, -1 padded."""
    from oracle import topk_blocks
    return topk_blocks(vals.astype(np.float64), n_valid, k)


def check_topk_against_oracle(got_blocks, ref_logits, n_valid, k):
    """The target's rule: sets equal where the k-th / (k+1)-th gap exceeds 1e-3 relative;
    otherwise every differing block is within 1e-3 relative of the k-th value."""
    from oracle import topk_blocks
    ref = topk_blocks(ref_logits, n_valid, k)
    for r in range(ref.shape[0]):
        g = set(got_blocks[r][got_blocks[r] >= 0].tolist())
        o = set(ref[r][ref[r] >= 0].tolist())
        if g == o:
            continue
        v = np.sort(ref_logits[r, :n_valid[r]])[::-1]
        kth, nxt = v[k - 1], v[k]
        assert abs(kth - nxt) <= 1e-3 * abs(kth), f"row {r}: sets differ though the k-th gap is clear"
        for j in g ^ o:
            assert abs(ref_logits[r, j] - kth) <= 1e-3 * abs(kth) + 1e-12, f"row {r}: block {j} far from the k-th"


def check_attention(out, lse, ref_out, ref_lse, label=""):
    out = np.asarray(out, dtype=np.float64)
    assert not np.isnan(out).any(), f"NaN in attention output {label}"
    for r in range(ref_out.shape[0]):
        d = out[r] - ref_out[r]
        rel = np.linalg.norm(d) / max(np.linalg.norm(ref_out[r]), 1e-300)
        assert rel <= 1e-3, f"row {r}: relative L2 {rel:.3e} {label}"
        assert np.max(np.abs(d)) <= 5e-3, f"row {r}: max-abs {np.max(np.abs(d)):.3e} {label}"
    if lse is not None:
        assert np.allclose(lse, ref_lse, rtol=1e-5, atol=1e-5), f"lse differs {label}"
