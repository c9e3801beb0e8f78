"""Decode of FP8 e4m3 latent codes, and the quantizing write's recipe.

Test infrastructure (see the package docstring).

[#1313, "Proposal", step 1 item 3]: FP8 rows are 512 one-byte values with one
fp32 scale per row. Reading: the OCP E4M3 "fn" encoding (1 sign, 4 exponent
bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal; S.1111.111 is
NaN; no infinities), and a row's value is code value x row scale.
"""
from __future__ import annotations

import numpy as np


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact value of each e4m3fn code as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, v)


# ---- quantizing write ---------------------------------------------------------------
# [#1313, "Proposal", step 1 item 3] proposes writing fp8 rows on the device but
# fixes no quantization recipe. The reading taken here, per row of 512 values:
#   scale = amax / 448 in fp32 (amax = max |x|; 448 is e4m3fn's largest finite value),
#   code  = the e4m3fn value nearest to clamp(x / scale, -448, 448) (fp32 quotient),
#           ties to the even code, sign from the quotient;
#   an all-zero row gets scale 0 and +0 codes.
# The decisions are taken in fp32, as the library takes them: numpy float32
# arithmetic is IEEE, so the quotients here are the ones the device computes.

_MAGS = None


def _e4m3_magnitudes() -> np.ndarray:
    """The 127 finite non-negative e4m3fn values, codes 0 .. 126, increasing."""
    global _MAGS
    if _MAGS is None:
        _MAGS = e4m3_decode(np.arange(127, dtype=np.uint8))
        assert np.all(np.diff(_MAGS) > 0)
    return _MAGS


def e4m3_encode_nearest(q: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn code of each finite q with |q| <= 448: the nearest value by brute
    force over the finite magnitudes, ties to the even code, sign bit from q's sign."""
    q = np.asarray(q, dtype=np.float64)
    assert np.all(np.isfinite(q)) and np.all(np.abs(q) <= 448.0)
    mags = _e4m3_magnitudes()
    a = np.abs(q)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)   # first magnitude >= a
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(q), 0x80, 0).astype(np.uint8)


def quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Codes (uint8 [n][512]) and scales (float32 [n]) of bf16 rows given as float32."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    q = np.zeros_like(x)
    nz = scale > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        q[nz] = x[nz] / scale[nz, None]
    q = np.clip(q, np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    return e4m3_encode_nearest(q), scale
