"""Decode of FP8 e4m3 latent codes.

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
