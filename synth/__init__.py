"""Seeded synthetic inputs, shared by the oracle's tests, the GPU tests and the bench.

This module holds none of the method's arithmetic: it only draws numbers.
Every value is a pure function of (seed, tag, flat index), so any row of a
multi-gigabyte pool can be regenerated on the host without keeping a copy, and
a device fill kernel (``synth.hip``) reproduces the same bits on the GPU.

Generator, from its published definitions:

* hash: the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014) applied to
  ``key + (index + 1) * 0x9E3779B97F4A7C15`` with ``key = mix(seed * gamma + tag)``;
* approximately normal integer: the sum of the four 16-bit fields of the hash
  minus its mean (an Irwin-Hall sum of 4 uniforms), ``s`` in [-131070, 131070];
* real value: ``float32(s) * float32(1 / (sigma * sqrt(d)))`` (one IEEE
  float32 multiply, so host and device agree bit for bit), then bf16 by
  round-to-nearest-even on the float32 bits;
* fp8 e4m3 (OCP "fn" variant) codes: ``s / 2048`` rounded to nearest even at
  e4m3 precision, computed in integers; row scales
  ``float32(c) * (0.5 + u)`` with ``u`` a 23-bit uniform.
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# sqrt(Var) of the sum of four independent uniform 16-bit integers
SIGMA = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)

# tensor tags
TAG_LATENT = 1   # latent + rope row, 576 values per row
TAG_PKEY = 2     # pooled index key, D_k values per key
TAG_Q = 3        # attention query, Hq x 576 per row
TAG_IQ = 4       # indexer query, H x D_k per row
TAG_W = 5        # indexer head weight, H per row (fp32)
TAG_LAT8 = 6     # fp8 latent code, 512 per row
TAG_SCALE8 = 7   # fp8 row scale, 1 per row


def _mix_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tag: int) -> int:
    """64-bit key of one tensor: mix(seed * gamma + tag)."""
    return _mix_int(seed * GAMMA + tag)


def hash64(key: int, idx: np.ndarray) -> np.ndarray:
    """SplitMix64 output of key + (idx + 1) * gamma, elementwise, as uint64."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        z = z ^ (z >> np.uint64(31))
    return z


def normal_int(h: np.ndarray) -> np.ndarray:
    """Irwin-Hall(4) integer in [-131070, 131070] from a 64-bit hash (int64)."""
    m = np.uint64(0xFFFF)
    s = (h & m) + ((h >> np.uint64(16)) & m) + ((h >> np.uint64(32)) & m) + (h >> np.uint64(48))
    return s.astype(np.int64) - 131070


def unit_scale(d: float) -> np.float32:
    """float32 multiplier that maps the integer s to N(0,1)/sqrt(d)."""
    return np.float32(1.0 / (SIGMA * math.sqrt(d)))


def f32_from_int(s: np.ndarray, c: np.float32) -> np.ndarray:
    return s.astype(np.float32) * np.float32(c)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite and far from overflow."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_values(seed: int, tag: int, idx: np.ndarray, d: float) -> np.ndarray:
    """bf16 bits of N(0,1)/sqrt(d) at the given flat indices."""
    s = normal_int(hash64(stream_key(seed, tag), idx))
    return bf16_bits(f32_from_int(s, unit_scale(d)))


def f32_values(seed: int, tag: int, idx: np.ndarray, d: float) -> np.ndarray:
    """float32 N(0,1)/sqrt(d) at the given flat indices (no bf16 rounding)."""
    s = normal_int(hash64(stream_key(seed, tag), idx))
    return f32_from_int(s, unit_scale(d))


def e4m3_code_from_int(s: np.ndarray) -> np.ndarray:
    """OCP e4m3fn code of the exact value s * 2**-11, round to nearest even.

    |s| <= 131070 keeps every value below 64, so no saturation is needed.
    Integer-only, so the device twin reproduces it exactly."""
    s = np.asarray(s, dtype=np.int64)
    sign = (s < 0).astype(np.int64)
    a = np.abs(s)
    nb = np.zeros_like(a)                 # bit length of a
    for k in range(63):
        nb += (a >= (np.int64(1) << k)).astype(np.int64)
    e = nb - 12                           # value in [2^e, 2^(e+1))
    # normal: a rounded to 4 significant bits, m4 in [8, 16]
    sh = np.maximum(nb - 4, 0)
    m4 = np.where(nb >= 4, _rne_shift(a, sh), a << np.maximum(4 - nb, 0))
    carry = m4 >= 16
    e = np.where(carry, e + 1, e)
    m4 = np.where(carry, 8, m4)
    code_n = ((e + 7) << 3) | (m4 - 8)
    # subnormal (e < -6): units of 2^-9, q = rne(a / 4) in [0, 8]
    code_s = _rne_shift(a, np.full_like(a, 2))
    code = np.where(e < -6, code_s, code_n)
    code = np.where(a == 0, 0, code)
    return ((sign << 7) | code).astype(np.uint8)


def _rne_shift(a: np.ndarray, k: np.ndarray) -> np.ndarray:
    """round(a / 2**k) to nearest, ties to even, for a >= 0 and k >= 0."""
    k = np.asarray(k, dtype=np.int64)
    q = a >> k
    r = a - (q << k)
    half = np.where(k > 0, np.int64(1) << np.maximum(k - 1, 0), 0)
    up = (k > 0) & ((r > half) | ((r == half) & ((q & 1) == 1)))
    return q + up.astype(np.int64)


def e4m3_codes(seed: int, tag: int, idx: np.ndarray) -> np.ndarray:
    return e4m3_code_from_int(normal_int(hash64(stream_key(seed, tag), idx)))


# fp8 rows: codes carry s/2048 ~ 18.5 N(0,1); the row scale brings them back to
# about N(0,1)/sqrt(576), times a per-row factor in [0.5, 1.5).
FP8_CODE_SIGMA = SIGMA / 2048.0


def fp8_row_scale_base(d: float = 576.0) -> np.float32:
    return np.float32(1.0 / (FP8_CODE_SIGMA * math.sqrt(d)))


def fp8_row_scales(seed: int, tag: int, idx: np.ndarray, d: float = 576.0) -> np.ndarray:
    h = hash64(stream_key(seed, tag), idx)
    u = (h >> np.uint64(41)).astype(np.float32) * np.float32(2.0 ** -23)
    return (np.float32(0.5) + u) * fp8_row_scale_base(d)
