"""The seeded input generator: determinism, distribution, and the fp8 encoding
against torch's float8_e4m3fn conversion (a library routine)."""
import math

import numpy as np
import torch

import synth
from synth.configs import adaptive_prefill, decode_batch, prefill_chunk, shared_prefix_decode, tiny


def test_splitmix_reference_values():
    # SplitMix64 with state 0 advanced once by gamma: first output 0xE220A8397B1DCDAF
    assert synth._mix_int(synth.GAMMA) == 0xE220A8397B1DCDAF
    assert int(synth.hash64(0, np.array([0]))[0]) == 0xE220A8397B1DCDAF


def test_deterministic_and_index_addressed():
    idx = np.arange(1000, dtype=np.uint64)
    a = synth.bf16_values(0, synth.TAG_LATENT, idx, 576)
    b = synth.bf16_values(0, synth.TAG_LATENT, idx[::-1], 576)[::-1]
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.bf16_values(1, synth.TAG_LATENT, idx, 576))


def test_distribution():
    v = synth.bf16_to_f64(synth.bf16_values(0, synth.TAG_Q, np.arange(400000), 128))
    assert abs(v.mean()) < 2e-3 / math.sqrt(128) * 10
    assert abs(v.std() * math.sqrt(128) - 1.0) < 5e-3


def test_e4m3_encoding_matches_torch():
    s = np.arange(-131070, 131071, 7, dtype=np.int64)
    ref = (torch.from_numpy(s).double() * 2.0 ** -11).float().to(torch.float8_e4m3fn)
    assert np.array_equal(synth.e4m3_code_from_int(s), ref.view(torch.uint8).numpy())


def test_fp8_scales_range():
    sc = synth.fp8_row_scales(0, synth.TAG_SCALE8, np.arange(10000))
    base = float(synth.fp8_row_scale_base())
    assert sc.min() >= 0.5 * base and sc.max() < 1.5 * base


def test_workloads_shapes():
    t = tiny()
    assert t.pt.shape == (2, 4) and len(set(t.pt.ravel())) == 8 and t.pt.max() < 16
    d = decode_batch()
    assert d.pt.shape == (8, 256) and len(set(d.pt.ravel())) == 2048
    p = prefill_chunk()
    assert len(p.rows) == 2048 and p.rows[0] == (0, 97952) and p.rows[-1] == (0, 99999)
    s = shared_prefix_decode()
    assert s.pt.shape == (8, 2049) and np.all(s.pt[:, :2048] == s.pt[0, :2048])
    assert len(set(s.pt[:, 2048])) == 8 and all(1 <= L - 2048 * 512 <= 511 for L in s.lengths)
    a = adaptive_prefill()
    assert a.fp8 and a.lengths[0] == 390000


def test_shared_prefix_rows_are_shared():
    s = shared_prefix_decode()
    assert np.array_equal(s.latent_bits(3, 0, [5, 1048575]), s.latent_bits(3, 7, [5, 1048575]))
    assert not np.array_equal(s.latent_bits(3, 0, [1048576]), s.latent_bits(3, 7, [1048576]))
    assert np.array_equal(s.pkey_bits(0, 1, [262143]), s.pkey_bits(0, 5, [262143]))
    assert not np.array_equal(s.pkey_bits(0, 1, [262144]), s.pkey_bits(0, 5, [262144]))
