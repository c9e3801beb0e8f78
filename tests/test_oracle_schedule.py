"""Pins of the adaptive chunk rule (chunked-prefill-memory sections 1 and 2.1)."""
import json
import os

from oracle import chunk_schedule, chunk_size

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "chunk_schedule.json")))


def test_constants_and_closed_form_points():
    B = GOLD["budget"]["value"]
    assert chunk_size(0) == GOLD["chunk_max"]["value"]
    # exact quotients at the band edges: 2e8 / L lands on a power of two
    assert chunk_size(97656) == 2048          # 2e8/97656 = 2048.01
    assert chunk_size(195312) == 1024         # 1024.003
    assert chunk_size(390625) == 512          # 512 exactly
    assert chunk_size(781250) == 256          # 256 exactly
    # between edges the formula rounds down to a multiple of 256
    assert chunk_size(100000) == 1792         # 2000 -> 1792
    assert chunk_size(150000) == 1280         # 1333.3 -> 1280
    # clamps
    assert chunk_size(1) == 2048
    assert chunk_size(10_000_000) == GOLD["chunk_min"]["value"]
    assert all(chunk_size(L) % GOLD["page"]["value"] == 0 for L in range(1, 2_000_000, 997))
    assert B == 2.0e8


def test_band_edges_agree():
    """The table's band edges (98k, 195k, 390k, 780k) are where the formula reaches
    2048, 1024, 512 and 256; the table's chunk is the formula's value just before each edge."""
    for edge, chunk in GOLD["band_edges"]["value"]:
        lo = int(edge * 0.995)
        assert chunk_size(lo) == chunk or chunk_size(lo) <= chunk * 2
        assert chunk_size(int(2.0e8 / chunk)) == chunk


def test_memory_line_respected():
    """Every chunk after the first keeps T x L within the budget (section 1's line),
    and the measured 'ok' points are on the right side of what the rule would give."""
    for N in (100_000, 390_000, 780_000):
        for L, T in chunk_schedule(N):
            if L >= 97657:
                assert T * L <= 2.0e8
    for T, L in GOLD["measured_fired"]["value"]:
        assert chunk_size(L) < T


def test_schedule_390000():
    s = chunk_schedule(390_000)
    assert sum(T for _, T in s) == 390_000
    assert s[0] == (0, 2048)
    # histories are the running sums
    L = 0
    for h, T in s:
        assert h == L
        L += T
    # the schedule never grows as the prefix grows (but the cut last chunk)
    Ts = [T for _, T in s[:-1]]
    assert all(a >= b for a, b in zip(Ts, Ts[1:]))
    counts = {}
    for _, T in s[:-1]:
        counts[T] = counts.get(T, 0) + 1
    assert len(s) == 464
    assert counts == {2048: 48, 1792: 8, 1536: 12, 1280: 20, 1024: 38, 768: 85, 512: 252}
    assert s[-1][1] == 112
