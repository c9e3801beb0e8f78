"""Pins of the oracle's byte counts and pool plan against the figures the pages print
(tests/golden/plan_figures.json names each figure's page and section)."""
import json
import os

import pytest

from oracle import Geom, block_layout, bytes_per_token, bytes_per_token_rank, kv_pool_plan, page_bytes
from oracle.plan import ONE_WINDOW_FIRST, WINDOWS_FIRST, PlanNoMem

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "plan_figures.json")))
MiB = 1 << 20
GiB = 1 << 30

# The pages' engine counts no rope plane (12 caches of 1,024 B latent + 64 B key share).
PAGES_GEOM = Geom(n_caches=12, rope_dim=0, index_dim=128)


def test_bytes_per_token_pages_accounting():
    assert bytes_per_token(PAGES_GEOM) == GOLD["bytes_per_token_bf16_12_caches"]["value"]
    L = block_layout(PAGES_GEOM)
    assert 12 * L.lat_row == GOLD["latent_bytes_per_token_12_caches"]["value"]
    # one page spans the 12 caches: 512 rows x 13,056 B = 6.375 MiB
    assert page_bytes(PAGES_GEOM) == 512 * 13056 == int(6.375 * MiB)


def test_fp8_row_bytes():
    g = Geom(n_caches=1, rope_dim=0, fp8=True)
    L = block_layout(g)
    assert L.lat_row + 4 == GOLD["fp8_row_bytes"]["value"]
    # the scales sit after the page's rows
    assert L.off_scale == 512 * L.lat_row and L.off_latent == 0


def test_owner_split_bytes_per_rank():
    for w, v in GOLD["owner_split_bytes_per_rank"]["value"].items():
        assert bytes_per_token_rank(PAGES_GEOM, int(w)) == v


def test_rope_and_fp8_totals():
    # With the 64-bf16 rope plane of each row, and with fp8 rows.
    assert bytes_per_token(Geom(n_caches=12)) == 12 * (1024 + 128 + 64) == 14592
    assert bytes_per_token(Geom(n_caches=12, rope_dim=0, fp8=True)) == 12 * (516 + 64) == 6960
    assert bytes_per_token(Geom(n_caches=12, fp8=True)) == 12 * (516 + 128 + 64) == 8496


def _tp2_room():
    return int(GOLD["room_tp2_gib"]["value"] * GiB)


# Fixed bytes per stream: the pages print "180 MiB fixed"; 12.93 GiB per 1M window and
# 90.48 GiB for seven windows both come out within their printed digits for 176-180 MiB.
FIXED_TP2 = 176 * MiB


def test_window_pages_1M():
    p = kv_pool_plan(PAGES_GEOM, _tp2_room(), 1048576, 1, FIXED_TP2, 16 * GiB, 8)
    assert p.window_pages == GOLD["window_pages_1M"]["value"]


def test_pool_pages_1M_parallel8_tp2():
    p = kv_pool_plan(PAGES_GEOM, _tp2_room(), 1048576, 1, FIXED_TP2, 16 * GiB, 8, ONE_WINDOW_FIRST)
    g = GOLD["pool_pages_1M_parallel8_tp2"]
    assert p.total_pages == g["value"]
    assert p.total_pages * 512 == g["tokens"]
    c = GOLD["cache_gib_tp2_1M"]
    assert abs(p.cache_bytes / GiB - c["value"]) <= c["tol"]
    # the proposed order leaves this case as it is (n = 1)
    q = kv_pool_plan(PAGES_GEOM, _tp2_room(), 1048576, 1, FIXED_TP2, 16 * GiB, 8, WINDOWS_FIRST)
    assert q.n_windows == 1 and q.total_pages == p.total_pages


def test_window_gib_and_seven_streams():
    P = page_bytes(PAGES_GEOM)
    per_stream = (2049 * P + FIXED_TP2) / GiB
    g = GOLD["window_gib_per_stream_1M"]
    assert abs(per_stream - g["value"]) <= g["tol"]
    g = GOLD["seven_streams_gib_1M"]
    assert abs(7 * per_stream - g["value"]) <= g["tol"]
    assert abs(FIXED_TP2 / MiB - GOLD["fixed_mib_tp2"]["value"]) <= 5


def test_256k_parallel8():
    p = kv_pool_plan(PAGES_GEOM, _tp2_room(), 262144, 1, FIXED_TP2, 16 * GiB, 8, ONE_WINDOW_FIRST)
    g = GOLD["pages_256k_parallel8"]
    assert p.total_pages == g["value"] and p.total_pages * 512 == g["tokens"]
    q = kv_pool_plan(PAGES_GEOM, _tp2_room(), 262144, 1, FIXED_TP2, 16 * GiB, 8, WINDOWS_FIRST)
    assert q.n_windows == GOLD["windows_256k_streams"]["value"]
    # never fewer rows than windows would hold
    assert q.total_pages * 512 >= q.n_windows * 262144


def test_tp3_three_figures_consistent():
    """The three TP=3 figures (3,355 pages and a 16 GiB cache today; 4,098 pages and
    11.4 GiB proposed; windows: 2 streams and 12.0 GiB) come from one room. Solve the
    room from today's figures, then the proposed plan must give the other two."""
    P = page_bytes(PAGES_GEOM)
    fixed = 107 * MiB      # the one per-stream value that also gives the windows' 12.0 GiB
    room = GOLD["tp3_today_pages"]["value"] * P + 8 * fixed + 16 * GiB
    today = kv_pool_plan(PAGES_GEOM, room, 1048576, 1, fixed, 16 * GiB, 8, ONE_WINDOW_FIRST)
    assert today.total_pages == GOLD["tp3_today_pages"]["value"]
    assert today.cache_bytes == 16 * GiB
    new = kv_pool_plan(PAGES_GEOM, room, 1048576, 1, fixed, 16 * GiB, 8, WINDOWS_FIRST)
    assert new.n_windows == GOLD["tp3_windows_streams"]["value"]
    assert new.total_pages == GOLD["tp3_new_pages"]["value"]
    g = GOLD["tp3_new_cache_gib"]
    assert abs(new.cache_bytes / GiB - g["value"]) <= g["tol"]
    # windows (no pages): n windows of 2,049 pages each plus their fixed parts
    win_cache = room - new.n_windows * (2049 * P + fixed)
    g = GOLD["tp3_windows_cache_gib"]
    assert abs(win_cache / GiB - g["value"]) <= g["tol"]


def test_kept_state_bytes_follow_at():
    """A kept state is a fixed part plus at rows: 1.38 GB at 100k tokens, 13.8 GB for
    the whole 1M window, with the same fixed part."""
    g = GOLD["kept_state_100k_tp3_gb"]
    bpt = bytes_per_token(PAGES_GEOM)
    fixed = g["value"] * 1e9 - 100000 * bpt
    assert 0 < fixed < 0.1e9
    full = 2049 * 512 * bpt + fixed
    assert abs(full / 1e9 - g["full_window_gb"]) <= 0.05


def test_no_room_refused():
    with pytest.raises(PlanNoMem):
        kv_pool_plan(PAGES_GEOM, 10 * GiB, 1048576, 1, FIXED_TP2, 16 * GiB, 8)
