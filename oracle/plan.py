"""Bytes per token and the pool plan (page budget).

Test infrastructure (see the package docstring).

* Bytes per token: each of the 12 caches keeps a 512-bf16 latent row (1,024 B)
  and one pooled index key per 4 tokens; the pages count 13,056 B a token and
  rank, 12 x (1,024 + 64), 12,288 of it latent [#1142, "What happens now";
  #1313, "Step 2"]. The 64 B share is the pooled key's: a 256 B key (128 bf16)
  every 4 tokens. FP8 rows are 512 B plus a 4 B scale, 516 B a row and cache
  [#1313, "Proposal", step 1 item 3].
* Owner split: per rank a token costs the replicated pooled keys plus 1/W of
  the latent, 768 + 12,288 / W [#1313, "Step 2", "Owner"].
* Plan order: one window's pages first, a page for each other stream, then the
  prompt cache (up to its cap), then the rest as pages [#1313, "Why"]. The
  proposed step 1 sets aside as many windows as the room holds,
  n = min(lanes, 1 + (room - window) / (window + fixed)), before the cache
  [#1313, "Proposal", step 1 item 1].

Readings:

* Window pages = ceil((window + lookahead) / 512), with the MTP head's one-row
  lookahead [#1732, "What this changes": lookahead of 1]; 2,049 pages for a
  1,048,576-token window follows.
* Under the proposed order the streams hold max(n windows, one window + a page
  per other stream): n = 1 must leave the plan "unchanged from on today" and
  n = 2 at three ranks gives "4,098 pages for the streams" [#1313, "Proposal"].
* The pages' own byte counts leave out the 64-bf16 rope part; call this with
  ``rope_dim=0`` to reproduce them.
"""
from __future__ import annotations

from dataclasses import dataclass

from .layout import Geom, block_layout, page_bytes

ONE_WINDOW_FIRST = 0
WINDOWS_FIRST = 1


def bytes_per_token(g: Geom) -> int:
    """Pool bytes a token takes over all caches (latent, scale, rope, its pooled-key share)."""
    L = block_layout(g)
    per_cache = L.lat_row + (4 if g.fp8 else 0) + L.rope_row + L.pkey_row // g.pool_ratio
    return g.n_caches * per_cache


def bytes_per_token_rank(g: Geom, world: int) -> int:
    """Per-rank bytes a token takes when the latent rows sit on one owner rank and
    the pooled keys are replicated. [#1313, "Step 2", "Owner"]"""
    L = block_layout(g)
    replicated = g.n_caches * (L.pkey_row // g.pool_ratio)
    owned = g.n_caches * (L.lat_row + (4 if g.fp8 else 0) + L.rope_row)
    assert owned % world == 0
    return replicated + owned // world


@dataclass(frozen=True)
class Plan:
    page_bytes: int
    window_pages: int
    n_windows: int
    stream_pages: int
    total_pages: int
    cache_bytes: int
    fixed_bytes: int


class PlanNoMem(Exception):
    pass


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def kv_pool_plan(g: Geom, room: int, window_tokens: int, lookahead: int, fixed_per_stream: int,
                 cache_cap: int, lanes: int, policy: int = ONE_WINDOW_FIRST) -> Plan:
    P = page_bytes(g)
    wp = _cdiv(window_tokens + lookahead, g.page_rows)
    base_pages = wp + (lanes - 1)
    if policy == WINDOWS_FIRST:
        n = 1
        if room >= wp * P:
            n = min(lanes, 1 + (room - wp * P) // (wp * P + fixed_per_stream))
        n = max(n, 1)
        stream_pages = max(n * wp, base_pages)
    else:
        n = 1
        stream_pages = base_pages
    fixed = lanes * fixed_per_stream
    need = stream_pages * P + fixed
    if room < need:
        raise PlanNoMem(f"needs {need} bytes, room is {room}")
    cache = min(cache_cap, room - need)
    rest = (room - need - cache) // P
    return Plan(P, wp, n, stream_pages, stream_pages + rest, cache, fixed)
