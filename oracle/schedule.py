"""Adaptive prefill chunk size.

Test infrastructure (see the package docstring).

[CPM, section 2.1]: chunk(L) = clamp(round_down_to_page(BUDGET / L), CHUNK_MIN,
CHUNK_MAX) with BUDGET = 2.0e8 token^2, CHUNK_MAX = 2048, CHUNK_MIN = 256 and a
page of 256, where L is the prefix (history) before the chunk. The budget comes
from the measured rule T x L <~ 2.0e8 of section 1.

Readings: the formula is followed, not the section's band table (which moves
in powers of two); chunk(0) = CHUNK_MAX (L = 0 leaves the formula undefined,
and a new request's first chunk is sized statically in that section); the last
chunk is cut to what is left of the prompt.
"""
from __future__ import annotations

BUDGET = 2.0e8
CHUNK_MIN = 256
CHUNK_MAX = 2048
PAGE = 256


def chunk_size(history: int, budget: float = BUDGET, cmin: int = CHUNK_MIN,
               cmax: int = CHUNK_MAX, page: int = PAGE) -> int:
    if history <= 0:
        return cmax
    raw = int(budget // history)          # floor(BUDGET / L)
    down = (raw // page) * page           # round down to the page
    return min(cmax, max(cmin, down))


def chunk_schedule(n_tokens: int, **kw) -> list[tuple[int, int]]:
    """[(history, chunk)] covering [0, n_tokens)."""
    out = []
    L = 0
    while L < n_tokens:
        c = min(chunk_size(L, **kw), n_tokens - L)
        out.append((L, c))
        L += c
    return out
