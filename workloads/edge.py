"""Edge-case batches: band boundaries, start residues and tie-heavy rows.

Input generation only. Each row gets a window length, a start residue
(row_start % 4) and a value pattern; columns outside a row's window hold the
1e3 sentinel, so any read outside the window would be selected.
"""
from __future__ import annotations

import numpy as np

from .configs import OUTSIDE_SCORE, PAGE_SIZE, Problem, random_page_tables

PATTERNS = ("normal", "fp16", "alphabet", "equal", "neg_inf", "increasing", "decreasing",
            "zeros_mixed", "one_pos_inf", "rising_head", "dense")

_ALPHABET = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.0, np.inf], dtype=np.float32)


def _tie_class(rng, L: int, above: int, tied: int) -> np.ndarray:
    """``above`` elements at 10, ``tied`` at 5 (distinct random positions),
    the rest uniform in (-1, 1): for above < k < above + tied the k-th key is
    shared by ``tied`` elements, of which k - above are taken."""
    v = rng.uniform(-1.0, 1.0, size=L).astype(np.float32)
    idx = rng.permutation(L)[:above + tied]
    v[idx[:above]] = 10.0
    v[idx[above:]] = 5.0
    return v


def _values(rng, pattern, L: int) -> np.ndarray:
    """``pattern`` is a name from PATTERNS or ("ties", above, tied)."""
    if isinstance(pattern, tuple):
        kind, above, tied = pattern
        assert kind == "ties" and above + tied <= L
        return _tie_class(rng, L, above, tied)
    if pattern == "normal":
        return rng.standard_normal(L, dtype=np.float32)
    if pattern == "fp16":
        return rng.standard_normal(L, dtype=np.float32).astype(np.float16).astype(np.float32)
    if pattern == "alphabet":
        return rng.choice(_ALPHABET, size=L)
    if pattern == "equal":
        return np.full(L, 0.75, dtype=np.float32)
    if pattern == "neg_inf":
        return np.full(L, -np.inf, dtype=np.float32)
    if pattern == "increasing":
        return np.linspace(-3.0, 3.0, L, dtype=np.float32) + np.float32(0)
    if pattern == "decreasing":
        return np.linspace(3.0, -3.0, L, dtype=np.float32)
    if pattern == "zeros_mixed":
        v = rng.choice(np.array([-0.0, 0.0], dtype=np.float32), size=L)
        v[rng.integers(0, L, size=max(1, L // 100))] = 1.0
        return v
    if pattern == "rising_head":
        # rising over the first 16384 positions, low noise after them: a
        # long row's largest keys all sit in its first 16384 columns, and
        # the largest of those at their end
        h = min(L, 16384)
        v = np.float32(-2.0) + np.float32(0.1) * rng.standard_normal(L, dtype=np.float32)
        v[:h] = np.linspace(-3.0, 3.0, h, dtype=np.float32)
        return v
    if pattern == "dense":
        # every value in [0.75, 0.8125): one bin of the top 12 key bits,
        # spread over its four 14-bit sub-bins, so the k-th key's fine bin
        # holds hundreds of elements with others above it in the same
        # coarse bin
        return rng.uniform(0.75, 0.8125, size=L).astype(np.float32)
    if pattern == "one_pos_inf":
        v = np.full(L, -np.inf, dtype=np.float32)
        v[rng.integers(0, L)] = np.inf
        return v
    raise ValueError(pattern)


def edge_batch(seed: int, mode: str, k: int, rows, page_size: int = PAGE_SIZE,
               name: str = "edge", stride: int = None) -> Problem:
    """``rows`` is a list of (seq_len, residue, pattern); negative seq_len allowed.

    row_start = 4 * (b % 3) + residue, so starts differ between rows; the
    score stride fits the longest window plus its start and is a multiple of 4.
    With ``stride`` given, the score stride is exactly that (a multiple of 4)
    and a row whose shifted window would not fit starts at its residue
    instead; every window must then fit (residue + seq_len <= stride).
    """
    rng = np.random.default_rng(seed)
    R = len(rows)
    lens = np.array([r[0] for r in rows], dtype=np.int32)
    starts = np.array([4 * (b % 3) + r[1] for b, r in enumerate(rows)], dtype=np.int32)
    if stride is not None:
        assert stride % 4 == 0 and stride >= 4
        res = np.array([r[1] for r in rows], dtype=np.int32)
        spill = starts.astype(np.int64) + np.maximum(lens, 0) > stride
        starts[spill] = res[spill]
        assert (starts.astype(np.int64) + np.maximum(lens, 0) <= stride).all(), \
            "a window does not fit the stride"
    else:
        need = int((starts.astype(np.int64) + np.maximum(lens, 0)).max()) if R else 4
        stride = max(4, (need + 3) // 4 * 4)
    scores = np.full((R, stride), OUTSIDE_SCORE, dtype=np.float32)
    for b, (L, _, pattern) in enumerate(rows):
        if L > 0:
            scores[b, starts[b]:starts[b] + L] = _values(rng, pattern, L)
    if mode == "ragged":
        offs = rng.integers(0, 1 << 20, size=R).astype(np.int32)
        return Problem(name, "ragged", k, scores, lens, row_starts=starts, out_offsets=offs)
    width = max(1, -(-max(int(np.maximum(lens, 0).max()) if R else 1, 1) // page_size))
    pt = random_page_tables(rng, R, width, max(width, 1 << 12))
    return Problem(name, "paged", k, scores, lens, row_starts=starts, page_table=pt,
                   page_size=page_size)
