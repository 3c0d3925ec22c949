"""Pins for the oracle: checks against what the pages and mathematics fix.

Every pin takes an oracle object (``oracle.Oracle``) so the same checks can be
run against deliberately broken builds of the oracle (see
``test_oracle_mutants.py``). None of these pins re-types the oracle's sort:
each one uses a different route to the answer:

- ``pin_brute_force``: enumerate every n-subset of a tiny row and keep the
  one that dominates its complement pairwise (the definition of the
  selection under the tie rule), with tie-heavy scores.
- ``pin_argmax_rounds``: a second algorithm, k rounds of "take the first
  strict maximum", on rows up to a few hundred long.
- ``pin_stable_argsort``: the special case that reduces to a library
  routine: numpy's stable argsort of the negated scores.
- ``pin_torch_topk_tie_free``: torch.topk set equality where the boundary is
  tie-free (what the reference's own test used).
- ``pin_closed_forms``: closed-form rows (trivial, all equal, monotone,
  +inf among -inf, identity page tables, absolute RAGGED columns).
- ``pin_hand_cases``: the hand-derived fixtures in ``golden/``.
- ``pin_invariants``: per-row invariants on a workload.
"""
from __future__ import annotations

import itertools

import numpy as np

from tests._helpers import load_hand_cases, valid_counts

TIE_ALPHABET = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.0, np.inf], dtype=np.float32)


def _positions_from_sel(sel_row):
    return [int(v) for v in sel_row if v >= 0]


def dominant_subsets(w, n):
    """Every n-subset X of range(len(w)) in which each x in X beats each y
    outside X: w[x] > w[y], or w[x] == w[y] and x < y."""
    L = len(w)
    idx = np.arange(L)
    found = []
    for X in itertools.combinations(range(L), n):
        inside = np.zeros(L, dtype=bool)
        inside[list(X)] = True
        wx, wy = w[inside][:, None], w[~inside][None, :]
        ix, iy = idx[inside][:, None], idx[~inside][None, :]
        beats = (wx > wy) | ((wx == wy) & (ix < iy))
        if beats.all():
            found.append(list(X))
    return found


def argmax_rounds(w, k):
    """k rounds: take the first position holding a strict maximum, remove it."""
    alive = list(range(len(w)))
    chosen = []
    for _ in range(min(k, len(w))):
        best = alive[0]
        for j in alive[1:]:
            if w[j] > w[best]:
                best = j
        chosen.append(best)
        alive.remove(best)
    return sorted(chosen)


def _tiny_batch(rng, rows, stride, max_len, outside):
    """Tiny rows with tie-heavy window scores and a shifted window."""
    scores = np.full((rows, stride), outside, dtype=np.float32)
    seq_lens = rng.integers(0, max_len + 1, size=rows).astype(np.int32)
    starts = np.zeros(rows, dtype=np.int32)
    for b in range(rows):
        L = int(seq_lens[b])
        starts[b] = rng.integers(0, stride - L + 1)
        scores[b, starts[b]:starts[b] + L] = rng.choice(TIE_ALPHABET, size=L)
    return scores, seq_lens, starts


def pin_brute_force(orc, rows=1200, seed=7):
    rng = np.random.default_rng(seed)
    scores, seq_lens, starts = _tiny_batch(rng, rows, 12, 9, np.inf)
    for k in (1, 2, 3, 5, 8):
        sel = orc.select(scores, seq_lens, starts, k, threads=2)
        for b in range(rows):
            L, s = int(seq_lens[b]), int(starts[b])
            w = scores[b, s:s + L]
            n = min(k, L)
            subsets = dominant_subsets(w, n)
            assert len(subsets) == 1, (b, k, w, subsets)
            assert _positions_from_sel(sel[b]) == subsets[0], (b, k, w, sel[b])
            assert (sel[b, n:] == -1).all()


def pin_argmax_rounds(orc, seed=11):
    rng = np.random.default_rng(seed)
    rows, stride = 40, 224
    scores = rng.choice(TIE_ALPHABET, size=(rows, stride)).astype(np.float32)
    scores[rows // 2:] = rng.standard_normal((rows - rows // 2, stride)).astype(np.float16)
    seq_lens = rng.integers(0, 201, size=rows).astype(np.int32)
    starts = rng.integers(0, 20, size=rows).astype(np.int32)
    for k in (1, 7, 64):
        sel = orc.select(scores, seq_lens, starts, k, threads=2)
        for b in range(rows):
            L, s = int(seq_lens[b]), int(starts[b])
            want = argmax_rounds(list(scores[b, s:s + L]), k)
            assert _positions_from_sel(sel[b]) == want, (b, k)


def pin_stable_argsort(orc, scores, seq_lens, k, row_starts=None):
    """Rows with L > k: the selection equals the first k of a stable argsort of
    the negated window (a stable sort keeps the lower index among equals, and
    -(+0.0) == -(-0.0))."""
    sel = orc.select(scores, seq_lens, row_starts, k)
    for b in range(scores.shape[0]):
        L = int(seq_lens[b])
        s = 0 if row_starts is None else int(row_starts[b])
        if L <= k:
            continue
        w = scores[b, s:s + L]
        want = np.sort(np.argsort(-w, kind="stable")[:k])
        assert np.array_equal(sel[b], want), b


def pin_torch_topk_tie_free(orc, scores, seq_lens, k):
    import torch

    sel = orc.select(scores, seq_lens, None, k)
    checked = 0
    for b in range(scores.shape[0]):
        L = int(seq_lens[b])
        if L <= k:
            continue
        w = torch.from_numpy(scores[b, :L].copy())
        vals, idx = torch.topk(w, k + 1)
        if vals[k - 1] == vals[k]:
            continue  # tie at the boundary: the set is not unique for topk
        assert set(idx[:k].tolist()) == set(sel[b].tolist()), b
        checked += 1
    assert checked > 0


def pin_closed_forms(orc):
    k = 5
    L = 11
    stride = 16
    rows = []
    rows.append(np.full(L, 0.25, np.float32))  # all equal -> 0..k-1
    rows.append(np.arange(L, 0, -1).astype(np.float32))  # decreasing -> 0..k-1
    rows.append(np.arange(L).astype(np.float32))  # increasing -> L-k..L-1
    spike = np.full(L, -np.inf, np.float32)
    spike[7] = np.inf
    rows.append(spike)  # +inf at 7, then 0..3
    scores = np.full((len(rows), stride), 1e3, np.float32)
    starts = np.array([0, 1, 2, 3], np.int32)
    for b, r in enumerate(rows):
        scores[b, starts[b]:starts[b] + L] = r
    lens = np.full(len(rows), L, np.int32)
    sel = orc.select(scores, lens, starts, k)
    assert sel[0].tolist() == [0, 1, 2, 3, 4]
    assert sel[1].tolist() == [0, 1, 2, 3, 4]
    assert sel[2].tolist() == [6, 7, 8, 9, 10]
    assert sel[3].tolist() == [0, 1, 2, 3, 7]

    # L <= k -> positions 0..L-1 whatever the scores hold (NaN included)
    nan_rows = np.full((3, 8), np.nan, np.float32)
    tl = np.array([0, 3, 5], np.int32)
    sel = orc.select(nan_rows, tl, None, 5)
    assert sel.tolist() == [[-1] * 5, [0, 1, 2, -1, -1], [0, 1, 2, 3, 4]]

    # RAGGED with out_offset = row_start gives absolute columns of the row
    rng = np.random.default_rng(3)
    sc = rng.standard_normal((6, 64)).astype(np.float32)
    st = rng.integers(0, 20, 6).astype(np.int32)
    ln = rng.integers(10, 44, 6).astype(np.int32)
    out = orc.ragged(sc, ln, st, st, 8)
    for b in range(6):
        cols = out[b]
        assert ((cols >= st[b]) & (cols < st[b] + ln[b])).all()
        inside = sc[b, st[b]:st[b] + ln[b]]
        assert np.array_equal(np.sort(sc[b, cols])[::-1], np.sort(inside)[::-1][:8])

    # PAGED through an identity table equals the raw positions, any page size
    for p in (1, 2, 64):
        width = 64 // p
        ident = np.tile(np.arange(width, dtype=np.int32), (6, 1))
        raw = orc.select(sc, ln, st, 8)
        assert np.array_equal(orc.paged(sc, ln, st, ident, p, 8), raw)


def pin_hand_cases(orc):
    for c in load_hand_cases():
        sc = c["scores"][None, :]
        lens = np.array([c["seq_len"]], np.int32)
        starts = np.array([c["row_start"]], np.int32)
        k = c["k"]
        if c["mode"] == "ragged":
            out = orc.ragged(sc, lens, starts, np.array([c["out_offset"]], np.int32), k)
        else:
            pt = np.array([c["page_table"]], np.int32)
            out = orc.paged(sc, lens, starts, pt, c["page_size"], k)
        want = c["expected"] + [-1] * (k - len(c["expected"]))
        assert out[0].tolist() == want, (c["name"], out[0].tolist(), want)


def check_row_invariants(scores, seq_lens, row_starts, k, sel, outside=None):
    """Invariants of one selection result (raw positions, oracle layout)."""
    n = valid_counts(seq_lens, k)
    for b in range(scores.shape[0]):
        L = max(int(seq_lens[b]), 0)
        s = 0 if row_starts is None else int(row_starts[b])
        row = sel[b]
        J = row[:n[b]]
        assert (row[n[b]:] == -1).all(), b
        assert ((J >= 0) & (J < L)).all(), b
        assert len(np.unique(J)) == n[b], b
        if L <= k:
            assert np.array_equal(J, np.arange(L)), b
            continue
        w = scores[b, s:s + L]
        mask = np.zeros(L, dtype=bool)
        mask[J] = True
        lo, hi = w[mask].min(), w[~mask].max()
        assert lo >= hi, b
        if lo == hi:  # ties at the boundary: selected ones sit lower
            assert J[w[J] == lo].max() < np.nonzero((~mask) & (w == lo))[0].min(), b
        if outside is not None:
            assert not (scores[b, s + J] == outside).any(), b


def check_emit(problem, sel, out):
    """RAGGED / PAGED emit recomputed in numpy from raw positions."""
    n = valid_counts(problem.seq_lens, problem.k)
    for b in range(problem.num_rows):
        J = sel[b, :n[b]].astype(np.int64)
        if problem.mode == "ragged":
            want = J + int(problem.out_offsets[b])
        else:
            p = problem.page_size
            want = problem.page_table[b, J // p].astype(np.int64) * p + J % p
        assert np.array_equal(out[b, :n[b]], np.sort(want)), b
        assert (out[b, n[b]:] == -1).all(), b


def pin_invariants(orc, problem, sample_rows=None):
    p = problem
    if sample_rows is not None:
        rows = np.asarray(sample_rows)
        scores = p.scores[rows]
        lens = p.seq_lens[rows]
        starts = None if p.row_starts is None else p.row_starts[rows]
    else:
        scores, lens, starts = p.scores, p.seq_lens, p.row_starts
    sel = orc.select(scores, lens, starts, p.k)
    outside = 1e3 if p.name == "ragged_extend" else None
    check_row_invariants(scores, lens, starts, p.k, sel, outside=outside)
    return sel


def pin_packed_emit(orc, seed=23):
    """Packed PAGED emit (a table-row map and per-row table starts).

    - A hand case: table rows [[7, 3], [5, 9]], page size 2; row 0 uses table
      row 0 from table position 1 and selects window positions {0, 2}:
      positions 1 and 3 map to 7*2+1 = 15 and 3*2+1 = 7; row 1 uses table
      row 1 from position 0 and selects {1}: 5*2+1 = 11.
    - The identity map with zero starts reduces to the PAGED emit.
    - Random maps and starts against a brute force that expands each table
      row into one entry per table position (no shifts or masks).
    - The pages' shifted packed layout: query rows of a request share its
      table (row_to_batch by query counts) and start at its first table
      position (score window start minus the request's KV start).
    """
    sel = np.array([[0, 2, -1], [1, -1, -1]], np.int32)
    pt = np.array([[7, 3], [5, 9]], np.int32)
    got = orc.emit_paged_packed(sel, pt, 2, table_rows=np.array([0, 1], np.int32),
                                table_starts=np.array([1, 0], np.int32))
    assert np.array_equal(got, np.array([[7, 15, -1], [11, -1, -1]], np.int32)), got

    rng = np.random.default_rng(seed)
    for page_size in (1, 2, 64):
        R, k, T, W = 40, 16, 7, 12
        sel = np.full((R, k), -1, np.int32)
        span = W * page_size
        for b in range(R):
            n = int(rng.integers(0, min(k, span // 2) + 1))
            sel[b, :n] = np.sort(rng.choice(span // 2, size=n, replace=False))
        table = rng.integers(0, 1 << 20, size=(T, W)).astype(np.int32)
        ident = orc.emit_paged_packed(sel, table[:1].repeat(R, 0), page_size)
        assert np.array_equal(ident, orc.emit_paged(sel, table[:1].repeat(R, 0), page_size))
        rows = rng.integers(0, T, size=R).astype(np.int32)
        starts = rng.integers(0, span // 2, size=R).astype(np.int32)
        got = orc.emit_paged_packed(sel, table, page_size, table_rows=rows, table_starts=starts)
        for b in range(R):
            expanded = np.repeat(table[rows[b]].astype(np.int64) * page_size, page_size) + \
                np.tile(np.arange(page_size), W)
            J = sel[b][sel[b] >= 0]
            want = np.sort(expanded[starts[b] + J])
            assert np.array_equal(got[b, :len(J)], want), (page_size, b)
            assert (got[b, len(J):] == -1).all()

    # the pages' shifted packed layout, end to end from scores
    batch, per_row, k, p = 3, 300, 20, 4
    q_lens = np.array([2, 1, 3])
    cu = np.arange(batch + 1) * per_row
    row_to_batch = np.repeat(np.arange(batch), q_lens).astype(np.int32)
    R = len(row_to_batch)
    row_starts = cu[:-1][row_to_batch].astype(np.int32)
    table_starts = (row_starts - cu[:-1][row_to_batch]).astype(np.int32)
    seq_lens = rng.integers(k + 1, per_row + 1, size=R).astype(np.int32)
    scores = rng.standard_normal((R, batch * per_row)).astype(np.float32)
    table = rng.integers(0, 1000, size=(batch, per_row // p)).astype(np.int32)
    got = orc.paged_packed(scores, seq_lens, row_starts, table, p, k,
                           table_rows=row_to_batch, table_starts=table_starts)
    for b in range(R):
        w = scores[b, row_starts[b]:row_starts[b] + seq_lens[b]]
        J = np.argsort(-w, kind="stable")[:k]
        want = np.sort(table[row_to_batch[b], J // p].astype(np.int64) * p + J % p)
        assert np.array_equal(got[b], want), b
