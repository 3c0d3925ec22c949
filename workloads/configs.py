"""Workload generators (input generation only; see the package docstring)."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BASE_SEED = 20260000
PAGE_SIZE = 64

# workload name -> index used to derive its seed (BASE_SEED + index)
WORKLOADS = {
    "paged_small": 0,
    "paged_decode": 1,
    "ragged_extend": 2,
    "paged_long": 3,
    "paged_mixed": 4,
}

# slot width of one request in the flattened KV of ``ragged_extend``:
# 16385 columns so that the four slot bases 0, 16385, 32770, 49155 take every
# residue modulo 4 while the longest window (16384) still fits in its slot.
RAGGED_SLOT = 16385
RAGGED_REQUESTS = 4
RAGGED_ROWS_PER_REQUEST = 1024
OUTSIDE_SCORE = 1e3

MIXED_PINNED = (1024, 1025, 8192, 8193, 16385, 65535, 65537)


@dataclass
class Problem:
    """One launch worth of inputs (host numpy arrays)."""

    name: str
    mode: str  # "paged" or "ragged"
    k: int
    scores: np.ndarray  # float32 [num_rows, stride]
    seq_lens: np.ndarray  # int32 [num_rows]
    row_starts: Optional[np.ndarray] = None  # int32 [num_rows] or None
    out_offsets: Optional[np.ndarray] = None  # int32 [num_rows] (ragged)
    page_table: Optional[np.ndarray] = None  # int32 [num_rows, width] (paged)
    page_size: int = PAGE_SIZE
    extra: dict = field(default_factory=dict)

    @property
    def num_rows(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def stride(self) -> int:
        return int(self.scores.shape[1])

    def window_lengths(self) -> np.ndarray:
        return np.maximum(self.seq_lens.astype(np.int64), 0)

    def score_bytes(self) -> int:
        """Bytes of scores the selection must read: 4*L for rows with L > k."""
        L = self.window_lengths()
        return int(4 * L[L > self.k].sum())


def random_page_tables(rng, rows: int, width: int, pages: int) -> np.ndarray:
    """Each row: the first ``width`` entries of a permutation of ``pages`` pages."""
    pt = np.empty((rows, width), dtype=np.int32)
    for r in range(rows):
        pt[r] = rng.permutation(pages)[:width].astype(np.int32)
    return pt


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def paged_small(seed: int) -> Problem:
    rng = np.random.default_rng(seed)
    R, stride = 4, 3000
    seq_lens = rng.integers(1, 3001, size=R).astype(np.int32)
    scores = _normal(rng, (R, stride))
    pt = random_page_tables(rng, R, 256, 256)
    return Problem("paged_small", "paged", 512, scores, seq_lens, page_table=pt)


def paged_decode(seed: int, rows: int = 128, pt_width: int = 4096) -> Problem:
    rng = np.random.default_rng(seed)
    L = 8192
    seq_lens = np.full(rows, L, dtype=np.int32)
    scores = _normal(rng, (rows, L))
    pt = random_page_tables(rng, rows, pt_width, 4096)
    return Problem("paged_decode", "paged", 2048, scores, seq_lens, page_table=pt)


def ragged_extend(seed: int) -> Problem:
    rng = np.random.default_rng(seed)
    reqs, per = RAGGED_REQUESTS, RAGGED_ROWS_PER_REQUEST
    R = reqs * per
    stride = reqs * RAGGED_SLOT
    cu = np.arange(reqs + 1, dtype=np.int64) * RAGGED_SLOT
    i = np.tile(np.arange(per, dtype=np.int32), reqs)
    seq_lens = (15361 + i).astype(np.int32)
    base = np.repeat(cu[:-1], per).astype(np.int32)
    assert set((base % 4).tolist()) == {0, 1, 2, 3}
    scores = np.full((R, stride), OUTSIDE_SCORE, dtype=np.float32)
    inside = _normal(rng, (R, int(seq_lens.max())))
    for b in range(R):
        s, L = int(base[b]), int(seq_lens[b])
        scores[b, s:s + L] = inside[b, :L]
    return Problem("ragged_extend", "ragged", 2048, scores, seq_lens, row_starts=base,
                   out_offsets=base.copy(), extra={"cu_seqlens": cu})


def paged_long(seed: int, rows: int = 8) -> Problem:
    rng = np.random.default_rng(seed)
    L = 131072
    seq_lens = np.full(rows, L, dtype=np.int32)
    scores = _normal(rng, (rows, L)).astype(np.float16).astype(np.float32)
    pt = random_page_tables(rng, rows, L // PAGE_SIZE, L // PAGE_SIZE)
    return Problem("paged_long", "paged", 2048, scores, seq_lens, page_table=pt)


def paged_mixed(seed: int) -> Problem:
    rng = np.random.default_rng(seed)
    R, Lmax = 512, 131072
    u = rng.random(R)
    seq_lens = np.clip(np.floor(np.exp(u * np.log(Lmax + 1))), 1, Lmax).astype(np.int32)
    scores = _normal(rng, (R, Lmax))
    pt = random_page_tables(rng, R, Lmax // PAGE_SIZE, Lmax // PAGE_SIZE)
    pinned_rows = rng.choice(R, size=len(MIXED_PINNED), replace=False)
    seq_lens[pinned_rows] = np.asarray(MIXED_PINNED, dtype=np.int32)
    return Problem("paged_mixed", "paged", 1024, scores, seq_lens, page_table=pt,
                   extra={"pinned_rows": pinned_rows})


_MAKERS = {
    "paged_small": paged_small,
    "paged_decode": paged_decode,
    "ragged_extend": ragged_extend,
    "paged_long": paged_long,
    "paged_mixed": paged_mixed,
}


def make_workload(name: str, seed: Optional[int] = None) -> Problem:
    """Build a named workload with its default seed (BASE_SEED + index)."""
    if seed is None:
        seed = BASE_SEED + WORKLOADS[name]
    return _MAKERS[name](seed)


def scaled_decode(rows: int, seed: Optional[int] = None) -> Problem:
    """``paged_decode``'s per-row shape with ``rows`` rows (sustained-rate runs)."""
    if seed is None:
        seed = BASE_SEED + 101
    # only the first 8192 / 64 = 128 table entries are addressed; keep those
    p = paged_decode(seed, rows=rows, pt_width=128)
    p.name = f"paged_decode_x{rows}"
    return p


def short_mix(rows: int, mode: str, seed: Optional[int] = None) -> Problem:
    """Many rows of the short class (span <= 8192 columns) with mixed shapes:
    window starts at column 0..3 (every residue mod 4); even rows log-uniform
    lengths in [1, 8192 - start] (mostly trivial, L <= k), odd rows uniform in
    [1001, 8192 - start]; k = 1000, N(0,1)
    scores of which every 16th row is rounded to fp16 (ties at the cut).
    PAGED: page size 64, 128 table entries per row from 4096 pages; RAGGED:
    random output offsets below 2^20."""
    if seed is None:
        seed = BASE_SEED + 105
    rng = np.random.default_rng(seed)
    stride = 8192 + 4
    starts = rng.integers(0, 4, size=rows).astype(np.int32)
    u = rng.random(rows)
    logu = np.floor(np.exp(u * np.log(8193 - starts)))
    unif = 1001 + np.floor(u * (8192 - starts - 1000))
    seq_lens = np.where(np.arange(rows) % 2 == 0, logu, unif)
    seq_lens = np.clip(seq_lens, 1, 8192 - starts).astype(np.int32)
    scores = _normal(rng, (rows, stride))
    scores[::16] = scores[::16].astype(np.float16).astype(np.float32)
    name = f"short_mix_{mode}_x{rows}"
    if mode == "paged":
        pt = random_page_tables(rng, rows, 128, 4096)
        return Problem(name, "paged", 1000, scores, seq_lens, row_starts=starts, page_table=pt)
    offs = rng.integers(0, 1 << 20, size=rows).astype(np.int32)
    return Problem(name, "ragged", 1000, scores, seq_lens, row_starts=starts, out_offsets=offs)


def scaled_long(rows: int, seed: Optional[int] = None) -> Problem:
    """``paged_long``'s per-row shape with ``rows`` rows (sustained-rate runs)."""
    if seed is None:
        seed = BASE_SEED + 103
    p = paged_long(seed, rows=rows)
    p.name = f"paged_long_x{rows}"
    return p


def scaled_paged(L: int, rows: int, fp16: bool = False, seed: Optional[int] = None) -> Problem:
    """PAGED decode rows of one window length ``L`` (sustained-rate runs
    between the decode and long-context shapes): N(0,1) fp32 scores (rounded
    to fp16 if ``fp16``), k = 2048, page size 64, each row's L / 64 table
    entries a random permutation of 4096 (or L / 64, if more) pages."""
    if seed is None:
        seed = BASE_SEED + 107
    rng = np.random.default_rng(seed)
    seq_lens = np.full(rows, L, dtype=np.int32)
    scores = _normal(rng, (rows, L))
    if fp16:
        scores = scores.astype(np.float16).astype(np.float32)
    width = -(-L // PAGE_SIZE)
    pt = random_page_tables(rng, rows, width, max(width, 4096))
    return Problem(f"paged_L{L}_x{rows}", "paged", 2048, scores, seq_lens, page_table=pt)


# Sustained-rate launches: the paged decode row shape (N(0,1) fp32, k = 2048,
# page size 64) at window lengths from 8192 to 131072, each with enough rows
# for 1 GiB of scores per launch (131072: the fp16-rounded long-context rows).
SUSTAINED_LENGTHS = (8192, 16384, 24576, 32768, 40960, 49152, 65536, 98304, 131072)


def sustained_rows(L: int) -> int:
    """Rows of a sustained launch of window length L: ceil(2^30 / (4 L))."""
    return -(-(1 << 30) // (4 * L))


def sustained_name(L: int) -> str:
    if L == 8192:
        return "paged_decode_x32768"
    if L == 131072:
        return "paged_long_x2048"
    return f"paged_L{L}_x{sustained_rows(L)}"


def sustained(L: int) -> Problem:
    """The sustained launch of window length L (see SUSTAINED_LENGTHS)."""
    if L == 8192:
        return scaled_decode(sustained_rows(L))
    if L == 131072:
        return scaled_long(sustained_rows(L))
    return scaled_paged(L, sustained_rows(L))


def all_trivial(seed: Optional[int] = None) -> Problem:
    """128 PAGED rows whose windows all fit in k (L uniform in [1, 2048],
    k = 2048): every row takes the trivial path, so a launch should read no
    scores at all (a counter check)."""
    if seed is None:
        seed = BASE_SEED + 109
    rng = np.random.default_rng(seed)
    R = 128
    seq_lens = rng.integers(1, 2049, size=R).astype(np.int32)
    scores = _normal(rng, (R, 8192))
    pt = random_page_tables(rng, R, 128, 4096)
    return Problem("all_trivial", "paged", 2048, scores, seq_lens, page_table=pt)


def packed_paged(seed: int, q_lens, kv_len: int, k: int, max_shift: int = 0,
                 page_size: int = PAGE_SIZE):
    """Packed PAGED rows (the pages' packed layout): request r owns KV
    columns [r * kv_len, (r + 1) * kv_len) of a batch-wide score axis and one
    page-table row; its q_lens[r] query rows each select inside that span.
    Row b of request r starts its window shift_b columns into the request
    (shift_b uniform in [0, max_shift]): row_start = r * kv_len + shift_b and
    table start shift_b. seq_len uniform in [k + 1, kv_len - shift_b]. N(0,1)
    scores inside each window, 1e3 outside.

    Returns (problem, table_rows, table_starts); the problem's page table has
    one row per request."""
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens)
    batch = len(q_lens)
    table_rows = np.repeat(np.arange(batch), q_lens).astype(np.int32)
    R = len(table_rows)
    shifts = rng.integers(0, max_shift + 1, size=R).astype(np.int32)
    seq_lens = rng.integers(k + 1, kv_len - shifts + 1).astype(np.int32)
    row_starts = (table_rows.astype(np.int64) * kv_len + shifts).astype(np.int32)
    stride = (batch * kv_len + 3) // 4 * 4
    scores = np.full((R, stride), OUTSIDE_SCORE, dtype=np.float32)
    for b in range(R):
        s, L = int(row_starts[b]), int(seq_lens[b])
        scores[b, s:s + L] = rng.standard_normal(L, dtype=np.float32)
    width = -(-kv_len // page_size)
    pt = random_page_tables(rng, batch, width, max(width, 4096))
    p = Problem(f"packed_paged_{batch}x{kv_len}", "paged", k, scores, seq_lens,
                row_starts=row_starts, page_table=pt, page_size=page_size)
    return p, table_rows, shifts
