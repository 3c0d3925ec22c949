"""CPU oracle for the windowed per-row top-k selection (RAGGED and PAGED emit).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library
(``row_top_selection_amd``) never imports it, and this package imports
nothing from the GPU library.

The arithmetic lives in ``topk_oracle.c`` (plain C, full sort per row); its
header lists the passages of the pages that each rule follows. This module
only builds that file with gcc, marshals numpy arrays to it, and exposes:

- :func:`select`  - selected window positions, ascending, then -1 padding
- :func:`ragged`  - RAGGED outputs (position + out_offset), same layout
- :func:`paged`   - PAGED outputs (page-table mapped), valid slots sorted
- ``Oracle.paged_packed`` - packed PAGED outputs (a table-row map and table
  starts per row), valid slots sorted

All results are int32 ``[num_rows, k]`` with the valid slots first.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "topk_oracle.c"
_LIB_DIR = _HERE / "_build"
_LIB = _LIB_DIR / "liboracle_topk.so"

_default = None


def build(force: bool = True, src: Path = _SRC, lib: Path = _LIB) -> Path:
    """Compile ``topk_oracle.c`` (or ``src``) with gcc into ``lib``."""
    if force or not lib.exists() or lib.stat().st_mtime < src.stat().st_mtime:
        lib.parent.mkdir(exist_ok=True)
        tmp = lib.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
             str(src), "-o", str(tmp)],
            check=True,
        )
        os.replace(tmp, lib)
    return lib


class Oracle:
    """ctypes front end of one build of the oracle library."""

    def __init__(self, path):
        lib = ctypes.CDLL(str(path))
        P = ctypes.c_void_p
        lib.oracle_select.argtypes = [P, ctypes.c_int64, P, P, ctypes.c_int32,
                                      ctypes.c_int32, P, ctypes.c_int32]
        lib.oracle_select.restype = ctypes.c_int
        lib.oracle_emit_ragged.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P]
        lib.oracle_emit_ragged.restype = None
        lib.oracle_emit_paged.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P,
                                          ctypes.c_int64, ctypes.c_int32, P]
        lib.oracle_emit_paged.restype = ctypes.c_int
        lib.oracle_emit_paged_packed.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P,
                                                 ctypes.c_int64, ctypes.c_int32, P, P, P]
        lib.oracle_emit_paged_packed.restype = ctypes.c_int
        self.lib = lib

    def select(self, scores, seq_lens, row_starts, k, threads=None):
        return _select(self.lib, scores, seq_lens, row_starts, k, threads)

    def emit_ragged(self, sel, out_offsets):
        return _emit_ragged(self.lib, sel, out_offsets)

    def emit_paged(self, sel, page_table, page_size):
        return _emit_paged(self.lib, sel, page_table, page_size)

    def ragged(self, scores, seq_lens, row_starts, out_offsets, k, threads=None):
        """RAGGED outputs: ascending (position + out_offset), then -1."""
        return self.emit_ragged(self.select(scores, seq_lens, row_starts, k, threads),
                                out_offsets)

    def paged(self, scores, seq_lens, row_starts, page_table, page_size, k, threads=None):
        """PAGED outputs: ascending page-table-mapped positions, then -1."""
        return self.emit_paged(self.select(scores, seq_lens, row_starts, k, threads),
                               page_table, page_size)

    def emit_paged_packed(self, sel, page_table, page_size, table_rows=None, table_starts=None):
        return _emit_paged_packed(self.lib, sel, page_table, page_size, table_rows, table_starts)

    def paged_packed(self, scores, seq_lens, row_starts, page_table, page_size, k,
                     table_rows=None, table_starts=None, threads=None):
        """Packed PAGED outputs: row b maps window position j through table
        row table_rows[b] at table position table_starts[b] + j."""
        return self.emit_paged_packed(self.select(scores, seq_lens, row_starts, k, threads),
                                      page_table, page_size, table_rows, table_starts)


def default() -> Oracle:
    """The oracle built from ``topk_oracle.c`` (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle(build(force=False))
    return _default


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _i32(a, n, name):
    a = np.ascontiguousarray(a, dtype=np.int32)
    if a.shape != (n,):
        raise ValueError(f"{name} must have shape ({n},), got {a.shape}")
    return a


def _select(lib, scores, seq_lens, row_starts, k, threads=None):
    """Selected window positions per row.

    ``scores`` is a 2-D float32 array ``[num_rows, stride]``; row b's window is
    ``scores[b, s_b : s_b + L_b]`` with ``s_b = row_starts[b]`` (0 if
    ``row_starts`` is None) and ``L_b = max(seq_lens[b], 0)``.
    Returns int32 ``[num_rows, k]``: ascending positions, then -1.
    """
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if scores.ndim != 2:
        raise ValueError("scores must be 2-D [num_rows, stride]")
    R, stride = scores.shape
    seq_lens = _i32(seq_lens, R, "seq_lens")
    if row_starts is not None:
        row_starts = _i32(row_starts, R, "row_starts")
        ends = row_starts.astype(np.int64) + np.maximum(seq_lens, 0)
        if R and (row_starts.min() < 0 or ends.max() > stride):
            raise ValueError("window outside the score row")
    elif R and np.maximum(seq_lens, 0).max() > stride:
        raise ValueError("window outside the score row")
    k = int(k)
    sel = np.empty((R, k), dtype=np.int32)
    if R == 0:
        return sel
    rc = lib.oracle_select(_ptr(scores), stride, _ptr(seq_lens), _ptr(row_starts),
                           R, k, _ptr(sel), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_select failed with code {rc}")
    return sel


def _emit_ragged(lib, sel, out_offsets):
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    R, k = sel.shape
    out_offsets = _i32(out_offsets, R, "out_offsets")
    out = np.empty_like(sel)
    if R:
        lib.oracle_emit_ragged(_ptr(sel), R, k, _ptr(out_offsets), _ptr(out))
    return out


def _emit_paged(lib, sel, page_table, page_size):
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    R, k = sel.shape
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    if page_table.ndim != 2 or page_table.shape[0] != R:
        raise ValueError("page_table must be [num_rows, width]")
    out = np.empty_like(sel)
    if R:
        rc = lib.oracle_emit_paged(_ptr(sel), R, k, _ptr(page_table),
                                   page_table.shape[1], int(page_size), _ptr(out))
        if rc != 0:
            raise ValueError("page_size must be a power of two >= 1")
    return out


def _emit_paged_packed(lib, sel, page_table, page_size, table_rows, table_starts):
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    R, k = sel.shape
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    if page_table.ndim != 2:
        raise ValueError("page_table must be [table_rows, width]")
    T, W = page_table.shape
    tr = None if table_rows is None else _i32(table_rows, R, "table_rows")
    ts = None if table_starts is None else _i32(table_starts, R, "table_starts")
    rows = tr if tr is not None else np.arange(R)
    if R and (rows.min() < 0 or rows.max() >= T):
        raise ValueError("table row outside the page table")
    q_max = (0 if ts is None else ts.astype(np.int64)) + sel.max(axis=1).astype(np.int64)
    if R and (q_max // int(page_size)).max() >= W:
        raise ValueError("table position outside the page-table row")
    out = np.empty_like(sel)
    if R:
        rc = lib.oracle_emit_paged_packed(_ptr(sel), R, k, _ptr(page_table), W, int(page_size),
                                          _ptr(tr), _ptr(ts), _ptr(out))
        if rc == 1:
            raise ValueError("page_size must be a power of two >= 1")
        if rc == 2:
            raise ValueError("negative table position")
    return out


def select(scores, seq_lens, row_starts, k, threads=None):
    """Selected window positions: ascending, then -1 (see :class:`Oracle`)."""
    return default().select(scores, seq_lens, row_starts, k, threads)


def ragged(scores, seq_lens, row_starts, out_offsets, k, threads=None):
    """RAGGED outputs: ascending (position + out_offset), then -1."""
    return default().ragged(scores, seq_lens, row_starts, out_offsets, k, threads)


def paged(scores, seq_lens, row_starts, page_table, page_size, k, threads=None):
    """PAGED outputs: ascending page-table-mapped positions, then -1."""
    return default().paged(scores, seq_lens, row_starts, page_table, page_size, k, threads)
