"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/topk_oracle.c``, applies one plausible mistake as a
text substitution, builds the copy into a temporary directory and runs the
pins against it. A mutant that passes every pin means the pins are too weak.
The real oracle source is never modified.
"""
from pathlib import Path

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pins as pins

SRC = Path(oracle.__file__).resolve().parent / "topk_oracle.c"

MUTANTS = {
    # ties broken toward the higher position
    "tie_order_flipped": (
        "    if (a->j < b->j) return -1;\n    if (a->j > b->j) return 1;",
        "    if (a->j < b->j) return 1;\n    if (a->j > b->j) return -1;"),
    # smallest instead of largest scores
    "ascending_scores": (
        "    if (a->w > b->w) return -1;\n    if (a->w < b->w) return 1;",
        "    if (a->w > b->w) return 1;\n    if (a->w < b->w) return -1;"),
    # window start ignored
    "row_start_ignored": (
        "int64_t s = job->row_starts ? job->row_starts[b] : 0;",
        "int64_t s = 0;"),
    # trivial path writes one position too many
    "trivial_off_by_one": (
        "out[t] = t < L ? t : -1;",
        "out[t] = t <= L ? t : -1;"),
    # the k-th pick replaced by the (k+1)-th
    "kth_replaced": (
        "for (int32_t t = 0; t < n; ++t) out[t] = e[t].j;",
        "for (int32_t t = 0; t < n; ++t) out[t] = e[t + (t == n - 1)].j;"),
    # page index taken from the next position
    "page_index_shifted": (
        "page_table[b * pt_stride + (j >> bits)]",
        "page_table[b * pt_stride + ((j + 1) >> bits)]"),
    # in-page offset dropped
    "page_offset_dropped": (
        "out[b * k + t] = page * page_size + (j & (page_size - 1));",
        "out[b * k + t] = page * page_size;"),
    # every row uses row 0's offset
    "ragged_offset_row0": (
        "out[b * k + t] = j < 0 ? -1 : j + out_offsets[b];",
        "out[b * k + t] = j < 0 ? -1 : j + out_offsets[0];"),
    # signed zeros compared by bit pattern (-0.0 below +0.0)
    "signed_zero_by_bits": (
        "    if (a->w > b->w) return -1;",
        "    if (a->w == 0.0f && b->w == 0.0f && signbit(a->w) != signbit(b->w))\n"
        "        return signbit(a->w) ? 1 : -1;\n"
        "    if (a->w > b->w) return -1;"),
    # packed rows read their own table row instead of the mapped one
    "packed_table_row_ignored": (
        "int64_t tr = table_rows ? table_rows[b] : b;",
        "int64_t tr = b;"),
    # packed rows' table start dropped
    "packed_table_start_ignored": (
        "int64_t q = ts + j;",
        "int64_t q = j;"),
    # table start added after the page split (in-page offset only)
    "packed_start_in_offset_only": (
        "int64_t page = page_table[tr * pt_stride + q / page_size];",
        "int64_t page = page_table[tr * pt_stride + j / page_size];"),
    # the window is read one column late
    "window_shifted": (
        "e[j].w = row[j];",
        "e[j].w = row[j + 1 < L ? j + 1 : j];"),
}


def _run_pins(orc):
    """Run the pins; return the name of the first that fails, else None."""
    checks = [
        ("hand_cases", lambda: pins.pin_hand_cases(orc)),
        ("closed_forms", lambda: pins.pin_closed_forms(orc)),
        ("brute_force", lambda: pins.pin_brute_force(orc, rows=300)),
        ("argmax_rounds", lambda: pins.pin_argmax_rounds(orc)),
        ("invariants_small", lambda: _emit_check(orc, "paged_small")),
        ("packed_emit", lambda: pins.pin_packed_emit(orc)),
    ]
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            return name
    return None


def _emit_check(orc, name):
    p = workloads.make_workload(name)
    sel = pins.pin_invariants(orc, p)
    pins.check_emit(p, sel, orc.emit_paged(sel, p.page_table, p.page_size))


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, tmp_path):
    before, after = MUTANTS[mutant]
    text = SRC.read_text()
    assert text.count(before) == 1, f"mutation anchor for {mutant} not found once"
    text = text.replace(before, after)
    if "signbit" in after:
        text = "#include <math.h>\n" + text
    src = tmp_path / "mutant.c"
    src.write_text(text)
    lib = oracle.build(force=True, src=src, lib=tmp_path / "libmutant.so")
    caught_by = _run_pins(oracle.Oracle(lib))
    assert caught_by is not None, f"planted mistake '{mutant}' passed every pin"


def test_unmutated_copy_passes(tmp_path):
    src = tmp_path / "copy.c"
    src.write_text(SRC.read_text())
    lib = oracle.build(force=True, src=src, lib=tmp_path / "libcopy.so")
    assert _run_pins(oracle.Oracle(lib)) is None
    assert np.array_equal(oracle.Oracle(lib).select(np.ones((1, 4), np.float32),
                                                    np.array([4], np.int32), None, 2),
                          np.array([[0, 1]], np.int32))
