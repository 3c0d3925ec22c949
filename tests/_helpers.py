"""Test helpers: fixture loading and output comparison (no selection logic)."""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(v):
    if isinstance(v, str):
        return float(v)  # "nan", "inf", "-inf"
    return float(v)


def load_hand_cases():
    with open(os.path.join(GOLDEN_DIR, "hand_cases.json")) as f:
        doc = json.load(f)
    cases = []
    for c in doc["cases"]:
        c = dict(c)
        c["scores"] = np.asarray([_num(v) for v in c["scores"]], dtype=np.float32)
        cases.append(c)
    return cases


def valid_counts(seq_lens, k) -> np.ndarray:
    """min(k, max(L, 0)) per row: how many leading slots hold a selection."""
    return np.minimum(np.maximum(np.asarray(seq_lens, dtype=np.int64), 0), int(k))


def canonical(out: np.ndarray, seq_lens, k) -> np.ndarray:
    """First min(k, L) slots of each row sorted ascending, the rest untouched.

    Kernel outputs put the valid entries first in any order and -1 after
    them; sorting the valid prefix gives the comparison form.
    """
    out = np.array(out, dtype=np.int32, copy=True)
    n = valid_counts(seq_lens, k)
    if out.shape[0] and np.all(n == out.shape[1]):
        return np.sort(out, axis=1)
    for r in range(out.shape[0]):
        out[r, :n[r]] = np.sort(out[r, :n[r]])
    return out


def assert_rows_equal(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Exact equality with a readable first mismatch."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    bad = np.nonzero((got != want).any(axis=1))[0]
    if bad.size:
        r = int(bad[0])
        diff = np.nonzero(got[r] != want[r])[0]
        raise AssertionError(
            f"{what}: {bad.size} rows differ; first row {r}, first slots {diff[:8].tolist()}: "
            f"got {got[r, diff[:8]].tolist()} want {want[r, diff[:8]].tolist()}")
