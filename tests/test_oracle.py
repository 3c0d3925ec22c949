"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import workloads
from tests import oracle_pins as pins


@pytest.fixture(scope="module")
def orc(oracle_mod):
    return oracle_mod.default()


def test_hand_cases(orc):
    pins.pin_hand_cases(orc)


def test_packed_emit(orc):
    pins.pin_packed_emit(orc)


def test_brute_force_tiny_rows(orc):
    pins.pin_brute_force(orc)


def test_argmax_rounds(orc):
    pins.pin_argmax_rounds(orc)


def test_closed_forms(orc):
    pins.pin_closed_forms(orc)


@pytest.mark.parametrize("name", ["paged_small", "paged_decode", "paged_long"])
def test_stable_argsort(orc, name):
    p = workloads.make_workload(name)
    pins.pin_stable_argsort(orc, p.scores, p.seq_lens, p.k, p.row_starts)


def test_stable_argsort_ragged_sample(orc):
    p = workloads.make_workload("ragged_extend")
    rows = np.arange(0, p.num_rows, 97)
    pins.pin_stable_argsort(orc, p.scores[rows], p.seq_lens[rows], p.k, p.row_starts[rows])


def test_torch_topk_tie_free(orc):
    p = workloads.make_workload("paged_decode")
    pins.pin_torch_topk_tie_free(orc, p.scores, p.seq_lens, p.k)


@pytest.mark.parametrize("name", ["paged_small", "paged_decode", "paged_long", "paged_mixed",
                                  "ragged_extend"])
def test_workload_invariants_and_emit(orc, name):
    p = workloads.make_workload(name)
    sel = pins.pin_invariants(orc, p)
    if p.mode == "ragged":
        out = orc.emit_ragged(sel, p.out_offsets)
    else:
        out = orc.emit_paged(sel, p.page_table, p.page_size)
    pins.check_emit(p, sel, out)


def test_trivial_rows_never_read_scores(orc):
    """Poisoning the scores of rows with L <= k changes nothing."""
    p = workloads.make_workload("paged_mixed")
    poisoned = p.scores.copy()
    trivial = p.seq_lens <= p.k
    poisoned[trivial] = np.nan
    a = orc.paged(p.scores, p.seq_lens, None, p.page_table, p.page_size, p.k)
    b = orc.paged(poisoned, p.seq_lens, None, p.page_table, p.page_size, p.k)
    assert trivial.any() and np.array_equal(a, b)


def test_thread_count_does_not_matter(orc):
    p = workloads.make_workload("paged_mixed")
    a = orc.select(p.scores, p.seq_lens, None, p.k, threads=1)
    b = orc.select(p.scores, p.seq_lens, None, p.k, threads=7)
    assert np.array_equal(a, b)


def test_argument_errors(orc):
    with pytest.raises(ValueError):
        orc.select(np.zeros((2, 8), np.float32), np.array([9, 1], np.int32), None, 4)
    with pytest.raises(ValueError):
        orc.paged(np.zeros((1, 8), np.float32), np.array([8], np.int32), None,
                  np.zeros((1, 8), np.int32), 3, 4)
    assert orc.select(np.zeros((0, 8), np.float32), np.zeros(0, np.int32), None, 4).shape == (0, 4)
