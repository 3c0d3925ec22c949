"""GPU parity: the HIP path through the C ABI against the oracle, exact.

Comparison form: the first min(k, L) slots of every row sorted ascending
must equal the oracle's list, the rest must be -1. RAGGED with zero offsets
on the same inputs must equal the oracle's raw positions, so a page-table
error cannot hide behind the PAGED map.
"""
import numpy as np
import pytest

import workloads
from tests._helpers import assert_rows_equal, canonical
from tests import gpu_run
from workloads.edge import PATTERNS, edge_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc(oracle_mod):
    return oracle_mod.default()


def expected(orc, p):
    if p.mode == "ragged":
        return orc.ragged(p.scores, p.seq_lens, p.row_starts, p.out_offsets, p.k)
    return orc.paged(p.scores, p.seq_lens, p.row_starts, p.page_table, p.page_size, p.k)


def check(orc, p, use_plan, with_raw=True):
    print(f"[gpu] {p.name} mode={p.mode} rows={p.num_rows} k={p.k} plan={use_plan}", flush=True)
    d = gpu_run.to_dev(p)
    got, canary_ok = gpu_run.run(p, d, use_plan=use_plan)
    assert canary_ok, "write outside out"
    assert_rows_equal(canonical(got, p.seq_lens, p.k), expected(orc, p), p.name)
    if with_raw:
        raw, _ = gpu_run.run(p, d, use_plan=use_plan, raw=True)
        sel = orc.select(p.scores, p.seq_lens, p.row_starts, p.k)
        assert_rows_equal(canonical(raw, p.seq_lens, p.k), sel, p.name + " raw")
    assert gpu_run.scores_unchanged(p, d), "scores were modified"
    return got


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
@pytest.mark.parametrize("use_plan", [False, True])
def test_workload(orc, name, use_plan):
    p = workloads.make_workload(name)
    check(orc, p, use_plan, with_raw=not use_plan)


def _edge_rows(k):
    rows = []
    for r in range(4):
        for L in (0, -3, 1, k - 1, k, k + 1, 8189 - r, 8192 - r, 8193 - r, 18432 - r,
                  18433 - r, 20000, 65537):
            rows.append((L, r, "normal"))
    for r in range(4):
        for pat in PATTERNS:
            for L in (3000, 12000, 30000):
                rows.append((L, r, pat))
    rows += [(131072, 1, "fp16"), (131072, 3, "equal"), (131072, 0, "alphabet"),
             (131072, 2, "normal")]
    return rows


@pytest.mark.parametrize("mode", ["ragged", "paged"])
@pytest.mark.parametrize("k", [2048, 1000, 7, 1])
def test_edge_batch(orc, mode, k):
    p = edge_batch(1000 + k, mode, k, _edge_rows(k), name=f"edge_{mode}_k{k}")
    check(orc, p, use_plan=(k == 1000))


@pytest.mark.parametrize("page_size", [1, 2, 4096])
def test_page_sizes(orc, page_size):
    rows = [(L, r, pat) for r in range(4) for L in (5000, 9000, 25000)
            for pat in ("normal", "alphabet")]
    p = edge_batch(77, "paged", 512, rows, page_size=page_size, name=f"pages_{page_size}")
    check(orc, p, use_plan=False, with_raw=False)


def test_register_rows_are_byte_deterministic(orc):
    p = workloads.make_workload("paged_decode")
    d = gpu_run.to_dev(p)
    first, _ = gpu_run.run(p, d)
    for _ in range(3):
        again, _ = gpu_run.run(p, d)
        assert np.array_equal(first, again)


def test_repeat_runs_give_the_same_sets(orc):
    p = workloads.make_workload("paged_mixed")
    d = gpu_run.to_dev(p)
    first, _ = gpu_run.run(p, d, use_plan=True)
    for _ in range(2):
        again, _ = gpu_run.run(p, d, use_plan=True)
        assert np.array_equal(canonical(first, p.seq_lens, p.k),
                              canonical(again, p.seq_lens, p.k))


def test_zero_rows_noop():
    import torch

    import row_top_selection_amd as dt

    s = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    lens = torch.zeros(0, dtype=torch.int32, device="cuda")
    out = dt.ragged(s, lens, lens, 4)
    torch.cuda.synchronize()
    assert out.shape == (0, 4)
