"""dsatopk_paged_noalloc (the plan in the library's static device memory)
against dsatopk_paged with a plan buffer the caller allocates: two calls in
a row on the same GPU, the second with a smaller batch, each exact against
the existing entry point (rows compared as sorted lists: split rows order
their outputs by segment arrival)."""
import pytest

import workloads
from tests import gpu_run
from tests._helpers import assert_rows_equal, canonical

pytestmark = pytest.mark.gpu


def _both(p):
    import torch

    import row_top_selection_amd as dt

    d = gpu_run.to_dev(p)
    plan = dt.plan(d["lens"], p.k, row_starts=d["starts"])
    ref = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, row_starts=d["starts"],
                   plan=plan)
    got = dt.paged_noalloc(d["scores"], d["lens"], d["pt"], p.page_size, p.k,
                           row_starts=d["starts"])
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_paged_on_two_calls():
    """512 mixed rows (split rows merge through the scratch's exchange
    areas), then 8 long rows (a smaller batch over what the first call left
    in the scratch)."""
    for p in (workloads.make_workload("paged_mixed"), workloads.make_workload("paged_long")):
        print(f"[gpu] noalloc {p.name} rows={p.num_rows}", flush=True)
        ref, got = _both(p)
        assert_rows_equal(canonical(got, p.seq_lens, p.k), canonical(ref, p.seq_lens, p.k),
                          p.name)
