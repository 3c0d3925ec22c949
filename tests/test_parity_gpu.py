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

# long rows of a batch are split when there are at most this many (the plan
# buffer reserves this many exchange areas)
SPLIT_CAP = 256


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


def test_many_rows_use_the_narrow_kernel(orc):
    """More than 512 rows: short rows take the 256-thread kernel."""
    p = workloads.scaled_decode(1024)
    check(orc, p, use_plan=False, with_raw=False)


@pytest.mark.parametrize("use_plan", [False, True])
@pytest.mark.parametrize("mode", ["paged", "ragged"])
def test_large_short_batch(orc, mode, use_plan):
    """4096 rows of spans up to 8192 floats in a score stride of 8196 (the
    mid-stride kernel's 8-float4 rows), with mixed lengths and window
    offsets, trivial rows among them, and fp16 ties."""
    p = workloads.short_mix(4096, mode)
    assert (p.seq_lens <= p.k).any() and (p.seq_lens > p.k).any()
    got = check(orc, p, use_plan, with_raw=False)
    again, _ = gpu_run.run(p, gpu_run.to_dev(p), use_plan=use_plan)
    assert np.array_equal(got, again), "register rows are byte-deterministic"


def _edge_rows(k):
    rows = []
    for r in range(4):
        for L in (0, -3, 1, k - 1, k, k + 1, 8189 - r, 8192 - r, 8193 - r, 18432 - r,
                  18433 - r, 20000, 32768 - r, 32769 - r, 40960 - r, 40961 - r, 53248 - r,
                  53249 - r, 65536 - r, 65537 - r):
            rows.append((L, r, "normal"))
    for r in range(4):
        for pat in PATTERNS:
            for L in (3000, 12000, 30000):
                rows.append((L, r, pat))
    rows += [(131072, 1, "fp16"), (131072, 3, "equal"), (131072, 0, "alphabet"),
             (131072, 2, "normal")]
    # streamed rows whose largest keys crowd the first columns (the list's
    # opening threshold is then above the k-th key: two-pass re-read), rise
    # along the row (the list fills and is compacted again and again), are
    # all -inf, or rise over the first 16384 columns only (more pairs reach
    # the opening threshold than the list holds)
    rows += [(131072, 2, "decreasing"), (40000, 3, "decreasing"), (131072, 0, "increasing"),
             (65537, 1, "neg_inf"), (131072, 1, "rising_head"), (65536, 3, "rising_head")]
    return rows


@pytest.mark.parametrize("use_plan", [False, True, "stale"])
@pytest.mark.parametrize("mode", ["ragged", "paged"])
@pytest.mark.parametrize("k", [2048, 1000, 7, 1])
def test_edge_batch(orc, mode, k, use_plan):
    """Every length class, start residue and value pattern: without a plan
    (long rows streamed), with the batch's plan (long rows split) and with a
    plan built for other lengths (long rows the plan does not split are read
    in register pieces by the register kernel, and rows that defeat the
    pieces' threshold by its two-pass path)."""
    p = edge_batch(1000 + k, mode, k, _edge_rows(k), name=f"edge_{mode}_k{k}")
    check(orc, p, use_plan=use_plan, with_raw=use_plan is False)


# Score strides that select each register kernel (a row's span never exceeds
# the stride): up to 8192 floats the short-row kernels (512 threads per row
# up to 512 rows, 256 threads above), up to 16384 the mid kernel (8 or 16
# float4 per thread by the row's span).
BANDS = {
    "wide": (8192, 1),    # <= 512 rows: rows_wide_kernel
    "short": (8192, 0),   # the rows repeated past 512 rows: rows_short_kernel
    "mid": (16384, 1),    # spans on both sides of 8192: both mid-kernel branches
}


def _band_rows(k, stride):
    """Every start residue; lengths -3, 0, 1, k-1, k, k+1 and the four spans
    below the stride (plus, in the mid band, the spans around 8192); every
    value pattern and tie classes of at most 64 and more than 64 elements at
    a short and at the longest span."""
    rows = []
    for r in range(4):
        top = [stride - r - d for d in range(4)]
        mids = [8189 - r, 8192 - r, 8193 - r, 12000] if stride > 8192 else [4097]
        for L in (-3, 0, 1, k - 1, k, k + 1, *mids, *top):
            rows.append((L, r, "normal"))
        for pat in PATTERNS:
            for L in (3000, stride - r):
                rows.append((L, r, pat))
        for L in (3000, stride - r):
            for tied, need in ((64, 1), (64, 37), (64, 63), (65, 40), (2, 1), (33, 17),
                               (200, 150)):
                if need <= k and k - need + tied <= L:
                    rows.append((L, r, ("ties", k - need, tied)))
    return rows


@pytest.mark.parametrize("mode", ["ragged", "paged"])
@pytest.mark.parametrize("k", [2048, 1000, 7, 1])
@pytest.mark.parametrize("band", list(BANDS))
def test_band_edges(orc, band, k, mode):
    """The edge suite on the register kernels of short strides: the
    512-thread wide kernel (the paged decode kernel), the 256-thread short
    kernel and both branches of the mid kernel, with trivial rows, every
    start residue, signed zeros, infinities, equal rows and tie classes."""
    stride, reps = BANDS[band]
    rows = _band_rows(k, stride)
    rows = rows * (reps or 512 // len(rows) + 1)
    p = edge_batch(5000 + k + 7 * stride + reps, mode, k, rows, stride=stride,
                   name=f"band_{band}_{mode}_k{k}")
    assert p.stride == stride
    assert (p.num_rows <= 512) == (band != "short")
    check(orc, p, use_plan=False, with_raw=(mode == "paged"))


def _rank_bin_row(rng, L, above, cnt, dup):
    """above keys at 5.0, then cnt keys inside one bin of the top 14 key
    bits (floats just above 0.75, every dup-th one repeating its
    predecessor: position ties inside the bin), the rest in (-1, 0.5)."""
    v = rng.uniform(-1.0, 0.5, size=L).astype(np.float32)
    idx = rng.permutation(L)[:above + cnt]
    v[idx[:above]] = 5.0
    bits = np.uint32(0x3F400001) + rng.permutation(1 << 16)[:cnt].astype(np.uint32)
    if dup:
        bits[dup::dup] = bits[dup - 1:-1:dup][:len(bits[dup::dup])]
    v[idx[above:]] = bits.view(np.float32)
    return v


@pytest.mark.parametrize("mode", ["paged", "ragged"])
@pytest.mark.parametrize("k", [2048, 1100])
def test_decode_rank_bin_sizes(orc, mode, k):
    """The decode rows' direct rank around its capacity: the k-th key's
    14-bit bin holding 2, 64, 255, 256 (ranked) and 257, 400 (the 12-bit
    fallback) elements, of which 1, half or all but one are taken, with and
    without repeated keys, at every start residue (wide kernel: stride
    8192, at most 512 rows)."""
    from workloads.configs import OUTSIDE_SCORE, PAGE_SIZE, Problem, random_page_tables

    rng = np.random.default_rng(7100 + k)
    stride, L = 8192, 8000
    rows = []
    for cnt in (2, 64, 255, 256, 257, 400):
        for take in sorted({1, cnt // 2, cnt - 1} - {0}):
            for dup in (0, 3):
                rows.append((cnt, take, dup))
    R = len(rows) * 4
    scores = np.full((R, stride), OUTSIDE_SCORE, dtype=np.float32)
    starts = np.zeros(R, dtype=np.int32)
    lens = np.full(R, L, dtype=np.int32)
    for i, (cnt, take, dup) in enumerate(rows):
        for r in range(4):
            b = 4 * i + r
            starts[b] = r + 4 * (b % 3)
            scores[b, starts[b]:starts[b] + L] = _rank_bin_row(rng, L, k - take, cnt, dup)
    assert R <= 512 and (starts + lens <= stride).all()
    if mode == "ragged":
        offs = rng.integers(0, 1 << 20, size=R).astype(np.int32)
        p = Problem(f"rank_bins_{mode}_k{k}", "ragged", k, scores, lens, row_starts=starts,
                    out_offsets=offs)
    else:
        pt = random_page_tables(rng, R, -(-L // PAGE_SIZE), 1 << 12)
        p = Problem(f"rank_bins_{mode}_k{k}", "paged", k, scores, lens, row_starts=starts,
                    page_table=pt, page_size=PAGE_SIZE)
    check(orc, p, use_plan=False, with_raw=(mode == "paged"))


def _long_all_rows(k, stride=65536):
    """Every start residue; lengths -3, 0, 1, k-1, k, k+1, 12000, the spans
    around 40960 and 49152 and the four spans below the stride; every value
    pattern and tie classes of at most 64 and more than 64 elements."""
    rows = []
    for r in range(4):
        top = [stride - r - d for d in range(4)]
        for L in (-3, 0, 1, k - 1, k, k + 1, 12000, 40959 - r, 40960 - r, 40961 - r,
                  49152 - r, *top):
            rows.append((L, r, "normal"))
        for pat in PATTERNS:
            for L in (3000, 45000 - r, stride - r):
                rows.append((L, r, pat))
        for L in (3000, stride - r):
            for tied, need in ((64, 1), (64, 37), (65, 40), (2, 1), (200, 150)):
                if need <= k and k - need + tied <= L:
                    rows.append((L, r, ("ties", k - need, tied)))
    return rows


@pytest.mark.parametrize("mode,k,use_plan,stride", [
    ("paged", 2048, True, 57344), ("ragged", 1, True, 57344),
    ("paged", 7, False, 65536), ("ragged", 2048, False, 65536),
    ("paged", 2048, True, 65536), ("ragged", 1, True, 65536)])
def test_large_batch_at_long_strides(orc, mode, k, use_plan, stride):
    """A batch of 1024 rows or more at a score stride of 57344 or 65536
    floats, with every row kind (trivial, short, register-length and long,
    up to the stride), every start residue, the value patterns and tie
    classes. Up to 57344 (65536 without a plan) the long-row kernel alone
    serves every row and a given plan is not used; at 65536 with a plan
    the register kernel serves them, the long rows in pieces."""
    rows = _long_all_rows(k, stride)
    rows = rows * (1024 // len(rows) + 1)
    p = edge_batch(6000 + k + stride, mode, k, rows, stride=stride,
                   name=f"long_all_{mode}_k{k}_s{stride}")
    assert p.stride == stride and p.num_rows >= 1024
    check(orc, p, use_plan=use_plan, with_raw=(mode == "paged"))


def test_all_trivial_rows(orc):
    """Every row's window fits in k: the trivial path alone, compared with
    the oracle (the counter run shows that it reads no scores)."""
    p = workloads.all_trivial()
    check(orc, p, use_plan=True, with_raw=True)


def _tie_rows(k):
    rows = []
    for L in (3000, 12000, 30000, 60000, 131072):
        for tied, need in ((64, 1), (64, 37), (64, 63), (65, 40), (2, 1), (33, 17), (200, 150)):
            if need <= k and k - need + tied <= L:
                rows.append((L, L % 4, ("ties", k - need, tied)))
    return rows


@pytest.mark.parametrize("use_plan", [False, True])
@pytest.mark.parametrize("mode", ["ragged", "paged"])
@pytest.mark.parametrize("k", [2048, 100])
def test_tie_class_sizes(orc, mode, k, use_plan):
    """The k-th key shared by 2 to 200 elements, of which 1 to 150 are
    taken (lowest positions first): tie classes of at most 64 elements and
    larger ones, on every row length class."""
    p = edge_batch(3000 + k, mode, k, _tie_rows(k), name=f"ties_{mode}_k{k}")
    check(orc, p, use_plan=use_plan, with_raw=not use_plan)


def _plan_words(plan):
    return plan.cpu().numpy().view(np.int32)


# The plan's layout (int32 words), as the library writes it: a 64-word
# header (words 4..7 the rows per class, 12 the split rows, 13 their work
# items, 14 the error word, 15 the poll limit, 16 the segment length), then
# per row its class-list entry, class, segment count and exchange slot,
# then 2 words per work item (up to 33 per split row), then one
# 10432-word exchange area per split row (histogram 0..4095, candidate
# pairs 4096..8191, their emitted values 8192..10239, counters from 10240
# on, each on a 128-byte line of its own).
MAX_SEG = 33
X_WORDS = 10432


def _layout(R):
    cap = min(R, SPLIT_CAP)
    items = 64 + 4 * R
    xarea = (items + 2 * cap * MAX_SEG + 63) // 64 * 64
    return items, xarea


@pytest.mark.parametrize("name", ["paged_long", "paged_mixed"])
def test_plan_reuse_and_exchange_reset(orc, name):
    """One plan serves several calls; split rows' exchange areas end
    zeroed and no segment ever gave up waiting."""
    import torch

    import row_top_selection_amd as dt

    p = workloads.make_workload(name)
    d = gpu_run.to_dev(p)
    plan = dt.plan(d["lens"], p.k, row_starts=d["starts"])
    torch.cuda.synchronize()
    words = _plan_words(plan)
    n_split, n_items = int(words[12]), int(words[13])
    assert n_split > 0 and n_items >= 2 * n_split
    assert words[16] in (4096, 8192)
    want = expected(orc, p)
    for _ in range(3):
        out = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, plan=plan)
        torch.cuda.synchronize()
        assert_rows_equal(canonical(out.cpu().numpy(), p.seq_lens, p.k), want, name)
    assert dt.plan_error(plan) == 0, "a segment gave up waiting for its row"
    words = _plan_words(plan)
    _, xarea = _layout(p.num_rows)
    x = words[xarea: xarea + n_split * X_WORDS].reshape(n_split, X_WORDS)
    # histograms and counters must be zero again; the candidate pairs and
    # values (words 4096..10239) are overwritten before they are read
    assert not x[:, :4096].any(), "exchange histograms were not left zeroed"
    assert not x[:, 10240:].any(), "exchange counters were not reset"


@pytest.mark.parametrize("R", [1, 65, 300, 1000])
def test_plan_of_any_batch_size_splits_and_zeroes(orc, R):
    """Plans whose workgroups take 256, 320 and 1024 threads (the least
    multiple of 64 covering the rows, at least 256), each over a batch of
    trivial rows with long rows at its first, middle and last positions:
    the plan splits every long row and zeroes each split row's exchange
    area in a buffer that starts out full of garbage, and the transform
    with it equals the oracle."""
    import torch

    import row_top_selection_amd as dt

    long_at = sorted({0, R // 2, R - 1})
    rows = [(100, 0, "normal")] * R
    for i in long_at:
        rows[i] = (70000 - i % 4, i % 4, "normal")
    p = edge_batch(7100 + R, "paged", 2048, rows, name=f"plan_block_{R}")
    print(f"[gpu] plan block R={R}", flush=True)
    d = gpu_run.to_dev(p)
    plan = torch.full((dt.plan_bytes(R),), 0x5A, dtype=torch.uint8, device=d["lens"].device)
    dt.plan(d["lens"], p.k, row_starts=d["starts"], out=plan)
    torch.cuda.synchronize()
    words = _plan_words(plan)
    n_split = int(words[12])
    assert words[4 + 3] == len(long_at) and n_split == len(long_at)
    _, xarea = _layout(R)
    x = words[xarea: xarea + n_split * X_WORDS].reshape(n_split, X_WORDS)
    assert not x[:, :4096].any(), "exchange histograms were not zeroed"
    assert not x[:, 10240:].any(), "exchange counters were not zeroed"
    out = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, row_starts=d["starts"],
                   plan=plan)
    torch.cuda.synchronize()
    assert_rows_equal(canonical(out.cpu().numpy(), p.seq_lens, p.k), expected(orc, p), p.name)
    assert dt.plan_error(plan) == 0


def test_split_row_that_gives_up_reads_minus_one(orc):
    """A plan whose work list leaves out one segment of a split row, with a
    small poll limit: that row's other segments give up waiting (bounded
    polls, every kernel exits), the row's outputs are all -1, the plan's
    error word is set, and every other row is exact. A fresh plan then
    serves the same batch exactly."""
    import torch

    import row_top_selection_amd as dt

    p = workloads.make_workload("paged_long")
    d = gpu_run.to_dev(p)
    want = expected(orc, p)
    plan = dt.plan(d["lens"], p.k)
    torch.cuda.synchronize()
    w = torch.from_numpy(_plan_words(plan).copy())
    items, _ = _layout(p.num_rows)
    n_items = int(w[13])
    row_items = [i for i in range(n_items) if int(w[items + 2 * i]) == 3]
    assert len(row_items) >= 2
    w[items + 2 * row_items[1]] = -1  # no worker serves this segment
    w[15] = 4096  # polls before a wait gives up
    plan.copy_(w.view(torch.uint8).to(plan.device))
    print("[gpu] split row with a missing segment", flush=True)
    out = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, plan=plan)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[3] == -1).all(), "the row that lost a segment must read -1"
    others = [b for b in range(p.num_rows) if b != 3]
    assert_rows_equal(canonical(got[others], p.seq_lens[others], p.k), want[others], "others")
    assert dt.plan_error(plan) == 1
    plan = dt.plan(d["lens"], p.k, out=plan)
    out = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, plan=plan)
    torch.cuda.synchronize()
    assert_rows_equal(canonical(out.cpu().numpy(), p.seq_lens, p.k), want, "fresh plan")
    assert dt.plan_error(plan) == 0


def test_binding_rejects_misplaced_arguments():
    """The binding refuses arguments the C ABI would misread: a page table
    that is not int32, and outputs or a plan that are not on the scores'
    device (nothing is launched)."""
    import torch

    import row_top_selection_amd as dt

    s = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    lens = torch.full((4,), 64, dtype=torch.int32, device="cuda")
    pt = torch.zeros((4, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        dt.paged(s, lens, pt.long(), 64, 8)
    with pytest.raises(ValueError):
        dt.paged(s, lens, pt.cpu(), 64, 8)
    with pytest.raises(ValueError):
        dt.paged(s, lens, pt, 64, 8, out=torch.zeros((4, 8), dtype=torch.int32))
    with pytest.raises(ValueError):
        dt.paged(s, lens, pt, 64, 8, out_raw=torch.zeros((4, 8), dtype=torch.int32))
    with pytest.raises(ValueError):
        dt.paged(s, lens, pt, 64, 8, plan=torch.zeros(dt.plan_bytes(4), dtype=torch.uint8))
    with pytest.raises(ValueError):
        dt.ragged(s, lens, lens, 8, out=torch.zeros((4, 8), dtype=torch.int32))
    with pytest.raises(ValueError):
        dt.ragged(s, lens, lens, 8, plan=torch.zeros(dt.plan_bytes(4), dtype=torch.uint8))
    with pytest.raises(ValueError):
        dt.plan(lens, 8, out=torch.zeros(dt.plan_bytes(4), dtype=torch.uint8))


def test_stale_plan_gives_same_outputs(orc):
    """A plan built for other lengths still yields exact results."""
    import torch

    import row_top_selection_amd as dt

    p = workloads.make_workload("paged_mixed")
    d = gpu_run.to_dev(p)
    other = torch.from_numpy(np.roll(p.seq_lens, 7)).to(d["lens"].device)
    plan = dt.plan(other, p.k)
    out = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, plan=plan)
    torch.cuda.synchronize()
    assert_rows_equal(canonical(out.cpu().numpy(), p.seq_lens, p.k), expected(orc, p), "stale")
    assert dt.plan_error(plan) == 0


def test_plan_of_a_larger_batch_gives_same_outputs(orc):
    """A plan built for more rows (the batch's lengths followed by long
    rows) is large enough for the call but belongs to another batch size:
    the row kernels keep their own order and split nothing, and the
    results stay exact."""
    import torch

    import row_top_selection_amd as dt

    p = workloads.make_workload("paged_mixed")
    d = gpu_run.to_dev(p)
    more = np.concatenate([p.seq_lens, np.full(5, 131072, dtype=np.int32)])
    plan = dt.plan(torch.from_numpy(more).to(d["lens"].device), p.k)
    assert plan.numel() >= dt.plan_bytes(p.num_rows)
    out = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, plan=plan)
    torch.cuda.synchronize()
    assert_rows_equal(canonical(out.cpu().numpy(), p.seq_lens, p.k), expected(orc, p),
                      "larger plan")


@pytest.mark.parametrize("page_size", [1, 2, 4096])
def test_page_sizes(orc, page_size):
    rows = [(L, r, pat) for r in range(4) for L in (5000, 9000, 25000)
            for pat in ("normal", "alphabet")]
    p = edge_batch(77, "paged", 512, rows, page_size=page_size, name=f"pages_{page_size}")
    check(orc, p, use_plan=False, with_raw=False)


@pytest.mark.parametrize("page_size", [1, 2, 8, 16])
def test_page_sizes_short_stride(orc, page_size):
    """Rows in a score stride of 8192 with few rows (the rows of small
    batches, 512 threads each): for an 8192-float window, page sizes 1, 2
    and 8 need more table entries than the row's LDS copy holds, so the
    emit reads the table from memory; 16 fills the copy exactly."""
    rows = [(L, r, pat) for r in range(4) for L in (3000, 4097, 8192 - r)
            for pat in ("normal", "alphabet")]
    p = edge_batch(78, "paged", 1000, rows, page_size=page_size, name=f"short_pages_{page_size}",
                   stride=8192)
    assert p.stride == 8192 and p.num_rows <= 512
    check(orc, p, use_plan=False, with_raw=True)


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


@pytest.mark.parametrize("name", ["paged_decode", "paged_long", "ragged_extend", "paged_mixed"])
def test_graph_replay_matches_eager(orc, name):
    """plan + transform captured in a HIP graph: every replay, with eager
    work and synchronizations between replays, selects what the eager call
    and the oracle select (split rows included: their exchange areas must be
    zero again for the next replay; the mixed batch's register rows in the
    plan's class order). Register-path rows are byte-equal; the split path
    orders a row's outputs by segment arrival."""
    import torch

    import row_top_selection_amd as dt

    p = workloads.make_workload(name)
    print(f"[gpu] graph replay {name}", flush=True)
    d = gpu_run.to_dev(p)
    out = torch.empty((p.num_rows, p.k), dtype=torch.int32, device="cuda")
    plan = dt.plan(d["lens"], p.k, row_starts=d["starts"])

    def step():
        dt.plan(d["lens"], p.k, row_starts=d["starts"], out=plan)
        if p.mode == "ragged":
            dt.ragged(d["scores"], d["lens"], d["offs"], p.k, row_starts=d["starts"], plan=plan,
                      out=out)
        else:
            dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, row_starts=d["starts"],
                     plan=plan, out=out)

    step()
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    assert_rows_equal(canonical(eager, p.seq_lens, p.k), expected(orc, p), name)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.zeros(1 << 20, device="cuda")
    for it in range(4):
        out.fill_(-5)
        scratch.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        if name == "paged_decode":
            assert np.array_equal(got, eager), f"replay {it} differs from the eager call"
        assert_rows_equal(canonical(got, p.seq_lens, p.k), expected(orc, p),
                          f"{name} replay {it}")
    assert dt.plan_error(plan) == 0, "a segment gave up waiting for its row"


def test_many_long_rows_are_read_in_pieces(orc):
    """More long rows than the split path takes: the plan splits none of
    them, and every long row is read in pieces by one workgroup of the
    register kernel (with the plan) or streamed by one of the long-row
    kernel (without it)."""
    import torch

    import row_top_selection_amd as dt

    p = workloads.scaled_long(SPLIT_CAP + 1)
    print(f"[gpu] {p.name} in pieces / streamed", flush=True)
    d = gpu_run.to_dev(p)
    plan = dt.plan(d["lens"], p.k)
    torch.cuda.synchronize()
    words = _plan_words(plan)
    assert words[12] == 0, "no row may be split"
    assert words[4 + 3] == p.num_rows, "every row is a long row"
    want = expected(orc, p)
    for use_plan in (True, False):
        got, ok = gpu_run.run(p, d, use_plan=use_plan)
        assert ok
        assert_rows_equal(canonical(got, p.seq_lens, p.k), want, f"{p.name} plan={use_plan}")


@pytest.mark.parametrize("L", list(workloads.SUSTAINED_LENGTHS) + ["split256"])
def test_sustained_launch_sampled_rows(orc, L):
    """The launches the benchmark times for its sustained figures (about
    1 GiB of scores at each window length from 8192 to 131072: every CU
    serves several rounds of rows, and the waves of a workgroup drift
    furthest apart), and the largest split batch (256 long rows, 4096
    segments), three times with the plan; 40 sampled rows against the oracle
    after each."""
    import torch

    import row_top_selection_amd as dt

    if L == "split256":
        name, p = "paged_long_x256", workloads.scaled_long(256)
    else:
        name, p = workloads.sustained_name(L), workloads.sustained(L)
    n = p.num_rows
    print(f"[gpu] {name} sustained launch", flush=True)
    d = gpu_run.to_dev(p)
    rows = np.unique(np.concatenate([np.arange(4), np.linspace(0, p.num_rows - 1, 36)
                                     .astype(np.int64)]))
    want = orc.paged(p.scores[rows], p.seq_lens[rows], None, p.page_table[rows], p.page_size,
                     p.k)
    plan = dt.plan(d["lens"], p.k)
    idx = torch.from_numpy(rows).to(d["scores"].device)
    for it in range(3):
        out = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, plan=plan)
        got = out[idx].cpu().numpy()
        assert_rows_equal(canonical(got, p.seq_lens[rows], p.k), want, f"{name} run {it}")
    words = _plan_words(plan)
    assert words[14] == 0, "a segment gave up waiting for its row"
    assert (words[12] == n) == (n <= SPLIT_CAP)


@pytest.mark.parametrize("k", [2048, 1000])
def test_streamed_ragged_rows_with_starts(orc, k):
    """A RAGGED launch of 640 rows: streamed rows with starts of every
    residue, every fifth row a register row. Streamed rows read the opening
    lines of the row 512 on (those rows' windows start anywhere, and some of
    them are not streamed); no plan, so every long row is streamed. 48
    sampled rows, half of them past row 512, against the oracle."""
    import torch

    import row_top_selection_amd as dt
    from workloads.configs import OUTSIDE_SCORE, Problem

    rng = np.random.default_rng(20261202 + k)
    R, stride = 640, 131072 + 16
    starts = rng.integers(0, 16, size=R).astype(np.int32)
    lens = rng.integers(32769, 131072 - 15, size=R).astype(np.int32)
    lens[::5] = rng.integers(k + 1, 16384, size=len(lens[::5]))
    scores = np.full((R, stride), OUTSIDE_SCORE, dtype=np.float32)
    for b in range(R):
        scores[b, starts[b]:starts[b] + lens[b]] = rng.standard_normal(lens[b], dtype=np.float32)
    offs = rng.integers(0, 1 << 20, size=R).astype(np.int32)
    p = Problem(f"streamed_ragged_k{k}", "ragged", k, scores, lens, row_starts=starts,
                out_offsets=offs)
    print(f"[gpu] {p.name} rows={R}", flush=True)
    d = gpu_run.to_dev(p)
    rows = np.unique(np.concatenate([rng.choice(512, 24, replace=False),
                                     512 + rng.choice(R - 512, 24, replace=False)]))
    want = orc.ragged(scores[rows], lens[rows], starts[rows], offs[rows], k)
    out = dt.ragged(d["scores"], d["lens"], d["offs"], k, row_starts=d["starts"])
    got = out[torch.from_numpy(rows).to(out.device)].cpu().numpy()
    assert_rows_equal(canonical(got, lens[rows], k), want, p.name)


PACKED = [
    # (id, query rows per request, KV columns per request, k, largest window shift)
    ("mixed_classes", [5, 2, 9], 20000, 2048, 999),
    ("pages_layout", [3, 1, 4], 12000, 1000, 0),
    ("long_rows", [3, 2], 131072 - 1024, 2048, 1000),
]


def _check_raw_pairs(out, raw, p, table_rows, table_starts):
    """Slot for slot, out is raw mapped through the row's table row from
    its table start; padding is -1 in both."""
    k, ps = p.k, p.page_size
    n = np.minimum(np.maximum(p.seq_lens, 0), k)
    for b in range(p.num_rows):
        j = raw[b, :n[b]].astype(np.int64)
        q = j + (0 if table_starts is None else int(table_starts[b]))
        t = b if table_rows is None else int(table_rows[b])
        want = p.page_table[t, q // ps].astype(np.int64) * ps + q % ps
        assert np.array_equal(out[b, :n[b]], want), b
        assert (out[b, n[b]:] == -1).all() and (raw[b, n[b]:] == -1).all(), b


@pytest.mark.parametrize("use_plan", [False, True])
@pytest.mark.parametrize("case", PACKED, ids=[c[0] for c in PACKED])
def test_packed_paged_with_raw_positions(orc, case, use_plan):
    """Packed rows (several query rows share a request's table row; table
    starts shift the lookup) with the raw positions written in the same
    launch, against the oracle's packed emit and its selection."""
    import torch

    import row_top_selection_amd as dt

    cid, q_lens, kv, k, shift = case
    p, tr, ts = workloads.packed_paged(4000 + len(cid), q_lens, kv, k, shift)
    print(f"[gpu] packed {cid} rows={p.num_rows} plan={use_plan}", flush=True)
    d = gpu_run.to_dev(p)
    dev = d["scores"].device
    plan = dt.plan(d["lens"], k, row_starts=d["starts"]) if use_plan else None
    out, raw = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, k, row_starts=d["starts"],
                        plan=plan, table_rows=torch.from_numpy(tr).to(dev),
                        table_starts=torch.from_numpy(ts).to(dev), out_raw=True)
    torch.cuda.synchronize()
    out, raw = out.cpu().numpy(), raw.cpu().numpy()
    want = orc.paged_packed(p.scores, p.seq_lens, p.row_starts, p.page_table, p.page_size, k,
                            table_rows=tr, table_starts=ts)
    assert_rows_equal(canonical(out, p.seq_lens, k), want, cid)
    sel = orc.select(p.scores, p.seq_lens, p.row_starts, k)
    assert_rows_equal(canonical(raw, p.seq_lens, k), sel, cid + " raw")
    _check_raw_pairs(out, raw, p, tr, ts)


@pytest.mark.parametrize("name", ["paged_small", "paged_decode", "paged_long", "paged_mixed"])
def test_raw_positions_beside_paged(orc, name):
    """The raw-position output on the plain PAGED workloads (with a plan):
    the same selection, slot for slot with the paged values."""
    import torch

    import row_top_selection_amd as dt

    p = workloads.make_workload(name)
    print(f"[gpu] raw {name}", flush=True)
    d = gpu_run.to_dev(p)
    plan = dt.plan(d["lens"], p.k, row_starts=d["starts"])
    out, raw = dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, p.k, row_starts=d["starts"],
                        plan=plan, out_raw=True)
    torch.cuda.synchronize()
    out, raw = out.cpu().numpy(), raw.cpu().numpy()
    assert_rows_equal(canonical(out, p.seq_lens, p.k), expected(orc, p), name)
    sel = orc.select(p.scores, p.seq_lens, p.row_starts, p.k)
    assert_rows_equal(canonical(raw, p.seq_lens, p.k), sel, name + " raw")
    _check_raw_pairs(out, raw, p, None, None)


def test_library_loaded_before_torch(orc, tmp_path):
    """A process that asks for the library before it imports torch: the
    binding loads torch's HIP runtime first, so the library binds to it and
    takes torch's streams (with the library loaded first, the process held a
    second HIP runtime that rejected them). A fresh interpreter, since the
    load order is per process."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    dst = tmp_path / "out.npy"
    code = "\n".join([
        "import sys",
        f"sys.path.insert(0, {root!r})",
        "import numpy as np",
        "import row_top_selection_amd as dt",
        "dt.lib()",
        "import torch",
        "import workloads",
        "p = workloads.make_workload('paged_small')",
        "dev = torch.device('cuda:0')",
        "out = dt.paged(torch.from_numpy(p.scores).to(dev), torch.from_numpy(p.seq_lens).to(dev),",
        "               torch.from_numpy(p.page_table).to(dev), p.page_size, p.k)",
        f"np.save({str(dst)!r}, out.cpu().numpy())",
    ])
    print("[gpu] library loaded before torch (subprocess)", flush=True)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=110)
    assert res.returncode == 0, res.stderr[-2000:]
    p = workloads.make_workload("paged_small")
    assert_rows_equal(canonical(np.load(dst), p.seq_lens, p.k), expected(orc, p), p.name)
