"""Run a workload through the C ABI on the GPU (test helper)."""
from __future__ import annotations

import numpy as np

CANARY = -777


def to_dev(p):
    import torch

    dev = torch.device("cuda")
    d = {
        "scores": torch.from_numpy(p.scores).to(dev),
        "lens": torch.from_numpy(p.seq_lens).to(dev),
        "starts": None if p.row_starts is None else torch.from_numpy(p.row_starts).to(dev),
    }
    if p.mode == "ragged":
        d["offs"] = torch.from_numpy(p.out_offsets).to(dev)
    else:
        d["pt"] = torch.from_numpy(p.page_table).to(dev)
    return d


def run(p, d=None, use_plan=False, raw=False, canary=True):
    """Returns (out as numpy [rows, k], canary rows intact?). use_plan:
    False, True, or "stale" (a plan built for the lengths rolled by one row,
    so long rows meet segment counts that are not theirs)."""
    import torch

    import row_top_selection_amd as dt

    d = d or to_dev(p)
    R, k = p.num_rows, p.k
    big = torch.full((R + 2, k), CANARY, dtype=torch.int32, device=d["scores"].device)
    out = big[1:R + 1]
    plan = None
    if use_plan == "stale":
        plan = dt.plan(torch.roll(d["lens"], 1), k, row_starts=d["starts"])
    elif use_plan:
        plan = dt.plan(d["lens"], k, row_starts=d["starts"])
    if raw:
        zeros = torch.zeros(R, dtype=torch.int32, device=d["scores"].device)
        dt.ragged(d["scores"], d["lens"], zeros, k, row_starts=d["starts"], plan=plan, out=out)
    elif p.mode == "ragged":
        dt.ragged(d["scores"], d["lens"], d["offs"], k, row_starts=d["starts"], plan=plan, out=out)
    else:
        dt.paged(d["scores"], d["lens"], d["pt"], p.page_size, k, row_starts=d["starts"],
                 plan=plan, out=out)
    torch.cuda.synchronize()
    b = big.cpu().numpy()
    ok = bool((b[0] == CANARY).all() and (b[-1] == CANARY).all())
    return b[1:R + 1].copy(), ok


def scores_unchanged(p, d) -> bool:
    back = d["scores"].cpu().numpy()
    return np.array_equal(back.view(np.uint32), p.scores.view(np.uint32))
