"""Benchmark of the dsatopk hot path on one GPU; prints one JSON line.

Step: one pass of the whole path over one batch: dsatopk_plan followed by
dsatopk_paged on the ``paged_decode`` workload (128 rows x 8192 fp32 scores,
k = 2048, page size 64, random page tables). Inputs are resident in HBM;
every step reads a different copy of the scores from a rotation of at least
1 GiB so that score reads miss the 256 MB Infinity Cache. The W warmup and K
timed steps are each captured once into a HIP graph and replayed, the way a
serving loop issues them; the same steps issued call by call from Python are
reported beside it ("eager"), where host launch overhead dominates.

Also reported (same JSON line):
  roofline      the paged transform kernel (rows_wide_kernel<true>: 128 short
                rows, 512 threads per row): algorithmic bytes per launch
                (scores of rows with L > k, outputs, page-table entries,
                lengths) over its mean launch time from HIP events around a
                graph of back-to-back launches.
  sustained     the same per-row shapes with enough rows for >= 1 GiB of
                scores per launch (L = 8192 ... 131072), timed in steady
                state: after 0.1 s of untimed replays (the GPU's clocks ramp
                up over the first ~10 ms of continuous work), the mean of 5
                replays of 20 launches. Each carries "mover": the same
                launch of bench_mover.hip, which reads the same windows and
                writes the same k outputs per row with no selection, timed
                the same way (what HBM allows for these bytes in this
                launch shape; absent when bench_mover.so is not built).
  workloads     every named workload, one launch per iteration, cold, after
                the same 0.1 s of untimed replays.
  cpu_baseline  the oracle on this host's cores over a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA top-k rows/s + achieved HBM GB/s (paged decode, L=8K–128K, k=2048)"
HBM_PEAK_GBPS = 8000.0
ROTATION_BYTES = 1 << 30
SETTLE_S = 0.1  # untimed replays before a sustained measurement
COPY_CALIBRATION_BYTES = 256 << 20
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_rows_wide_kernel_paged_decode.md")


def kernel_source_hash() -> str:
    """Hash of the HIP sources: counter figures taken from an older build of
    the kernels no longer describe them."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_top_selection_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


MOVER_SRC = os.path.join(ROOT, "bench_mover.hip")
MOVER_SO = os.path.join(ROOT, "bench_mover.so")


def build_mover(verbose: bool = False) -> str:
    """Compile bench_mover.hip (the same-bytes mover) for gfx950 beside it."""
    import subprocess

    from row_top_selection_amd import build as hip_build

    tmp = MOVER_SO + ".tmp%d" % os.getpid()
    cmd = [hip_build.HIPCC, "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", MOVER_SRC,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, MOVER_SO)
    return MOVER_SO


_mover = None


def mover_lib():
    """The built same-bytes mover, or None when bench_mover.so is absent."""
    global _mover
    if _mover is None and os.path.exists(MOVER_SO):
        import ctypes

        import torch  # noqa: F401  (its HIP runtime first, as the library binding does)

        lib = ctypes.CDLL(MOVER_SO)
        lib.bench_mover.restype = ctypes.c_int
        lib.bench_mover.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p]
        _mover = lib
    return _mover


def measured_traffic():
    """HBM bytes per launch of the paged transform kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernels."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    try:
        d = json.loads(text[start + 7:end])
    except ValueError:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def algorithmic_bytes(p) -> dict:
    """Bytes one launch must move: scores of rows with L > k, the k int32
    outputs of every row, the page-table entries of selected rows' windows,
    and the per-row metadata (length, start, offset)."""
    L = p.window_lengths()
    score = int(4 * L[L > p.k].sum())
    out = 4 * p.k * p.num_rows
    table = 0
    if p.mode == "paged":
        table = int(4 * np.ceil(L / p.page_size).sum())
    meta = 4 * p.num_rows * (1 + (p.row_starts is not None) + (p.mode == "ragged"))
    return {"score": score, "out": out, "table": table, "meta": meta,
            "total": score + out + table + meta}


class Runner:
    """Device copies of one workload and a rotation of its score rows."""

    def __init__(self, p, rotate: bool = True, table_rows=None, table_starts=None,
                 raw: bool = False):
        import torch

        self.p = p
        dev = torch.device("cuda")
        # packed PAGED rows and the raw-position output (dsatopk_paged_packed)
        self.table_rows = None if table_rows is None else torch.from_numpy(table_rows).to(dev)
        self.table_starts = None if table_starts is None else \
            torch.from_numpy(table_starts).to(dev)
        self.out_raw = torch.empty((p.num_rows, p.k), dtype=torch.int32, device=dev) \
            if raw else None
        self.scores0 = torch.from_numpy(p.scores).to(dev)
        nbytes = p.scores.nbytes
        self.copies = max(1, -(-ROTATION_BYTES // nbytes)) if rotate else 1
        if self.copies > 1:
            self.rot = torch.empty((self.copies,) + tuple(p.scores.shape), dtype=torch.float32,
                                   device=dev)
            self.rot[:] = self.scores0
        else:
            self.rot = self.scores0[None]
        self.lens = torch.from_numpy(p.seq_lens).to(dev)
        self.starts = None if p.row_starts is None else torch.from_numpy(p.row_starts).to(dev)
        if p.mode == "ragged":
            self.offs = torch.from_numpy(p.out_offsets).to(dev)
        else:
            self.pt = torch.from_numpy(p.page_table).to(dev)
        self.out = torch.empty((p.num_rows, p.k), dtype=torch.int32, device=dev)
        import row_top_selection_amd as dt

        self.dt = dt
        self.plan = dt.plan(self.lens, p.k, row_starts=self.starts)

    def make_plan(self):
        self.dt.plan(self.lens, self.p.k, row_starts=self.starts, out=self.plan)

    def transform(self, i: int):
        p, dt = self.p, self.dt
        s = self.rot[i % self.copies]
        if p.mode == "ragged":
            dt.ragged(s, self.lens, self.offs, p.k, row_starts=self.starts, plan=self.plan,
                      out=self.out)
        else:
            dt.paged(s, self.lens, self.pt, p.page_size, p.k, row_starts=self.starts,
                     plan=self.plan, out=self.out, table_rows=self.table_rows,
                     table_starts=self.table_starts, out_raw=self.out_raw)

    def step(self, i: int):
        self.make_plan()
        self.transform(i)

    def move(self, i: int):
        """The same-bytes mover on copy i's scores (bench_mover.hip): the
        window reads of rows with L > k and k int32 outputs per row."""
        import torch

        s = self.rot[i % self.copies]
        starts = None if self.starts is None else self.starts.data_ptr()
        rc = mover_lib().bench_mover(s.data_ptr(), s.stride(0), self.lens.data_ptr(), starts,
                                     self.p.num_rows, self.p.k, self.out.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"bench_mover failed ({rc})")

    def free(self):
        del self.rot, self.scores0


def time_steps(fn, steps: int, warmup: int) -> float:
    """Seconds for `steps` calls of fn(i), bracketed by device syncs."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def capture_steps(fn, start: int, n: int):
    """A HIP graph of n consecutive steps fn(start), fn(start + 1), ... (the
    library's calls only launch kernels, so they capture as they are)."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(start + i)
    return g


def time_graph_steps(fn, steps: int, warmup: int) -> float:
    """Seconds for `steps` steps replayed from one captured graph, after a
    replay of `warmup` untimed steps; device syncs on both sides."""
    import torch

    gw = capture_steps(fn, 0, warmup) if warmup > 0 else None
    gk = capture_steps(fn, warmup, steps)
    if gw is not None:
        gw.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gk.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def kernel_time_us(fn, iters: int, warmup: int = 3, settle_s: float = 0.0,
                   reps: int = 1) -> float:
    """Mean duration of fn(i)'s launches: `iters` calls captured back to back
    in one HIP graph, replayed `reps` times between two HIP events recorded on
    the stream the graph runs on (torch's current stream), divided by
    iters * reps. The graph keeps host launch overhead out of short launches.
    With settle_s, untimed replays run for that long first: the GPU raises
    its clocks over the first ~10 ms of continuous work (the first replay
    after an idle spell runs about a tenth slower), so a steady rate is only
    seen after it."""
    import torch

    for i in range(warmup):
        fn(i)
    g = capture_steps(fn, warmup, iters)
    g.replay()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (iters * reps)


def cpu_baseline(p, budget_s: float = 12.0) -> dict:
    """The oracle, as it is, on this host's cores: repeated passes over the
    paged_decode batch until about `budget_s` of work."""
    import oracle

    orc = oracle.default()
    threads = oracle.default_threads()
    done = 0
    t0 = time.perf_counter()
    while True:
        orc.paged(p.scores, p.seq_lens, p.row_starts, p.page_table, p.page_size, p.k,
                  threads=threads)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {
        "value": done * p.num_rows / el,
        "unit": "rows/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} passes of the oracle over the full {p.num_rows}-row paged_decode "
                  f"batch ({el:.1f} s, {threads} threads)",
        "score_GBps": done * algorithmic_bytes(p)["score"] / el / 1e9,
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_configs() -> dict:
    """The oracle on every workload: one pass over the full batch with all
    host threads, and one thread over the batch's first rows (at most 32)."""
    import oracle

    orc = oracle.default()
    threads = oracle.default_threads()
    res = {"cpu": cpu_model(), "threads": threads}
    for name in workloads_names():
        p = only_workload(name)

        def run(sub, nthreads):
            t0 = time.perf_counter()
            if p.mode == "ragged":
                orc.ragged(p.scores[sub], p.seq_lens[sub],
                           None if p.row_starts is None else p.row_starts[sub],
                           p.out_offsets[sub], p.k, threads=nthreads)
            else:
                orc.paged(p.scores[sub], p.seq_lens[sub],
                          None if p.row_starts is None else p.row_starts[sub],
                          p.page_table[sub], p.page_size, p.k, threads=nthreads)
            return time.perf_counter() - t0

        full = slice(0, p.num_rows)
        head = slice(0, min(p.num_rows, 32))
        tf = run(full, threads)
        t1 = run(head, 1)
        L = p.window_lengths()
        score_head = int(4 * L[head][L[head] > p.k].sum())
        res[name] = {"rows": p.num_rows, "wall_s": tf, "rows_per_s": p.num_rows / tf,
                     "score_GBps": algorithmic_bytes(p)["score"] / tf / 1e9,
                     "one_thread": {"rows": head.stop, "wall_s": t1, "rows_per_s": head.stop / t1,
                                    "score_GBps": score_head / t1 / 1e9}}
    return res


def workloads_names():
    import workloads

    return list(workloads.WORKLOADS)


def describe(p) -> dict:
    L = p.window_lengths()
    return {"rows": p.num_rows, "k": p.k, "mode": p.mode,
            "seq_len": int(L[0]) if (L == L[0]).all() else [int(L.min()), int(L.max())]}


def sustained_makers():
    import workloads

    return {workloads.sustained_name(L): (lambda L=L: workloads.sustained(L))
            for L in workloads.SUSTAINED_LENGTHS}


def only_workload(name: str):
    import workloads

    sus = sustained_makers()
    if name in sus:
        return sus[name]()
    if name == "all_trivial":
        return workloads.all_trivial()
    return workloads.make_workload(name)


def measure_workload(p, iters: int, settle_s: float = SETTLE_S, reps: int = 1,
                     mover: bool = False, **packed) -> dict:
    r = Runner(p, **packed)
    us = kernel_time_us(r.transform, iters, settle_s=settle_s, reps=reps)
    b = algorithmic_bytes(p)
    if packed.get("raw"):
        b = dict(b, raw=b["out"], total=b["total"] + b["out"])
    res = dict(describe(p), transform_us=us, rows_per_s=p.num_rows / (us * 1e-6),
               score_GBps=b["score"] / (us * 1e3), total_GBps=b["total"] / (us * 1e3),
               hbm_frac=b["total"] / (us * 1e3) / HBM_PEAK_GBPS, bytes=b, rotation=r.copies)
    if mover and mover_lib() is not None and not packed:
        # the same reads and writes with no selection, timed the same way
        mus = kernel_time_us(r.move, iters, settle_s=settle_s, reps=reps)
        res["mover"] = {"us": mus, "score_frac": b["score"] / (mus * 1e3) / HBM_PEAK_GBPS,
                        "transform_over_mover": us / mus}
    r.free()
    return res


def measure_sustained() -> dict:
    import torch

    sus = {}
    for name, mk in sustained_makers().items():
        # steady state: 0.1 s of untimed replays, then 5 x 20 launches
        res = measure_workload(mk(), 20, reps=5, mover=True)
        res["score_frac"] = res["score_GBps"] / HBM_PEAK_GBPS
        res["timing"] = f"mean of 5 replays of 20 launches after {SETTLE_S} s of replays"
        sus[name] = res
        torch.cuda.empty_cache()
    return sus


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline step and roofline only")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 256 MiB (counter calibration)")
    ap.add_argument("--only", default=None,
                    help="only replay one workload's transform --steps times (counter runs): "
                         "a workload name, a sustained name, or all_trivial")
    ap.add_argument("--sustained-only", action="store_true",
                    help="only the sustained launches (and their mover), as one JSON line")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the selection shards by rows with no exchange, "
              "and multi-GPU runs are not part of this build (use --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_CALIBRATION_BYTES, "launches": 5}), flush=True)
        return 0
    if args.sustained_only:
        print(json.dumps({"sustained": measure_sustained(),
                          "kernel_source_hash": kernel_source_hash()}), flush=True)
        return 0
    if args.only:
        p = only_workload(args.only)
        r = Runner(p)
        for i in range(args.steps):
            r.transform(i)
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.only, "launches": args.steps,
                          "bytes_per_launch": algorithmic_bytes(p)}), flush=True)
        return 0
    p = workloads.make_workload("paged_decode")
    r = Runner(p)
    eager_secs = time_steps(r.step, args.steps, args.warmup)
    secs = time_graph_steps(r.step, args.steps, args.warmup)
    ms = 1e3 * secs / args.steps
    b = algorithmic_bytes(p)
    k_us = kernel_time_us(r.transform, max(args.steps, 50))
    plan_us = kernel_time_us(lambda i: r.make_plan(), 50)
    mover_us = kernel_time_us(r.move, max(args.steps, 50)) if mover_lib() is not None else None
    achieved = b["total"] / (k_us * 1e3)
    line = {
        "metric": METRIC,
        "value": p.num_rows * args.steps / secs,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "paged_decode: PAGED, 128 rows x 8192 fp32 N(0,1) scores, k=2048, "
                               "page_size=64, random page tables; step = plan + paged transform "
                               "on its own cold copy of the scores; the timed steps replay from "
                               "one captured HIP graph",
                   **describe(p), "page_size": p.page_size,
                   "cold_rotation_copies": r.copies},
        "score_GBps_step": b["score"] * args.steps / secs / 1e9,
        "eager": {"ms_per_step": 1e3 * eager_secs / args.steps,
                  "rows_per_s": p.num_rows * args.steps / eager_secs,
                  "note": "same steps issued call by call from Python (host-bound)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(),
                     "kernel": "dsatopk::rows_wide_kernel<true>", "kernel_us": k_us,
                     "kernel_source_hash": kernel_source_hash(),
                     "bytes_per_launch": b, "score_GBps": b["score"] / (k_us * 1e3),
                     "plan_us": plan_us, "mover_us": mover_us},
    }
    r.free()
    del r
    torch.cuda.empty_cache()
    if not args.quick:
        # paged decode rows from 8192 to 131072 columns, 1 GiB of scores per
        # launch (the decode and long-context shapes, and three between)
        line["sustained"] = measure_sustained()
        wl = {}
        for name in workloads.WORKLOADS:
            wl[name] = measure_workload(workloads.make_workload(name), 50, mover=True)
            torch.cuda.empty_cache()
        line["workloads"] = wl
        # the packed PAGED layout (4 requests x 1024 query rows sharing their
        # tables, windows from each request's first column) and the raw
        # positions written beside the paged ones
        pk, tr, ts = workloads.packed_paged(workloads.BASE_SEED + 111, [1024] * 4, 16385,
                                            2048, 0)
        line["packed"] = {
            "packed_extend": measure_workload(pk, 20, table_rows=tr, table_starts=ts, raw=True),
            "paged_decode_x32768_raw": measure_workload(workloads.scaled_decode(32768), 20,
                                                        reps=5, raw=True),
        }
        torch.cuda.empty_cache()
    line["cpu_baseline"] = cpu_baseline(p, args.cpu_budget)
    if not args.quick:
        line["cpu_configs"] = cpu_configs()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
