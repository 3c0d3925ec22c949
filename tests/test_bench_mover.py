"""The benchmark's same-bytes mover (bench_mover.hip): the launch bench.py
times beside each sustained selection launch as what HBM allows for the
same reads and writes. These tests pin that it reads exactly each row's
window and writes all k outputs of every row, so that its time stands for
those bytes."""
import ctypes
import os

import numpy as np
import pytest

import bench

THREADS, UNROLL = 256, 8


@pytest.fixture(scope="module")
def mover():
    if not os.path.exists(bench.MOVER_SO):
        bench.build_mover()
    lib = bench.mover_lib()
    assert lib is not None
    return lib


def test_mover_rejects_bad_sizes_before_launching(mover):
    # these return before any HIP call: the pointers are never used
    a = ctypes.c_void_p(0x10000)
    assert mover.bench_mover(a, 8, a, None, -1, 4, a, None) == 1
    assert mover.bench_mover(a, 8, a, a, 2, 0, a, None) == 1
    assert mover.bench_mover(a, 10, a, None, 2, 4, a, None) == 1
    assert mover.bench_mover(a, -4, a, None, 2, 4, a, None) == 1
    assert mover.bench_mover(a, 8, a, a, 0, 4, a, None) == 0


def expected_outputs(scores: np.ndarray, lens: np.ndarray, starts, k: int) -> np.ndarray:
    """Each thread's fp32 sum of its float4 loads (from the aligned column at
    or below the window start), in the kernel's order, as the low 16 bits of
    its bits, plus the slot index."""
    rows, stride = scores.shape
    out = np.empty((rows, k), dtype=np.int64)
    zero4 = np.zeros(4, dtype=np.float32)
    for b in range(rows):
        s = 0 if starts is None else min(max(int(starts[b]), 0), stride)
        L = min(max(int(lens[b]), 0), stride - s)
        base = np.zeros(THREADS, dtype=np.int64)
        if L > k:
            a = s & ~3
            nv = (s + L - a + 3) // 4
            row = scores[b, a:]
            for t in range(THREADS):
                acc = np.float32(0)
                for v0 in range(0, nv, UNROLL * THREADS):
                    xs = []
                    for u in range(UNROLL):
                        v = v0 + u * THREADS + t
                        xs.append(row[4 * v:4 * v + 4] if v < nv else zero4)
                    for x in xs:
                        acc = np.float32(acc + np.float32(np.float32(x[0] + x[1]) +
                                                          np.float32(x[2] + x[3])))
                base[t] = int(acc.view(np.uint32)) & 0xFFFF
        i = np.arange(k)
        out[b] = base[i % THREADS] + i
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("with_starts", [False, True])
def test_mover_reads_each_window_and_writes_every_slot(mover, with_starts):
    import torch

    rng = np.random.default_rng(7)
    k, stride = 2048, 20000
    lens = np.array([0, 5, 2048, 2049, 8191, 20000, -3, 17001, 19999, 9000, 9001, 12345],
                    dtype=np.int32)
    starts = np.array([0, 3, 1, 2, 3, 0, 7, 2998, 1, 10999, 5, 7654], dtype=np.int32) \
        if with_starts else None
    scores = rng.standard_normal((len(lens), stride)).astype(np.float32)
    dev = torch.device("cuda:0")
    s = torch.from_numpy(scores).to(dev)
    ln = torch.from_numpy(lens).to(dev)
    st = None if starts is None else torch.from_numpy(starts).to(dev)
    out = torch.full((len(lens), k), -7, dtype=torch.int32, device=dev)
    rc = mover.bench_mover(s.data_ptr(), stride, ln.data_ptr(),
                           None if st is None else st.data_ptr(), len(lens), k, out.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64)
    want = expected_outputs(scores, lens, starts, k)
    assert np.array_equal(got, want)
