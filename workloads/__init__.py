"""Seeded synthetic inputs for the windowed top-k selection.

This package holds input generation only: no selection, keying or emit
arithmetic. Both the oracle-side tests and the GPU-side tests and benchmark
draw their inputs from here, so the same seed gives the same bytes to both.

The five workload shapes stand in for DeepSeek-V4 indexer score rows, which
the pages describe as produced by the DeepGEMM indexer (sglang PR #35175
digest, "Motivation"): fp32 scores with N(0,1) values, page size 64, runtime
k. The shapes are the workload names below:

- ``paged_small``   4 rows, L ~ U{1..3000}, k=512, scores [4, 3000]
- ``paged_decode``  128 rows, L = 8192, k=2048, scores [128, 8192]
- ``ragged_extend`` 4 requests x 1024 query rows over a flattened KV of
  4 request slots of 16385 columns; row_start = out_offset = slot base,
  L = 15361 + i, k=2048; 1e3 outside each row's window
- ``paged_long``    8 rows, L = 131072, k=2048, N(0,1) rounded to fp16
- ``paged_mixed``   512 rows, log-uniform L in [1, 131072] with 7 pinned
  lengths, k=1024, scores [512, 131072]

Every generator uses ``numpy.random.default_rng(seed)`` and draws in the
fixed order seq_lens, scores, page tables, pinned rows.
"""
from .configs import (  # noqa: F401
    all_trivial,
    BASE_SEED,
    WORKLOADS,
    Problem,
    make_workload,
    packed_paged,
    scaled_decode,
    scaled_long,
    scaled_paged,
    short_mix,
    random_page_tables,
    SUSTAINED_LENGTHS,
    sustained,
    sustained_name,
    sustained_rows,
)
