"""Input generators: the structure the GPU parity batches rely on (CPU)."""
import numpy as np

from workloads.edge import edge_batch


def _keys(v):
    """Order-preserving 32-bit keys of float32 values (sign-magnitude flip),
    written out here from the float format for this check."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    neg = (u >> np.uint64(31)) == 1
    return np.where(neg, ~u & np.uint64(0xffffffff), u + np.uint64(0x7fffffff))


def test_dense_rows_fill_one_coarse_bin_across_its_fine_bins():
    """The dense pattern puts every key of a row in one bin of the top 12
    key bits and spreads them over its four bins of the top 14 bits (the
    decode rows' fallback from the 14-bit to the 12-bit digit)."""
    p = edge_batch(11, "ragged", 100, [(3000, 0, "dense"), (8000, 2, "dense")], stride=8192)
    for b in range(p.num_rows):
        s = int(p.row_starts[b])
        k = _keys(p.scores[b, s:s + int(p.seq_lens[b])])
        assert len(np.unique(k >> np.uint64(20))) == 1
        assert len(np.unique(k >> np.uint64(18))) == 4


def test_edge_batch_windows_and_sentinel():
    """Windows fit the stride; every column outside a window holds the 1e3
    sentinel, which a read outside the window would select."""
    rows = [(L, r, "normal") for r in range(4) for L in (-3, 0, 5, 4093)]
    p = edge_batch(12, "paged", 7, rows, stride=4096)
    assert p.stride == 4096
    for b in range(p.num_rows):
        s, L = int(p.row_starts[b]), max(int(p.seq_lens[b]), 0)
        assert s % 4 == rows[b][1] and s + L <= p.stride
        out = np.ones(p.stride, dtype=bool)
        out[s:s + L] = False
        assert (p.scores[b, out] == np.float32(1e3)).all()
        assert (p.scores[b, ~out] < 1e3).all()
