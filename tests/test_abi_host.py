"""C ABI checks that need no GPU: exports, status strings, host-side
argument validation (which returns before anything is launched)."""
import ctypes
import re
from pathlib import Path

import pytest

import row_top_selection_amd as dt

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "dsatopk.h"

# Fake device addresses: the validation under test returns before any HIP
# call, so these are never dereferenced.
A16 = 0x10000
A4 = 0x10004


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsatopk_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return dt.lib()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(dt.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(6):
        assert lib.dsatopk_status_string(code)
    assert lib.dsatopk_status_string(99) == b"unknown status"


def test_plan_bytes(lib):
    assert lib.dsatopk_plan_bytes(-1) == 0
    assert lib.dsatopk_plan_bytes(0) > 0
    assert lib.dsatopk_plan_bytes(100) >= lib.dsatopk_plan_bytes(10)


def paged(lib, **kw):
    a = dict(scores=A16, stride=64, lens=A16, starts=None, pt=A16, pts=8, ps=64, rows=4, k=16,
             plan=None, plan_bytes=0, out=A16, stream=None)
    a.update(kw)
    return lib.dsatopk_paged(a["scores"], a["stride"], a["lens"], a["starts"], a["pt"], a["pts"],
                             a["ps"], a["rows"], a["k"], a["plan"], a["plan_bytes"], a["out"],
                             a["stream"])


def paged_packed(lib, **kw):
    a = dict(scores=A16, stride=64, lens=A16, starts=None, pt=A16, pts=8, ps=64, rows=A16,
             tstarts=None, n=4, k=16, plan=None, plan_bytes=0, out=A16, raw=A16, stream=None)
    a.update(kw)
    return lib.dsatopk_paged_packed(a["scores"], a["stride"], a["lens"], a["starts"], a["pt"],
                                    a["pts"], a["ps"], a["rows"], a["tstarts"], a["n"], a["k"],
                                    a["plan"], a["plan_bytes"], a["out"], a["raw"], a["stream"])


def ragged(lib, **kw):
    a = dict(scores=A16, stride=64, lens=A16, starts=None, offs=A16, rows=4, k=16, plan=None,
             plan_bytes=0, out=A16, stream=None)
    a.update(kw)
    return lib.dsatopk_ragged(a["scores"], a["stride"], a["lens"], a["starts"], a["offs"],
                              a["rows"], a["k"], a["plan"], a["plan_bytes"], a["out"],
                              a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 1), (dict(k=2049), 1), (dict(k=-3), 1), (dict(rows=-1), 1),
    (dict(scores=None), 1), (dict(lens=None), 1), (dict(out=None), 1), (dict(stride=0), 1),
    (dict(pt=None), 1), (dict(pts=0), 1), (dict(ps=0), 1), (dict(ps=48), 1),
    (dict(ps=1 << 21), 1), (dict(scores=A4), 2), (dict(stride=66), 2),
    (dict(plan=A16, plan_bytes=1), 3), (dict(plan=A4, plan_bytes=1 << 30), 2),
])
def test_paged_rejects(lib, kw, code):
    assert paged(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 1), (dict(n=-1), 1), (dict(scores=None), 1), (dict(pt=None), 1),
    (dict(ps=48), 1), (dict(scores=A4), 2), (dict(plan=A16, plan_bytes=1), 3),
])
def test_paged_packed_rejects(lib, kw, code):
    assert paged_packed(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), 1), (dict(k=4096), 1), (dict(offs=None), 1), (dict(scores=A4 + 8), 2),
    (dict(stride=6), 2), (dict(plan=A16, plan_bytes=8), 3),
])
def test_ragged_rejects(lib, kw, code):
    assert ragged(lib, **kw) == code


def test_zero_rows_is_a_noop(lib):
    # nothing is launched and no pointer is looked at
    assert paged(lib, rows=0, scores=None, lens=None, out=None, pt=None) == 0
    assert ragged(lib, rows=0, scores=None, lens=None, out=None, offs=None) == 0
    assert paged_packed(lib, n=0, scores=None, lens=None, out=None, pt=None, raw=None) == 0
    assert lib.dsatopk_plan(None, None, 0, 16, None, 0, None) == 0


def test_plan_rejects(lib):
    assert lib.dsatopk_plan(A16, None, -1, 16, A16, 1 << 20, None) == 1
    assert lib.dsatopk_plan(A16, None, 4, 0, A16, 1 << 20, None) == 1
    assert lib.dsatopk_plan(None, None, 4, 16, A16, 1 << 20, None) == 1
    assert lib.dsatopk_plan(A16, None, 4, 16, None, 1 << 20, None) == 1
    assert lib.dsatopk_plan(A16, None, 4, 16, A16, 8, None) == 3
    assert lib.dsatopk_plan(A16, None, 4, 16, A4, 1 << 20, None) == 2


def test_binding_has_no_cpu_fallback(monkeypatch, tmp_path):
    """Without the built library every call raises instead of computing."""
    monkeypatch.setattr(dt, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(dt, "_handle", None)
    with pytest.raises(ImportError):
        dt.plan_bytes(4)


def test_library_has_no_oracle_dependency():
    """The GPU library's sources name nothing of the oracle."""
    for src in (ROOT / "row_top_selection_amd").rglob("*"):
        if src.suffix in (".py", ".hip", ".h", ".cpp"):
            text = src.read_text()
            assert "oracle" not in text.lower(), src


def test_noalloc_rejects_batches_above_its_scratch(lib):
    """dsatopk_paged_noalloc refuses a batch whose plan would not fit its
    static scratch, before any HIP call (fake pointers, no GPU needed)."""
    n = dt.NOALLOC_MAX_ROWS + 1
    st = lib.dsatopk_paged_noalloc(A16, 64, A16, None, A16, 8, 64, n, 16, A16, None)
    assert st == 5
    assert b"NOALLOC_MAX_ROWS" in lib.dsatopk_status_string(5)
    # the usual argument checks come before any HIP call too
    assert lib.dsatopk_paged_noalloc(A16, 64, A16, None, None, 8, 64, 4, 16, A16, None) == 1
    assert lib.dsatopk_paged_noalloc(A4, 64, A16, None, A16, 8, 64, 4, 16, A16, None) == 2
    assert lib.dsatopk_paged_noalloc(None, 64, None, None, None, 8, 64, 0, 16, None, None) == 0
