"""Python binding of ``libdsatopk.so`` (the C ABI in ``include/dsatopk.h``).

Argument marshalling only: every step of the selection runs in the HIP
kernels of the library. Tensors are torch CUDA (HIP) tensors; torch is used
for device memory and the current stream. If the library has not been
built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libdsatopk.so"

MAX_K = 2048
MAX_SEQ_LEN = 131072

STATUS = {
    0: "DSATOPK_OK",
    1: "DSATOPK_ERR_INVALID_ARG",
    2: "DSATOPK_ERR_ALIGNMENT",
    3: "DSATOPK_ERR_PLAN_TOO_SMALL",
    4: "DSATOPK_ERR_HIP",
    5: "DSATOPK_ERR_TOO_LARGE",
}

NOALLOC_MAX_ROWS = 262144

EXPORTS = ("dsatopk_status_string", "dsatopk_plan_bytes", "dsatopk_plan", "dsatopk_plan_error",
           "dsatopk_paged", "dsatopk_paged_packed", "dsatopk_ragged", "dsatopk_paged_noalloc")


class DsatopkError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_lib().dsatopk_status_string(status).decode()})")


_handle = None


def _lib():
    """The loaded library with argument types set (raises if not built)."""
    global _handle
    if _handle is None:
        if not LIB_PATH.exists():
            raise ImportError(f"{LIB_PATH} is not built: run row_top_selection_amd.build.build()")
        # torch's HIP runtime first: it carries the soname this library
        # links against, so the library binds to it. Loaded the other way
        # round, the process would hold a second HIP runtime, which knows
        # none of torch's streams.
        import torch  # noqa: F401

        lib = ctypes.CDLL(str(LIB_PATH))
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.dsatopk_status_string.argtypes = [ctypes.c_int]
        lib.dsatopk_status_string.restype = ctypes.c_char_p
        lib.dsatopk_plan_bytes.argtypes = [i32]
        lib.dsatopk_plan_bytes.restype = sz
        lib.dsatopk_plan.argtypes = [P, P, i32, i32, P, sz, P]
        lib.dsatopk_plan.restype = ctypes.c_int
        lib.dsatopk_plan_error.argtypes = [P, sz, P, P]
        lib.dsatopk_plan_error.restype = ctypes.c_int
        lib.dsatopk_paged.argtypes = [P, i64, P, P, P, i64, i32, i32, i32, P, sz, P, P]
        lib.dsatopk_paged.restype = ctypes.c_int
        lib.dsatopk_paged_packed.argtypes = [P, i64, P, P, P, i64, i32, P, P, i32, i32, P, sz,
                                             P, P, P]
        lib.dsatopk_paged_packed.restype = ctypes.c_int
        lib.dsatopk_ragged.argtypes = [P, i64, P, P, P, i32, i32, P, sz, P, P]
        lib.dsatopk_ragged.restype = ctypes.c_int
        lib.dsatopk_paged_noalloc.argtypes = [P, i64, P, P, P, i64, i32, i32, i32, P, P]
        lib.dsatopk_paged_noalloc.restype = ctypes.c_int
        _handle = lib
    return _handle


def lib():
    """Raw ctypes handle of libdsatopk.so."""
    return _lib()


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _on(t, like, name):
    """t must be a device tensor on like's device."""
    if not t.is_cuda or t.device != like.device:
        raise ValueError(f"{name} must be a device tensor on {like.device}")
    return t


def _vec_i32(t, n, name, like=None):
    import torch

    if t is None:
        return None
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 vector of length {n}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if like is not None:
        _on(t, like, name)
    return t


def _scores(scores):
    import torch

    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be a 2-D float32 tensor with contiguous columns")
    if not scores.is_cuda:
        raise ValueError("scores must be a device tensor")
    return scores


def _out(out, rows, k, like, name="out"):
    import torch

    if out is None:
        return torch.empty((rows, k), dtype=torch.int32, device=like.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, k) or not out.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape ({rows}, {k})")
    return _on(out, like, name)


def _plan_arg(plan, like):
    """(pointer, bytes) of a plan tensor on like's device, or (None, 0)."""
    import torch

    if plan is None:
        return None, 0
    if plan.dtype != torch.uint8 or not plan.is_contiguous():
        raise ValueError("plan must be a contiguous uint8 tensor from plan()")
    _on(plan, like, "plan")
    return plan.data_ptr(), plan.numel()


def plan_bytes(num_rows: int) -> int:
    return int(_lib().dsatopk_plan_bytes(int(num_rows)))


def plan(seq_lens, k: int, row_starts=None, out=None, stream=None):
    """Build a plan (uint8 device tensor) from ``seq_lens`` / ``row_starts``."""
    import torch

    n = int(seq_lens.shape[0])
    _vec_i32(seq_lens, n, "seq_lens")
    _vec_i32(row_starts, n, "row_starts", seq_lens)
    nbytes = plan_bytes(n)
    if out is None:
        out = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=seq_lens.device)
    else:
        _plan_arg(out, seq_lens)
    st = _lib().dsatopk_plan(_ptr(seq_lens), _ptr(row_starts), n, int(k), _ptr(out), out.numel(),
                             _stream(stream))
    if st != 0:
        raise DsatopkError(st, "dsatopk_plan")
    return out


def plan_error(plan, stream=None) -> int:
    """The plan's error word (synchronizes the stream): 1 if a split row's
    wait gave up in a transform call since the plan was built, else 0."""
    err = ctypes.c_int32(0)
    st = _lib().dsatopk_plan_error(_ptr(plan), plan.numel(), ctypes.byref(err), _stream(stream))
    if st != 0:
        raise DsatopkError(st, "dsatopk_plan_error")
    return int(err.value)


def paged(scores, seq_lens, page_table, page_size: int, k: int, row_starts=None, plan=None,
          out=None, stream=None, table_rows=None, table_starts=None, out_raw=None):
    """PAGED top-k: int32 ``[rows, k]`` of page-table-mapped positions.

    Packed rows (``dsatopk_paged_packed``): ``table_rows`` picks each row's
    page-table row, ``table_starts`` its table position of window position
    0; ``out_raw`` (int32 ``[rows, k]``, or True to allocate one) also
    receives the window positions, slot for slot. Returns ``out``, or
    ``(out, out_raw)`` when ``out_raw`` is given."""
    import torch

    scores = _scores(scores)
    rows = int(scores.shape[0])
    _vec_i32(seq_lens, rows, "seq_lens", scores)
    _vec_i32(row_starts, rows, "row_starts", scores)
    _vec_i32(table_rows, rows, "table_rows", scores)
    _vec_i32(table_starts, rows, "table_starts", scores)
    packed = table_rows is not None or table_starts is not None or out_raw is not None
    if page_table.dtype != torch.int32:
        raise ValueError("page_table must be int32")
    if page_table.dim() != 2 or page_table.stride(1) != 1:
        raise ValueError("page_table must be [table rows, width] with contiguous columns")
    _on(page_table, scores, "page_table")
    if table_rows is None and page_table.shape[0] != rows:
        raise ValueError("page_table must have one row per score row without table_rows")
    out = _out(out, rows, int(k), scores)
    if out_raw is True:
        out_raw = _out(None, rows, int(k), scores, "out_raw")
    elif out_raw is not None:
        out_raw = _out(out_raw, rows, int(k), scores, "out_raw")
    plan_ptr, plan_n = _plan_arg(plan, scores)
    if not packed:
        st = _lib().dsatopk_paged(
            _ptr(scores), scores.stride(0), _ptr(seq_lens), _ptr(row_starts), _ptr(page_table),
            page_table.stride(0), int(page_size), rows, int(k), plan_ptr, plan_n, _ptr(out),
            _stream(stream))
        if st != 0:
            raise DsatopkError(st, "dsatopk_paged")
        return out
    st = _lib().dsatopk_paged_packed(
        _ptr(scores), scores.stride(0), _ptr(seq_lens), _ptr(row_starts), _ptr(page_table),
        page_table.stride(0), int(page_size), _ptr(table_rows), _ptr(table_starts), rows,
        int(k), plan_ptr, plan_n, _ptr(out), _ptr(out_raw), _stream(stream))
    if st != 0:
        raise DsatopkError(st, "dsatopk_paged_packed")
    return out if out_raw is None else (out, out_raw)


def ragged(scores, seq_lens, out_offsets, k: int, row_starts=None, plan=None, out=None,
           stream=None):
    """RAGGED top-k: int32 ``[rows, k]`` of position + out_offsets[row]."""
    scores = _scores(scores)
    rows = int(scores.shape[0])
    _vec_i32(seq_lens, rows, "seq_lens", scores)
    _vec_i32(row_starts, rows, "row_starts", scores)
    _vec_i32(out_offsets, rows, "out_offsets", scores)
    out = _out(out, rows, int(k), scores)
    plan_ptr, plan_n = _plan_arg(plan, scores)
    st = _lib().dsatopk_ragged(
        _ptr(scores), scores.stride(0), _ptr(seq_lens), _ptr(row_starts), _ptr(out_offsets),
        rows, int(k), plan_ptr, plan_n, _ptr(out), _stream(stream))
    if st != 0:
        raise DsatopkError(st, "dsatopk_ragged")
    return out


def paged_noalloc(scores, seq_lens, page_table, page_size: int, k: int, row_starts=None,
                  out=None, stream=None):
    """PAGED top-k through ``dsatopk_paged_noalloc`` (the plan lives in the
    library's static device memory; nothing is allocated except ``out`` when
    it is not given)."""
    import torch

    scores = _scores(scores)
    rows = int(scores.shape[0])
    _vec_i32(seq_lens, rows, "seq_lens", scores)
    _vec_i32(row_starts, rows, "row_starts", scores)
    if page_table.dtype != torch.int32:
        raise ValueError("page_table must be int32")
    if page_table.dim() != 2 or page_table.stride(1) != 1 or page_table.shape[0] != rows:
        raise ValueError("page_table must be [rows, width] with contiguous columns")
    _on(page_table, scores, "page_table")
    out = _out(out, rows, int(k), scores)
    st = _lib().dsatopk_paged_noalloc(
        _ptr(scores), scores.stride(0), _ptr(seq_lens), _ptr(row_starts), _ptr(page_table),
        page_table.stride(0), int(page_size), rows, int(k), _ptr(out), _stream(stream))
    if st != 0:
        raise DsatopkError(st, "dsatopk_paged_noalloc")
    return out
