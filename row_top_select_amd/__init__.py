"""Python binding of the row_top_select C ABI (include/row_top_select.h).

Argument marshalling only: every step runs in the HIP kernels of
``librow_top_select.so``.  PyTorch provides device memory and the current
stream; tensors must live on the GPU.  Importing this package fails loudly if
the library has not been built (``python row_top_select_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librow_top_select.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python row_top_select_amd/build.py` "
        "(hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

RTS_OK, RTS_EINVAL, RTS_EUNSUPPORTED, RTS_EWORKSPACE, RTS_EHIP = 0, -1, -2, -3, -4
RTS_F32, RTS_BF16 = 0, 1

_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
_lib.rts_status_string.argtypes = [ctypes.c_int]
_lib.rts_status_string.restype = ctypes.c_char_p
_lib.topk_rows_workspace_size.argtypes = [ctypes.c_int, _i64, _i64, _i32]
_lib.topk_rows_workspace_size.restype = _sz
_lib.topk_rows.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i32, _p, _i64, _p, _sz, _p]
_lib.topk_rows_noalloc.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i32, _p, _i64, _p]
_lib.pack_candidates.argtypes = [_p, _i64, _i64, _i64, _p, _i32, _i64, _p, _p, _p]
_lib.merge_select_rank_major.argtypes = [_p, _i32, _i64, _i32, _i32, _p, _p, _p]
_lib.pack_pairs.argtypes = [_p, _i64, _i64, _i64, _p, _i32, _i64, _p, _i32, _i32, _p, _p]
_lib.merge_select_pairs_rank_major.argtypes = [_p, _i32, _i64, _i32, _i32, _p, _p]
_lib.merge_select_row_major.argtypes = [_p, _i32, _i64, _i32, _i32, _p, _p, _p]
_lib.merge_select_pairs_row_major.argtypes = [_p, _i32, _i64, _i32, _i32, _p, _p]
_lib.emit_rows.argtypes = [_p, _i64, _i32, _i32, _i32, _p, _p, _i64, _i32, _i64, _i32, _i64, _p, _i32,
                           _p, _p]
_lib.merge_select_rank_major_rows.argtypes = [_p, _i32, _i64, _i32, _i32, _p, _p, _p, _p]
_lib.merge_rescue_rank_major_rows.argtypes = [_p, _p, _i32, _i64, _i32, _i32, _p, _p, _p, _p]
_lib.rescue_push.argtypes = [_p, _i32, _i32, _i64, _i32, _i32, _p, _p, _p]
_lib.merge_rescue_rank_major.argtypes = [_p, _p, _i32, _i64, _i32, _i32, _p, _p, _p]
for _f in (_lib.topk_rows, _lib.topk_rows_noalloc, _lib.pack_candidates, _lib.merge_select_rank_major, _lib.pack_pairs,
           _lib.merge_select_pairs_rank_major, _lib.rescue_push, _lib.merge_rescue_rank_major,
           _lib.merge_select_row_major, _lib.merge_select_pairs_row_major, _lib.emit_rows,
           _lib.merge_select_rank_major_rows, _lib.merge_rescue_rank_major_rows):
    _f.restype = ctypes.c_int


class _KvRows(ctypes.Structure):
    """rts_kv_rows of include/row_top_select.h."""
    _fields_ = [("dcp_rank", ctypes.c_int32), ("req_id", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("table_rows", ctypes.c_int64),
                ("table_cols", ctypes.c_int32), ("ld_table", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("stride_rows", ctypes.c_int64),
                ("rows_out", ctypes.c_void_p), ("out_cols", ctypes.c_int32),
                ("valid_out", ctypes.c_void_p)]


class RtsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {rts_status_string(status)}")


def rts_status_string(status: int) -> str:
    return _lib.rts_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != RTS_OK:
        raise RtsError(status, where)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name):
    return None if t is None else _dev(t, name)


def _rows_ld(t: torch.Tensor, name: str):
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def _int32_vec(t, rows, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] < rows or (rows > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous int32 vector of >= {rows} entries")
    return t


def topk_rows_workspace_size(dtype, rows: int, cols: int, k: int) -> int:
    dt = RTS_BF16 if dtype in (torch.bfloat16, RTS_BF16) else RTS_F32
    return int(_lib.topk_rows_workspace_size(dt, rows, cols, k))


def topk_rows(logits: torch.Tensor, k: int, row_ends: torch.Tensor | None = None,
              out: torch.Tensor | None = None, workspace="auto", stream=None) -> torch.Tensor:
    """Exact per-row top-k column ids (score desc, id asc), -1 padded; see topk_rows in the header.

    ``out`` may be wider than k (columns past k are left untouched).  ``workspace``:
    "auto" (allocated here when the shape splits rows), None, or a uint8 GPU tensor.
    """
    if logits.dtype == torch.float32:
        dt = RTS_F32
    elif logits.dtype == torch.bfloat16:
        dt = RTS_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    rows, cols, ld = _rows_ld(logits, "logits")
    row_ends = _int32_vec(row_ends, rows, "row_ends")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    if out.dtype != torch.int32:
        raise TypeError("out must be int32")
    if out.device != logits.device:
        raise ValueError("out must be on the device of logits")
    out_rows, out_cols, ld_out = _rows_ld(out, "out")
    if out_rows < rows or out_cols < k:
        raise ValueError(f"out must hold at least [{rows}, {k}] (got {tuple(out.shape)})")
    if rows <= 1:
        ld_out = max(ld_out, k)
    ws, ws_bytes = None, 0
    if isinstance(workspace, str) and workspace == "auto":
        need = topk_rows_workspace_size(dt, rows, cols, k)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
            ws_bytes = need
    elif workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != logits.device or \
                not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the device of logits")
        ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    _check(_lib.topk_rows(_dev(logits, "logits"), dt, rows, cols, ld, _opt(row_ends, "row_ends"), k,
                          _dev(out, "out"), ld_out, _opt(ws, "workspace"), ws_bytes, _stream(stream)),
           "topk_rows")
    return out


def topk_rows_noalloc(logits: torch.Tensor, k: int, out: torch.Tensor,
                      row_ends: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """topk_rows into a caller-given ``out`` with no allocation at all (split rows use
    the library's static device scratch); see topk_rows_noalloc in the header."""
    if logits.dtype == torch.float32:
        dt = RTS_F32
    elif logits.dtype == torch.bfloat16:
        dt = RTS_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    rows, cols, ld = _rows_ld(logits, "logits")
    row_ends = _int32_vec(row_ends, rows, "row_ends")
    if out.dtype != torch.int32:
        raise TypeError("out must be int32")
    if out.device != logits.device:
        raise ValueError("out must be on the device of logits")
    out_rows, out_cols, ld_out = _rows_ld(out, "out")
    if out_rows < rows or out_cols < k:
        raise ValueError(f"out must hold at least [{rows}, {k}] (got {tuple(out.shape)})")
    if rows <= 1:
        ld_out = max(ld_out, k)
    _check(_lib.topk_rows_noalloc(_dev(logits, "logits"), dt, rows, cols, ld,
                                  _opt(row_ends, "row_ends"), k, _dev(out, "out"), ld_out,
                                  _stream(stream)), "topk_rows_noalloc")
    return out


def pack_candidates(logits_bf16: torch.Tensor, local_idx: torch.Tensor,
                    row_ends: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """B' packed rows int32 [rows, n + n/32] of a local top-n; see pack_candidates in the header."""
    if logits_bf16.dtype != torch.bfloat16:
        raise TypeError("logits must be bfloat16")
    rows, cols, ld = _rows_ld(logits_bf16, "logits")
    if local_idx.dtype != torch.int32:
        raise TypeError("local_idx must be int32")
    r2, n, ld_idx = _rows_ld(local_idx, "local_idx")
    if r2 != rows:
        raise ValueError("local_idx must have one row per logits row")
    if rows <= 1:
        ld_idx = max(ld_idx, n)
    row_ends = _int32_vec(row_ends, rows, "row_ends")
    width = n + n // 32
    if out is None:
        out = torch.empty((rows, width), dtype=torch.int32, device=logits_bf16.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, width) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous int32 [{rows}, {width}]")
    _check(_lib.pack_candidates(_dev(logits_bf16, "logits"), rows, cols, ld,
                                _dev(local_idx, "local_idx"), n, ld_idx, _opt(row_ends, "row_ends"),
                                _dev(out, "out"), _stream(stream)), "pack_candidates")
    return out


def merge_select_rank_major(gathered: torch.Tensor, k: int, out: torch.Tensor | None = None,
                            sat_word: torch.Tensor | None = None, want_sat: bool = True,
                            stream=None):
    """Select from int32 [W, R, n + n/32]; returns (ids [R, k], sat_word [R] or None)."""
    if gathered.dtype != torch.int32 or gathered.dim() != 3 or not gathered.is_contiguous():
        raise ValueError("gathered must be contiguous int32 [W, R, n + n/32]")
    world, rows, width = gathered.shape
    n = width * 32 // 33
    if n + n // 32 != width:
        raise ValueError("gathered's last dimension must be n + n/32")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=gathered.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, k) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous int32 [{rows}, {k}]")
    if sat_word is None and want_sat:
        sat_word = torch.empty((rows,), dtype=torch.int32, device=gathered.device)
    _check(_lib.merge_select_rank_major(_dev(gathered, "gathered"), world, rows, n, k, _dev(out, "out"),
                                        _opt(sat_word, "sat_word"), _stream(stream)),
           "merge_select_rank_major")
    return out, sat_word


def rescue_slots(n: int, k: int) -> int:
    """Receive slots per row of the second round: (k - 1) // n."""
    return (k - 1) // n


def _packed_width(t: torch.Tensor, name: str) -> int:
    w = t.shape[-1]
    m = w * 32 // 33
    if m + m // 32 != w:
        raise ValueError(f"{name}'s last dimension must be m + m/32")
    return m


def rescue_push(local_packed: torch.Tensor, rank: int, world: int, n: int, sat_word: torch.Tensor,
                recv: torch.Tensor, stream=None) -> torch.Tensor:
    """Rank ``rank``'s push of its packed local top-k [R, k + k/32] into the
    receive buffer ``recv`` [R, (k-1)//n, k + k/32] (in place); see the header."""
    lp = local_packed
    if lp.dtype != torch.int32 or lp.dim() != 2 or not lp.is_contiguous():
        raise ValueError("local_packed must be contiguous int32 [R, k + k/32]")
    rows = lp.shape[0]
    k = _packed_width(lp, "local_packed")
    sat_word = _int32_vec(sat_word, rows, "sat_word")
    if (recv.dtype != torch.int32 or not recv.is_contiguous() or
            tuple(recv.shape) != (rows, rescue_slots(n, k), k + k // 32)):
        raise ValueError(f"recv must be contiguous int32 [{rows}, {rescue_slots(n, k)}, {k + k // 32}]")
    _check(_lib.rescue_push(_dev(lp, "local_packed"), rank, world, rows, n, k,
                            _dev(sat_word, "sat_word"), _dev(recv, "recv"), _stream(stream)),
           "rescue_push")
    return recv


def merge_rescue_rank_major(gathered: torch.Tensor, recv: torch.Tensor, sat_word: torch.Tensor,
                            out: torch.Tensor, stream=None) -> torch.Tensor:
    """Second round of the packed merge: re-selects, in place in ``out`` [R, k]
    (round 1's ids), every row whose sat_word enters it; see the header."""
    if gathered.dtype != torch.int32 or gathered.dim() != 3 or not gathered.is_contiguous():
        raise ValueError("gathered must be contiguous int32 [W, R, n + n/32]")
    world, rows, _ = gathered.shape
    n = _packed_width(gathered, "gathered")
    if out.dtype != torch.int32 or out.dim() != 2 or out.shape[0] != rows or not out.is_contiguous():
        raise ValueError(f"out must be contiguous int32 [{rows}, k]")
    k = out.shape[1]
    sat_word = _int32_vec(sat_word, rows, "sat_word")
    if (recv.dtype != torch.int32 or not recv.is_contiguous() or
            tuple(recv.shape) != (rows, rescue_slots(n, k), k + k // 32)):
        raise ValueError(f"recv must be contiguous int32 [{rows}, {rescue_slots(n, k)}, {k + k // 32}]")
    _check(_lib.merge_rescue_rank_major(_dev(gathered, "gathered"), _dev(recv, "recv"), world, rows,
                                        n, k, _dev(sat_word, "sat_word"), _dev(out, "out"),
                                        _stream(stream)), "merge_rescue_rank_major")
    return out


def merge_select_row_major(gathered: torch.Tensor, k: int, out: torch.Tensor | None = None,
                           sat_word: torch.Tensor | None = None, want_sat: bool = True,
                           stream=None):
    """The packed select on row-major int32 [R, W, n + n/32]; returns (ids, sat_word)."""
    if gathered.dtype != torch.int32 or gathered.dim() != 3 or not gathered.is_contiguous():
        raise ValueError("gathered must be contiguous int32 [R, W, n + n/32]")
    rows, world, _ = gathered.shape
    n = _packed_width(gathered, "gathered")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=gathered.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, k) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous int32 [{rows}, {k}]")
    if sat_word is None and want_sat:
        sat_word = torch.empty((rows,), dtype=torch.int32, device=gathered.device)
    _check(_lib.merge_select_row_major(_dev(gathered, "gathered"), world, rows, n, k, _dev(out, "out"),
                                       _opt(sat_word, "sat_word"), _stream(stream)),
           "merge_select_row_major")
    return out, sat_word


def merge_select_pairs_row_major(gathered_pairs: torch.Tensor, k: int, world: int,
                                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The pair select on row-major int32 [R, W * kc, 2]; returns ids [R, k]."""
    g = gathered_pairs
    if g.dtype != torch.int32 or g.dim() != 3 or g.shape[2] != 2 or not g.is_contiguous():
        raise ValueError("gathered_pairs must be contiguous int32 [R, W * kc, 2]")
    rows, wkc, _ = g.shape
    if world < 1 or wkc % world != 0:
        raise ValueError("the candidate dimension must be world * kc")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=g.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, k) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous int32 [{rows}, {k}]")
    _check(_lib.merge_select_pairs_row_major(_dev(g, "gathered_pairs"), world, rows, wkc // world, k,
                                             _dev(out, "out"), _stream(stream)),
           "merge_select_pairs_row_major")
    return out


def emit_rows(ids: torch.Tensor, world: int, dcp_rank: int, req_id: torch.Tensor,
              block_table: torch.Tensor, block_size: int, stride_rows: int,
              rows_out: torch.Tensor | None = None, valid_out: torch.Tensor | None = None,
              stream=None):
    """This rank's owned physical KV rows of ``ids`` [R, k]; returns
    (rows_out [R, out_cols >= k], valid_out [R]); see emit_rows in the header."""
    if ids.dtype != torch.int32 or ids.dim() != 2 or not ids.is_contiguous():
        raise ValueError("ids must be contiguous int32 [R, k]")
    rows, k = ids.shape
    req_id = _int32_vec(req_id, rows, "req_id")
    if req_id is None:
        raise ValueError("req_id is required")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
            (block_table.shape[1] > 1 and block_table.stride(1) != 1):
        raise ValueError("block_table must be int32 [Q, B_max] with unit column stride")
    table_rows, table_cols = block_table.shape
    ld_table = block_table.stride(0) if table_rows > 1 else table_cols
    if rows_out is None:
        rows_out = torch.empty((rows, k), dtype=torch.int32, device=ids.device)
    if rows_out.dtype != torch.int32 or rows_out.dim() != 2 or rows_out.shape[0] != rows or \
            rows_out.shape[1] < k or not rows_out.is_contiguous():
        raise ValueError(f"rows_out must be contiguous int32 [{rows}, >= {k}]")
    if valid_out is None:
        valid_out = torch.empty((rows,), dtype=torch.int32, device=ids.device)
    valid_out = _int32_vec(valid_out, rows, "valid_out")
    _check(_lib.emit_rows(_dev(ids, "ids"), rows, k, world, dcp_rank, _dev(req_id, "req_id"),
                          _dev(block_table, "block_table"), table_rows, table_cols, ld_table,
                          block_size, stride_rows, _dev(rows_out, "rows_out"), rows_out.shape[1],
                          _dev(valid_out, "valid_out"), _stream(stream)), "emit_rows")
    return rows_out, valid_out


def _kv_rows(rows, k, dcp_rank, req_id, block_table, block_size, stride_rows, rows_out, valid_out,
             device):
    req_id = _int32_vec(req_id, rows, "req_id")
    if req_id is None:
        raise ValueError("req_id is required")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
            (block_table.shape[1] > 1 and block_table.stride(1) != 1):
        raise ValueError("block_table must be int32 [Q, B_max] with unit column stride")
    table_rows, table_cols = block_table.shape
    ld_table = block_table.stride(0) if table_rows > 1 else table_cols
    if rows_out is None:
        rows_out = torch.empty((rows, k), dtype=torch.int32, device=device)
    if rows_out.dtype != torch.int32 or rows_out.dim() != 2 or rows_out.shape[0] != rows or \
            rows_out.shape[1] < k or not rows_out.is_contiguous():
        raise ValueError(f"rows_out must be contiguous int32 [{rows}, >= {k}]")
    if valid_out is None:
        valid_out = torch.empty((rows,), dtype=torch.int32, device=device)
    valid_out = _int32_vec(valid_out, rows, "valid_out")
    kv = _KvRows(dcp_rank, req_id.data_ptr(), block_table.data_ptr(), table_rows, table_cols, ld_table,
                 block_size, stride_rows, rows_out.data_ptr(), rows_out.shape[1], valid_out.data_ptr())
    return kv, rows_out, valid_out


def merge_select_rank_major_rows(gathered: torch.Tensor, k: int, dcp_rank: int, req_id: torch.Tensor,
                                 block_table: torch.Tensor, block_size: int, stride_rows: int,
                                 rows_out: torch.Tensor | None = None,
                                 valid_out: torch.Tensor | None = None,
                                 out_ids: torch.Tensor | None = None,
                                 sat_word: torch.Tensor | None = None, stream=None):
    """Packed select writing this rank's owned physical rows (and optionally
    ids / sat_word); returns (rows_out, valid_out, out_ids, sat_word)."""
    if gathered.dtype != torch.int32 or gathered.dim() != 3 or not gathered.is_contiguous():
        raise ValueError("gathered must be contiguous int32 [W, R, n + n/32]")
    world, rows, _ = gathered.shape
    n = _packed_width(gathered, "gathered")
    kv, rows_out, valid_out = _kv_rows(rows, k, dcp_rank, req_id, block_table, block_size, stride_rows,
                                       rows_out, valid_out, gathered.device)
    if out_ids is not None and (out_ids.dtype != torch.int32 or tuple(out_ids.shape) != (rows, k) or
                                not out_ids.is_contiguous()):
        raise ValueError(f"out_ids must be contiguous int32 [{rows}, {k}]")
    sat_word = _int32_vec(sat_word, rows, "sat_word")
    _check(_lib.merge_select_rank_major_rows(_dev(gathered, "gathered"), world, rows, n, k,
                                             ctypes.byref(kv), _opt(out_ids, "out_ids"),
                                             _opt(sat_word, "sat_word"), _stream(stream)),
           "merge_select_rank_major_rows")
    return rows_out, valid_out, out_ids, sat_word


def merge_rescue_rank_major_rows(gathered: torch.Tensor, recv: torch.Tensor, sat_word: torch.Tensor,
                                 k: int, dcp_rank: int, req_id: torch.Tensor,
                                 block_table: torch.Tensor, block_size: int, stride_rows: int,
                                 rows_out: torch.Tensor, valid_out: torch.Tensor,
                                 out_ids: torch.Tensor | None = None, stream=None):
    """Second round rewriting the owned rows (and optionally ids) of the rows
    that enter it, in place; returns (rows_out, valid_out)."""
    if gathered.dtype != torch.int32 or gathered.dim() != 3 or not gathered.is_contiguous():
        raise ValueError("gathered must be contiguous int32 [W, R, n + n/32]")
    world, rows, _ = gathered.shape
    n = _packed_width(gathered, "gathered")
    kv, rows_out, valid_out = _kv_rows(rows, k, dcp_rank, req_id, block_table, block_size, stride_rows,
                                       rows_out, valid_out, gathered.device)
    sat_word = _int32_vec(sat_word, rows, "sat_word")
    if (recv.dtype != torch.int32 or not recv.is_contiguous() or
            tuple(recv.shape) != (rows, rescue_slots(n, k), k + k // 32)):
        raise ValueError(f"recv must be contiguous int32 [{rows}, {rescue_slots(n, k)}, {k + k // 32}]")
    if out_ids is not None and (out_ids.dtype != torch.int32 or tuple(out_ids.shape) != (rows, k) or
                                not out_ids.is_contiguous()):
        raise ValueError(f"out_ids must be contiguous int32 [{rows}, {k}]")
    _check(_lib.merge_rescue_rank_major_rows(_dev(gathered, "gathered"), _dev(recv, "recv"), world, rows,
                                             n, k, _dev(sat_word, "sat_word"), ctypes.byref(kv),
                                             _opt(out_ids, "out_ids"), _stream(stream)),
           "merge_rescue_rank_major_rows")
    return rows_out, valid_out


def pack_pairs(logits: torch.Tensor, local_idx: torch.Tensor, rank: int, world: int,
               row_ends: torch.Tensor | None = None, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """(score bits, gid) pairs int32 [rows, kc, 2]; see pack_pairs in the header."""
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    rows, cols, ld = _rows_ld(logits, "logits")
    if local_idx.dtype != torch.int32:
        raise TypeError("local_idx must be int32")
    r2, kc, ld_idx = _rows_ld(local_idx, "local_idx")
    if r2 != rows:
        raise ValueError("local_idx must have one row per logits row")
    if rows <= 1:
        ld_idx = max(ld_idx, kc)
    row_ends = _int32_vec(row_ends, rows, "row_ends")
    if out is None:
        out = torch.empty((rows, kc, 2), dtype=torch.int32, device=logits.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, kc, 2) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous int32 [{rows}, {kc}, 2]")
    _check(_lib.pack_pairs(_dev(logits, "logits"), rows, cols, ld, _dev(local_idx, "local_idx"), kc,
                           ld_idx, _opt(row_ends, "row_ends"), rank, world, _dev(out, "out"),
                           _stream(stream)), "pack_pairs")
    return out


def merge_select_pairs_rank_major(gathered_pairs: torch.Tensor, k: int,
                                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Select from int32 [W, R, kc, 2] read in place; returns ids [R, k]."""
    g = gathered_pairs
    if g.dtype != torch.int32 or g.dim() != 4 or g.shape[3] != 2 or not g.is_contiguous():
        raise ValueError("gathered_pairs must be contiguous int32 [W, R, kc, 2]")
    world, rows, kc, _ = g.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=g.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (rows, k) or not out.is_contiguous():
        raise ValueError(f"out must be contiguous int32 [{rows}, {k}]")
    _check(_lib.merge_select_pairs_rank_major(_dev(g, "gathered_pairs"), world, rows, kc, k,
                                              _dev(out, "out"), _stream(stream)),
           "merge_select_pairs_rank_major")
    return out


def raw_library() -> ctypes.CDLL:
    """The loaded shared library (for ABI-level tests)."""
    return _lib
