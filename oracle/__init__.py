"""CPU oracle for the row top-K select and the candidate merge.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the library in
``row_top_select_amd`` never does, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, qsort-based, see its header for
the passages each function follows).  This module only compiles it with gcc
when the shared object is missing or stale and marshals numpy arrays.

Parity pins for every function are in ``tests/test_oracle_*.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PLAIN = os.path.join(_HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, for
# checking the oracle itself (tests/test_oracle_sanitized.py): loaded instead
# of the plain one when ORACLE_SANITIZED=1, in a process started with the ASan
# runtime preloaded.
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
SANITIZED = os.environ.get("ORACLE_SANITIZED") == "1"
_LIB = _LIB_SAN if SANITIZED else _LIB_PLAIN
_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]
_SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined"]
_lock = threading.Lock()
_lib = None


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (gcc, OpenMP over rows), or
    with ``sanitize`` into ``liboracle_san.so`` under ASan and UBSan."""
    lib = _LIB_SAN if sanitize else _LIB_PLAIN
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *_FLAGS, *(_SAN_FLAGS if sanitize else []),
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(sanitize=SANITIZED)
            lib = ctypes.CDLL(_LIB)
            i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
            lib.oracle_topk_rows.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i32, p, i64,
                                             ctypes.c_int]
            lib.oracle_pack_candidates.argtypes = [p, i64, i64, i64, p, i32, i64, p, p]
            lib.oracle_merge_select_rank_major.argtypes = [p, i32, i64, i32, i32, p, p]
            lib.oracle_pack_pairs.argtypes = [p, i64, i64, i64, p, i32, i64, p, i32, i32, p]
            lib.oracle_merge_select_pairs_rank_major.argtypes = [p, i32, i64, i32, i32, p]
            lib.oracle_merge_rescue_rank_major.argtypes = [p, p, i32, i64, i32, i32, p, p]
            lib.oracle_rescue_push.argtypes = [p, i32, i32, i64, i32, i32, p, p]
            lib.oracle_emit_rows.argtypes = [p, i64, i32, i32, i32, p, p, i64, i32, i32, i64, p, i32,
                                             p]
            for f in (lib.oracle_topk_rows, lib.oracle_pack_candidates,
                      lib.oracle_merge_select_rank_major, lib.oracle_pack_pairs,
                      lib.oracle_merge_select_pairs_rank_major,
                      lib.oracle_merge_rescue_rank_major, lib.oracle_rescue_push,
                      lib.oracle_emit_rows):
                f.restype = ctypes.c_int
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (rc={rc})")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def topk_rows(x, row_ends, k, out=None, nthreads=0):
    """Exact per-row top-k ids of ``x`` (fp32 ndarray, or bf16 bits as uint16).

    ``row_ends`` is int32 [rows] or None (all rows full).  Returns int32
    [rows, k] (or fills ``out``, whose columns past k are left untouched).
    """
    lib = _load()
    if k < 1:
        raise ValueError("k must be >= 1")
    x = np.asarray(x)
    if x.dtype == np.float32:
        dt = 0
    elif x.dtype == np.uint16:
        dt = 1
    else:
        raise TypeError("x must be float32 or uint16 (bf16 bits)")
    if x.ndim != 2 or x.strides[1] != x.itemsize or x.strides[0] % x.itemsize:
        raise ValueError("x must be 2-D with unit column stride")
    rows, cols = x.shape
    ld = x.strides[0] // x.itemsize if rows > 1 else cols
    if row_ends is not None:
        row_ends = np.ascontiguousarray(row_ends, dtype=np.int32)
        assert row_ends.shape == (rows,)
    if out is None:
        out = np.empty((rows, k), dtype=np.int32)
    assert out.dtype == np.int32 and out.ndim == 2 and out.strides[1] == 4
    ld_out = out.strides[0] // 4 if rows > 1 else k
    _check(lib.oracle_topk_rows(_ptr(x), dt, rows, cols, ld, _ptr(row_ends), k, _ptr(out),
                                ld_out, nthreads), "topk_rows")
    return out


def pack_candidates(x_bf16, local_idx, row_ends=None):
    """B' packed rows int32 [rows, n + n/32] of a local top-n (``local_idx``)."""
    lib = _load()
    x = np.asarray(x_bf16)
    assert x.dtype == np.uint16 and x.ndim == 2 and x.strides[1] == 2
    local_idx = np.ascontiguousarray(local_idx, dtype=np.int32)
    rows, cols = x.shape
    n = local_idx.shape[1]
    if row_ends is not None:
        row_ends = np.ascontiguousarray(row_ends, dtype=np.int32)
    packed = np.empty((rows, n + n // 32), dtype=np.int32)
    ld = x.strides[0] // 2 if rows > 1 else cols
    _check(lib.oracle_pack_candidates(_ptr(x), rows, cols, ld, _ptr(local_idx), n, n,
                                      _ptr(row_ends), _ptr(packed)), "pack_candidates")
    return packed


def merge_select_rank_major(gathered, k, with_sat=True):
    """Select from int32 [W, R, n + n/32]; returns (ids [R, k], sat_word [R] or None)."""
    lib = _load()
    g = np.ascontiguousarray(gathered, dtype=np.int32)
    world, rows, width = g.shape
    n = width * 32 // 33
    assert n + n // 32 == width
    ids = np.empty((rows, k), dtype=np.int32)
    sat = np.empty((rows,), dtype=np.int32) if with_sat else None
    _check(lib.oracle_merge_select_rank_major(_ptr(g), world, rows, n, k, _ptr(ids), _ptr(sat)),
           "merge_select_rank_major")
    return ids, sat


def pack_pairs(x, local_idx, rank, world, row_ends=None):
    """(score bits, gid) pairs int32 [rows, kc, 2] of a local top-kc of fp32 ``x``."""
    lib = _load()
    x = np.asarray(x)
    assert x.dtype == np.float32 and x.ndim == 2 and x.strides[1] == 4
    local_idx = np.ascontiguousarray(local_idx, dtype=np.int32)
    rows, cols = x.shape
    kc = local_idx.shape[1]
    if row_ends is not None:
        row_ends = np.ascontiguousarray(row_ends, dtype=np.int32)
    pairs = np.empty((rows, kc, 2), dtype=np.int32)
    ld = x.strides[0] // 4 if rows > 1 else cols
    _check(lib.oracle_pack_pairs(_ptr(x), rows, cols, ld, _ptr(local_idx), kc, kc,
                                 _ptr(row_ends), rank, world, _ptr(pairs)), "pack_pairs")
    return pairs


def merge_select_pairs_rank_major(pairs, k):
    """Select from int32 [W, R, kc, 2]; returns ids [R, k]."""
    lib = _load()
    p = np.ascontiguousarray(pairs, dtype=np.int32)
    world, rows, kc, two = p.shape
    assert two == 2
    ids = np.empty((rows, k), dtype=np.int32)
    _check(lib.oracle_merge_select_pairs_rank_major(_ptr(p), world, rows, kc, k, _ptr(ids)),
           "merge_select_pairs_rank_major")
    return ids



def rescue_slots(n, k):
    """Receive slots per row: at most (k - 1) // n ranks can be saturated."""
    return (k - 1) // n


def rescue_push(local_packed, rank, world, n, sat_word, recv):
    """Copy rank ``rank``'s packed local top-k [R, k + k/32] into its receive
    slot of ``recv`` [R, S, k + k/32] on the rows whose mask has its bit (in place)."""
    lib = _load()
    lp = np.ascontiguousarray(local_packed, dtype=np.int32)
    rows, pw = lp.shape
    k = pw * 32 // 33
    assert k + k // 32 == pw and recv.dtype == np.int32 and recv.flags.c_contiguous
    assert recv.shape == (rows, rescue_slots(n, k), pw)
    sw = np.ascontiguousarray(sat_word, dtype=np.int32)
    _check(lib.oracle_rescue_push(_ptr(lp), rank, world, rows, n, k, _ptr(sw), _ptr(recv)),
           "rescue_push")
    return recv


def merge_rescue_rank_major(gathered, recv, sat_word, ids):
    """Second round of the packed merge: returns a copy of the round-1 ``ids``
    [R, k] with every row that enters the second round re-selected.

    ``gathered`` int32 [W, R, n + n/32], ``recv`` int32 [R, (k-1)//n, k + k/32].
    """
    lib = _load()
    g = np.ascontiguousarray(gathered, dtype=np.int32)
    world, rows, gw = g.shape
    n = gw * 32 // 33
    out = np.array(ids, dtype=np.int32, copy=True)
    k = out.shape[1]
    assert out.shape == (rows, k)
    rv = np.ascontiguousarray(recv, dtype=np.int32)
    assert rv.shape == (rows, rescue_slots(n, k), k + k // 32)
    sw = np.ascontiguousarray(sat_word, dtype=np.int32)
    _check(lib.oracle_merge_rescue_rank_major(_ptr(g), _ptr(rv), world, rows, n, k, _ptr(sw),
                                              _ptr(out)), "merge_rescue_rank_major")
    return out


def emit_rows(ids, world, dcp_rank, req_id, block_table, block_size, stride_rows, out_cols=None):
    """This rank's owned physical rows of the selected ``ids`` [R, k]; returns
    (rows_out [R, out_cols], valid_out [R]).  ``block_table`` int32 [Q, B_max]."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    rows, k = ids.shape
    out_cols = k if out_cols is None else out_cols
    rq = np.ascontiguousarray(req_id, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    rows_out = np.empty((rows, out_cols), np.int32)
    valid = np.empty((rows,), np.int32)
    _check(lib.oracle_emit_rows(_ptr(ids), rows, k, world, dcp_rank, _ptr(rq), _ptr(bt), bt.shape[0],
                                bt.shape[1], block_size, stride_rows, _ptr(rows_out), out_cols,
                                _ptr(valid)), "emit_rows")
    return rows_out, valid
