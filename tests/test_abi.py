"""The C-ABI library: it loads, exports every symbol the header declares, and
rejects invalid arguments on the host before touching the GPU (no compute call
happens in these tests, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "row_top_select.h")
LIB = os.path.join(ROOT, "row_top_select_amd", "librow_top_select.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        # by path: importing the package would first load the missing library
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_rts_build", os.path.join(ROOT, "row_top_select_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build(verbose=False)
    lib = ctypes.CDLL(LIB)
    i64, i32, p, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.topk_rows.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i32, p, i64, p, sz, p]
    lib.pack_candidates.argtypes = [p, i64, i64, i64, p, i32, i64, p, p, p]
    lib.merge_select_rank_major.argtypes = [p, i32, i64, i32, i32, p, p, p]
    lib.pack_pairs.argtypes = [p, i64, i64, i64, p, i32, i64, p, i32, i32, p, p]
    lib.merge_select_pairs_rank_major.argtypes = [p, i32, i64, i32, i32, p, p]
    lib.merge_select_row_major.argtypes = [p, i32, i64, i32, i32, p, p, p]
    lib.merge_select_pairs_row_major.argtypes = [p, i32, i64, i32, i32, p, p]
    lib.rescue_push.argtypes = [p, i32, i32, i64, i32, i32, p, p, p]
    lib.merge_rescue_rank_major.argtypes = [p, p, i32, i64, i32, i32, p, p, p]
    lib.emit_rows.argtypes = [p, i64, i32, i32, i32, p, p, i64, i32, i64, i32, i64, p, i32, p, p]
    lib.merge_select_rank_major_rows.argtypes = [p, i32, i64, i32, i32, p, p, p, p]
    lib.merge_rescue_rank_major_rows.argtypes = [p, p, i32, i64, i32, i32, p, p, p, p]
    lib.topk_rows_workspace_size.argtypes = [ctypes.c_int, i64, i64, i32]
    lib.topk_rows_workspace_size.restype = sz
    lib.rts_status_string.argtypes = [ctypes.c_int]
    lib.rts_status_string.restype = ctypes.c_char_p
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"topk_rows", "pack_candidates", "merge_select_rank_major", "pack_pairs",
                          "merge_select_pairs_rank_major", "topk_rows_workspace_size",
                          "rts_status_string", "merge_select_row_major",
                          "merge_select_pairs_row_major", "rescue_push", "merge_rescue_rank_major",
                          "emit_rows", "merge_select_rank_major_rows",
                          "merge_rescue_rank_major_rows"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.rts_status_string(code).startswith(b"RTS_")
    assert lib.rts_status_string(7) == b"unknown rts_status"


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def test_topk_rows_validation(lib):
    EINVAL, EUNSUP, EWS = -1, -2, -3
    f = lib.topk_rows
    assert f(FAKE, 2, 4, 8, 8, None, 2, FAKE, 2, None, 0, None) == EINVAL      # dtype
    assert f(FAKE, 0, -1, 8, 8, None, 2, FAKE, 2, None, 0, None) == EINVAL     # rows < 0
    assert f(FAKE, 0, 4, 8, 7, None, 2, FAKE, 2, None, 0, None) == EINVAL      # ld < cols
    assert f(FAKE, 0, 4, 8, 8, None, 0, FAKE, 2, None, 0, None) == EINVAL      # k < 1
    assert f(FAKE, 0, 4, 8, 8, None, 3, FAKE, 2, None, 0, None) == EINVAL      # ld_out < k
    assert f(FAKE, 0, 4, 8, 8, None, 2049, FAKE, 4096, None, 0, None) == EUNSUP
    assert f(None, 0, 4, 8, 8, None, 2, FAKE, 2, None, 0, None) == EINVAL      # null logits
    assert f(FAKE, 0, 4, 8, 8, None, 2, None, 2, None, 0, None) == EINVAL      # null out
    assert f(ctypes.c_void_p(0x10002), 0, 4, 8, 8, None, 2, FAKE, 2, None, 0, None) == EINVAL
    assert f(FAKE, 0, 4, 8, 8, None, 2, FAKE, 2, None, 64, None) == EINVAL     # bytes, no ptr
    # a split shape with a too-small workspace
    need = lib.topk_rows_workspace_size(0, 64, 102400, 512)
    assert need > 0
    assert f(FAKE, 0, 64, 102400, 102400, None, 512, FAKE, 512, FAKE, need - 8, None) == EWS
    assert f(FAKE, 0, 0, 8, 8, None, 2, FAKE, 2, None, 0, None) == 0           # nothing to do


def test_workspace_size(lib):
    assert lib.topk_rows_workspace_size(0, 4096, 102400, 512) == 0   # one wave per row suffices
    assert lib.topk_rows_workspace_size(0, 64, 102400, 512) % (512 * 8) == 0
    assert lib.topk_rows_workspace_size(5, 4, 4, 4) == 0


def test_merge_and_pack_validation(lib):
    EINVAL, EUNSUP = -1, -2
    assert lib.pack_candidates(FAKE, 4, 8, 8, FAKE, 48, 48, None, FAKE, None) == EINVAL   # n % 32
    assert lib.pack_candidates(FAKE, 4, 8, 8, FAKE, 32, 16, None, FAKE, None) == EINVAL   # ld_idx
    assert lib.merge_select_rank_major(FAKE, 17, 4, 32, 64, FAKE, None, None) == EINVAL   # world
    assert lib.merge_select_rank_major(FAKE, 0, 4, 32, 64, FAKE, None, None) == EINVAL
    assert lib.merge_select_rank_major(FAKE, 8, 4, 40, 64, FAKE, None, None) == EINVAL    # n % 32
    assert lib.merge_select_rank_major(FAKE, 8, 4, 32, 4096, FAKE, None, None) == EUNSUP  # k
    assert lib.merge_select_rank_major(FAKE, 16, 4, 4096, 512, FAKE, None, None) == EUNSUP
    assert lib.merge_select_rank_major(None, 8, 4, 32, 64, FAKE, None, None) == EINVAL
    assert lib.pack_pairs(FAKE, 4, 8, 8, FAKE, 4, 4, None, 3, 3, FAKE, None) == EINVAL     # rank
    assert lib.pack_pairs(FAKE, 4, 8, 8, FAKE, 4, 4, None, 0, 3, ctypes.c_void_p(0x10004),
                          None) == EINVAL                                                  # align
    assert lib.pack_pairs(FAKE, 4, 1 << 30, 1 << 30, FAKE, 4, 4, None, 0, 4, FAKE,
                          None) == EUNSUP                                                  # gid range
    assert lib.merge_select_pairs_rank_major(FAKE, 8, 4, 8192, 512, FAKE, None) == EUNSUP
    assert lib.merge_select_pairs_rank_major(FAKE, 8, 4, 64, 0, FAKE, None) == EINVAL


class KvRows(ctypes.Structure):
    """rts_kv_rows, restated from the header."""
    _fields_ = [("dcp_rank", ctypes.c_int32), ("req_id", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("table_rows", ctypes.c_int64),
                ("table_cols", ctypes.c_int32), ("ld_table", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("stride_rows", ctypes.c_int64),
                ("rows_out", ctypes.c_void_p), ("out_cols", ctypes.c_int32),
                ("valid_out", ctypes.c_void_p)]


def test_second_round_layout_and_rows_validation(lib):
    EINVAL, EUNSUP = -1, -2
    # row-major selects share the rank-major checks
    assert lib.merge_select_row_major(FAKE, 17, 4, 32, 64, FAKE, None, None) == EINVAL
    assert lib.merge_select_pairs_row_major(FAKE, 8, 4, 8192, 512, FAKE, None) == EUNSUP
    # push: rank outside the world, k not a multiple of 32, null recv
    assert lib.rescue_push(FAKE, 8, 8, 4, 384, 2048, FAKE, FAKE, None) == EINVAL
    assert lib.rescue_push(FAKE, 0, 8, 4, 384, 2000, FAKE, FAKE, None) == EINVAL
    assert lib.rescue_push(FAKE, 0, 8, 4, 384, 2048, FAKE, None, None) == EINVAL
    assert lib.rescue_push(FAKE, 0, 8, 4, 4096, 2048, FAKE, FAKE, None) == 0    # no slots: no-op
    # rescue: too many candidate slots, null sat_word
    assert lib.merge_rescue_rank_major(FAKE, FAKE, 16, 4, 32, 2048, FAKE, FAKE, None) == EUNSUP
    assert lib.merge_rescue_rank_major(FAKE, FAKE, 8, 4, 384, 2048, None, FAKE, None) == EINVAL
    # emit_rows: rank >= world, out_cols < k, block_size 0, ld_table < cols
    assert lib.emit_rows(FAKE, 4, 64, 8, 8, FAKE, FAKE, 2, 4, 4, 64, 64, FAKE, 64, FAKE, None) == EINVAL
    assert lib.emit_rows(FAKE, 4, 64, 8, 0, FAKE, FAKE, 2, 4, 4, 64, 64, FAKE, 63, FAKE, None) == EINVAL
    assert lib.emit_rows(FAKE, 4, 64, 8, 0, FAKE, FAKE, 2, 4, 4, 0, 64, FAKE, 64, FAKE, None) == EINVAL
    assert lib.emit_rows(FAKE, 4, 64, 8, 0, FAKE, FAKE, 2, 4, 3, 64, 64, FAKE, 64, FAKE, None) == EINVAL
    assert lib.emit_rows(FAKE, 4, 4096, 8, 0, FAKE, FAKE, 2, 4, 4, 64, 64, FAKE, 4096, FAKE,
                         None) == EUNSUP
    # fused rows: a missing or invalid rts_kv_rows
    assert lib.merge_select_rank_major_rows(FAKE, 8, 4, 384, 2048, None, None, None, None) == EINVAL
    kv = KvRows(8, FAKE.value, FAKE.value, 2, 4, 4, 64, 64, FAKE.value, 2048, FAKE.value)   # rank 8
    assert lib.merge_select_rank_major_rows(FAKE, 8, 4, 384, 2048, ctypes.byref(kv), None, None,
                                            None) == EINVAL
    kv.dcp_rank, kv.out_cols = 3, 2047                                                   # out_cols < k
    assert lib.merge_select_rank_major_rows(FAKE, 8, 4, 384, 2048, ctypes.byref(kv), None, None,
                                            None) == EINVAL
    kv.out_cols, kv.rows_out = 2048, None                                                # null rows_out
    assert lib.merge_rescue_rank_major_rows(FAKE, FAKE, 8, 4, 384, 2048, FAKE, ctypes.byref(kv),
                                            None, None) == EINVAL


def test_topk_rows_noalloc_validation(lib):
    EINVAL, EUNSUP = -1, -2
    f = lib.topk_rows_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert f(FAKE, 2, 4, 8, 8, None, 2, FAKE, 2, None) == EINVAL        # dtype
    assert f(FAKE, 0, 4, 8, 7, None, 2, FAKE, 2, None) == EINVAL        # ld < cols
    assert f(FAKE, 0, 4, 8, 8, None, 0, FAKE, 2, None) == EINVAL        # k < 1
    assert f(FAKE, 0, 4, 8, 8, None, 4, FAKE, 3, None) == EINVAL        # ld_out < k
    assert f(FAKE, 0, 4, 8, 8, None, 2049, FAKE, 4096, None) == EUNSUP  # k > 2048
    assert f(None, 0, 4, 8, 8, None, 2, FAKE, 2, None) == EINVAL        # null logits
    assert f(ctypes.c_void_p(0x10001), 0, 4, 8, 8, None, 2, FAKE, 2, None) == EINVAL  # misaligned
    assert f(FAKE, 0, 0, 8, 8, None, 2, FAKE, 2, None) == 0             # no rows: nothing to do


def test_split_workspace_fits_the_static_scratch(lib):
    # topk_rows_noalloc keeps split rows' partial lists in a 16 MiB static
    # array: no launch plan may need more, for any shape.
    worst = 0
    for rows in list(range(1, 700)) + [1024, 4096, 1 << 20]:
        for cols in (1000, 20000, 102400, 200000, 10 ** 6, 10 ** 7, (1 << 31) - 1):
            for k in (1, 64, 65, 512, 513, 1024, 1025, 2048):
                for dt in (0, 1):
                    worst = max(worst, lib.topk_rows_workspace_size(dt, rows, cols, k))
    assert 0 < worst <= 16 << 20
