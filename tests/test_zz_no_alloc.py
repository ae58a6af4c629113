"""topk_rows_noalloc through the C ABI against topk_rows (the same entry point
with a caller workspace), bit for bit, on consecutive calls that reuse the
library's static scratch: shapes that split rows over workgroups (the partial
lists live in the scratch), the second call of each pair smaller than the
first, and a shape that needs no split."""

import ctypes

import numpy as np
import pytest

import oracle
from gpu_common import assert_ids_equal, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rts():
    import row_top_select_amd
    return row_top_select_amd


def _noalloc(lib, x, dtype, ends, k, out):
    rows, cols = x.shape
    s = torch.cuda.current_stream().cuda_stream
    return lib.topk_rows_noalloc(ctypes.c_void_p(x.data_ptr()), dtype, rows, cols, x.stride(0),
                                 None if ends is None else ctypes.c_void_p(ends.data_ptr()), k,
                                 ctypes.c_void_p(out.data_ptr()), out.stride(0), ctypes.c_void_p(s))


# (rows, cols, k): each pair is (larger, smaller); all but the last split rows
CASES = [((64, 102400, 512), (16, 60000, 256)),
         ((300, 200000, 2048), (7, 150000, 2048)),
         ((40, 80000, 1024), (2, 9000, 100))]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_topk_rows(rts, first, second):
    lib = rts.raw_library()
    rng = np.random.default_rng(first[0] + second[0])
    for rows, cols, k in (first, second):
        want_split = rts.topk_rows_workspace_size(torch.float32, rows, cols, k) > 0
        say("noalloc", rows, cols, k, "split" if want_split else "no split")
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        ends = rng.integers(0, cols + 1, size=rows).astype(np.int32)
        ends[0] = cols
        xt, et = dev(x), dev(ends)
        ref = rts.topk_rows(xt, k, row_ends=et, workspace="auto")
        out = torch.full((rows, k + 3), 777, dtype=torch.int32, device="cuda")
        assert _noalloc(lib, xt, 0, et, k, out) == 0
        got = host(out)
        assert (got[:, k:] == 777).all(), "columns past k must stay untouched"
        assert_ids_equal(got[:, :k], host(ref), "noalloc vs topk_rows")
        if rows <= 16:
            assert_ids_equal(got[:, :k], oracle.topk_rows(x, ends, k), "noalloc vs oracle")


def test_noalloc_bf16_and_null_row_ends(rts):
    lib = rts.raw_library()
    rng = np.random.default_rng(12)
    for rows, cols, k in ((32, 120000, 512), (5, 70000, 64)):
        say("noalloc bf16", rows, cols, k)
        x = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32)).cuda() \
            .to(torch.bfloat16)
        ref = rts.topk_rows(x, k, workspace="auto")
        out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
        assert _noalloc(lib, x, 1, None, k, out) == 0
        assert_ids_equal(host(out), host(ref), "bf16 noalloc vs topk_rows")
