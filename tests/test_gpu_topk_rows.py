"""GPU parity of topk_rows against the CPU oracle (bit-exact ids).

Covers the pages' test plan for the prefill selector (empty/short rows, lengths
around k, full rows, strided output, untouched padding, -1 tails, graph replay
after updating row ends) plus every special value and adversarial order, and
the measured workloads at full size, every row against the oracle.
"""

import numpy as np
import pytest

import datagen
import oracle
from gpu_common import assert_ids_equal, bf16_dev, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rts():
    import row_top_select_amd
    return row_top_select_amd


def run_gpu(rts, x, ends, k, dtype="f32", out_cols=None, workspace="auto"):
    xt = dev(x) if dtype == "f32" else bf16_dev(x)
    et = None if ends is None else dev(ends.astype(np.int32))
    out = None
    if out_cols is not None:
        out = torch.full((x.shape[0], out_cols), 777, dtype=torch.int32, device="cuda")
    res = rts.topk_rows(xt, k, row_ends=et, out=out, workspace=workspace)
    return host(res)


def check(rts, x, ends, k, dtype="f32", what="", **kw):
    got = run_gpu(rts, x, ends, k, dtype, **kw)
    exp = oracle.topk_rows(x, ends, k)
    assert_ids_equal(got[:, :k], exp, what or f"{x.shape} k={k} {dtype}")
    return got


def test_tiny_config(rts):
    w = datagen.WORKLOADS["tiny"]
    say("tiny", w)
    check(rts, datagen.logits(w), datagen.row_ends(w), w.k, what="tiny 64x8192")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [1, 7, 64, 100, 512, 600, 2048])
def test_random_shapes(rts, dtype, k):
    rng = np.random.default_rng(1000 + k + (dtype == "bf16"))
    for trial in range(3):
        rows = int(rng.integers(1, 40))
        cols = int(rng.integers(1, 9000))
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        ends = rng.integers(-5, cols + 50, size=rows).astype(np.int32)
        ends[0] = cols
        if rows > 2:
            ends[1] = min(k, cols)
            ends[2] = max(0, min(k - 1, cols))
        say("random", dtype, k, rows, cols, trial)
        if dtype == "bf16":
            check(rts, datagen.bf16_bits(x), ends, k, "bf16")
        else:
            check(rts, x, ends, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_special_values_and_ties(rts, dtype):
    rng = np.random.default_rng(5)
    rows, cols, k = 24, 3000, 256
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1.0, -1.0],
                        np.float32)
    x = rng.choice(specials, size=(rows, cols))
    ints = rng.integers(-3, 4, size=(rows, cols)).astype(np.float32)
    x = np.where(rng.random((rows, cols)) < 0.5, ints, x)
    ends = rng.integers(0, cols + 1, size=rows).astype(np.int32)
    say("specials", dtype)
    if dtype == "bf16":
        check(rts, datagen.bf16_bits(x), ends, k, "bf16")
    else:
        check(rts, x, ends, k)


@pytest.mark.parametrize("cols", [20000, 8192, 3000])
@pytest.mark.parametrize("case", ["ascending", "descending", "equal", "nan", "inf_many",
                                  "plus100", "times1e-8", "neg"])
def test_adversarial_rows(rts, case, cols):
    # Three row lengths: 20000 (several pieces per row in the planner's
    # launch), 8192 and 3000 (one piece per row, many compactions per piece).
    rows, k = 16, 512
    rng = np.random.default_rng(9)
    base = rng.standard_normal((rows, cols)).astype(np.float32)
    if case == "ascending":
        x = np.tile(np.arange(cols, dtype=np.float32), (rows, 1))
    elif case == "descending":
        x = np.tile(-np.arange(cols, dtype=np.float32), (rows, 1))
    elif case == "equal":
        x = np.full((rows, cols), 2.5, np.float32)
    elif case == "nan":
        x = np.full((rows, cols), np.nan, np.float32)
        x[::2, ::97] = 1.0
    elif case == "inf_many":
        x = base.copy()
        x[rng.random((rows, cols)) < 0.05] = np.inf
    elif case == "plus100":
        x = base + np.float32(100.0)
    elif case == "times1e-8":
        x = base * np.float32(1e-8)
    else:
        x = -np.abs(base)
    ends = np.full(rows, cols, np.int32)
    ends[1] = 0
    ends[2] = 511
    ends[3] = 513
    say("adversarial", case, cols)
    check(rts, x, ends, k, what=f"{case} {cols}")


def test_null_row_ends_strided_io(rts):
    rng = np.random.default_rng(3)
    big = rng.standard_normal((33, 5003)).astype(np.float32)
    x = big[:, 1:4001]                      # misaligned start, ld = 5003
    k = 300
    xt = dev(big)[:, 1:4001]
    out = torch.full((33, k + 13), 777, dtype=torch.int32, device="cuda")
    say("strided")
    rts.topk_rows(xt, k, row_ends=None, out=out)
    got = host(out)
    assert (got[:, k:] == 777).all(), "columns past k must stay untouched"
    assert_ids_equal(got[:, :k], oracle.topk_rows(np.ascontiguousarray(x), None, k), "strided")


def test_workspace_split_equals_single(rts):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 60000)).astype(np.float32)
    ends = np.array([60000, 59999, 0, 1, 511, 512, 513, 40000], np.int32)
    say("split")
    a = run_gpu(rts, x, ends, 512, workspace="auto")
    b = run_gpu(rts, x, ends, 512, workspace=None)
    exp = oracle.topk_rows(x, ends, 512)
    assert_ids_equal(a, exp, "split")
    assert_ids_equal(b, exp, "single")


def test_determinism(rts):
    w = datagen.WORKLOADS["ties"]
    x = datagen.logits(w, blocks=[0])[:256]
    ends = datagen.row_ends(w)[:256]
    xt, et = dev(x), dev(ends)
    say("determinism")
    first = host(rts.topk_rows(xt, 512, row_ends=et))
    for _ in range(5):
        assert np.array_equal(host(rts.topk_rows(xt, 512, row_ends=et)), first)


def test_graph_replay_after_updating_row_ends(rts):
    rng = np.random.default_rng(8)
    rows, cols, k = 64, 9000, 512
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    xt = dev(x)
    et = dev(np.full(rows, cols, np.int32))
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    rts.topk_rows(xt, k, row_ends=et, out=out)      # warm up outside capture
    torch.cuda.synchronize()
    say("graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rts.topk_rows(xt, k, row_ends=et, out=out)
    for trial in range(4):
        ends = rng.integers(-2, cols + 2, size=rows).astype(np.int32)
        et.copy_(torch.from_numpy(ends))
        torch.cuda.synchronize()
        g.replay()
        got = host(out)
        assert_ids_equal(got, oracle.topk_rows(x, ends, k), f"replay {trial}")
        rts.topk_rows(xt, 3, row_ends=et)             # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["prefill", "ties", "long"])
def test_full_size_configs(rts, name):
    w = datagen.WORKLOADS[name]
    say("full", w)
    x = datagen.logits(w)
    ends = datagen.row_ends(w)
    got = run_gpu(rts, x, ends, w.k)
    exp = oracle.topk_rows(x, ends, w.k)
    assert_ids_equal(got, exp, name)


def test_decode_config(rts):
    w = datagen.WORKLOADS["decode"]
    say("decode", w)
    x = datagen.logits(w)
    ends = datagen.row_ends(w)
    assert_ids_equal(run_gpu(rts, x, ends, w.k), oracle.topk_rows(x, ends, w.k), "decode")


def test_verylong_config_every_row(rts):
    # The headline workload at full size, launched as the benchmark launches it
    # (no workspace), every row against the oracle.
    w = datagen.WORKLOADS["verylong"]
    say("verylong generate")
    x = datagen.logits(w, threads=8)
    ends = datagen.row_ends(w)
    xt, et = dev(x), dev(ends)
    say("verylong run")
    got = host(rts.topk_rows(xt, w.k, row_ends=et, workspace=None))
    del xt
    say("verylong oracle")
    assert_ids_equal(got, oracle.topk_rows(x, ends, w.k), "verylong")


# Distribution robustness (the pages' ablation at 8K queries x 8K keys: the same
# normal values, then +100 and *1e-8, which concentrate the scores; causal rows
# i + 1 long, so the first 511 rows end in -1 tails).  Full parity on every row.
@pytest.mark.parametrize("name", ["robust", "robust_plus100", "robust_scale1e8"])
def test_distribution_robustness(rts, name):
    w = datagen.WORKLOADS[name]
    say("robust", w)
    x = datagen.logits(w)
    ends = datagen.row_ends(w)
    got = run_gpu(rts, x, ends, w.k)
    assert_ids_equal(got, oracle.topk_rows(x, ends, w.k), name)
    assert (got[:w.k - 1, w.k - 1] == -1).all()  # rows shorter than k end in -1


def test_verylong_bf16_every_row(rts):
    # The headline shape in bf16 (its fp32 values rounded to nearest even),
    # every row against the oracle.
    w = datagen.WORKLOADS["verylong"]
    say("verylong bf16 generate")
    xb = datagen.bf16_bits(datagen.logits(w, threads=8))
    ends = datagen.row_ends(w)
    say("verylong bf16 run")
    got = host(rts.topk_rows(bf16_dev(xb), w.k, row_ends=dev(ends)))
    say("verylong bf16 oracle")
    assert_ids_equal(got, oracle.topk_rows(xb, ends, w.k), "verylong bf16")


# Short rows with a large k (k > 1024, rows of at most 16384 columns, 256 rows
# or more) take the whole-row-in-registers kernel; the rest of this file's
# shapes stream (1024 and 777 below stream, as neighbours).  Every row against
# the oracle.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols,k", [(16384, 2048), (16384, 1024), (8192, 2048), (8192, 1025),
                                    (3001, 1500), (12289, 777), (700, 2048), (16000, 1100)])
def test_block_rows_random(rts, dtype, cols, k):
    rng = np.random.default_rng(cols + k + (dtype == "bf16"))
    rows = 300
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    ends = rng.integers(-3, cols + 20, size=rows).astype(np.int32)
    ends[:4] = [cols, 0, min(k - 1, cols), min(k + 1, cols)]
    say("block rows", dtype, cols, k)
    if dtype == "bf16":
        check(rts, datagen.bf16_bits(x), ends, k, "bf16", what=f"block bf16 {cols} {k}")
    else:
        check(rts, x, ends, k, what=f"block {cols} {k}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["ties", "specials", "equal", "ascending", "plus100", "dup"])
def test_block_rows_adversarial(rts, case, dtype):
    rng = np.random.default_rng(17)
    rows, cols, k = 260, 16384, 2048
    if case == "ties":
        x = rng.integers(0, 64, size=(rows, cols)).astype(np.float32)
    elif case == "dup":
        # N(0,1) on a grid: even rows on 1/256 (up to about 23 copies of a
        # selected value), odd rows on 1/64 (about 64), so the fp32 rows'
        # ordering buckets hold tied keys (ranked by column) and overflow into
        # the sort network on alternate rows.
        grid = np.where(np.arange(rows)[:, None] % 2 == 0, 256.0, 64.0)
        x = (np.round(rng.standard_normal((rows, cols)) * grid) / grid).astype(np.float32)
    elif case == "specials":
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        u = rng.random((rows, cols))
        x[u < 0.01] = np.inf
        x[(u >= 0.01) & (u < 0.02)] = -np.inf
        x[(u >= 0.02) & (u < 0.05)] = np.nan
        x[(u >= 0.05) & (u < 0.06)] = -0.0
        x[(u >= 0.06) & (u < 0.07)] = 0.0
        x[:8] = np.nan                       # rows with no candidate at all
        x[8:16, ::3] = np.nan
    elif case == "equal":
        x = np.full((rows, cols), 1.25, np.float32)
    elif case == "ascending":
        x = np.tile(np.arange(cols, dtype=np.float32), (rows, 1))
    else:
        x = rng.standard_normal((rows, cols)).astype(np.float32) + np.float32(100.0)
    ends = np.full(rows, cols, np.int32)
    ends[1::7] = rng.integers(0, cols, size=len(ends[1::7]))
    say("block adversarial", case, dtype)
    if dtype == "bf16":
        check(rts, datagen.bf16_bits(x), ends, k, "bf16", what=f"block bf16 {case}")
    else:
        check(rts, x, ends, k, what=f"block {case}")


def test_block_rows_misaligned_bf16(rts):
    # bf16 rows one element past an 8-byte boundary (every element read on its
    # own), ragged row ends, k > 1024 on 8192 and 16384 columns
    rng = np.random.default_rng(29)
    for cols, k in ((8192, 1500), (16383, 2048)):
        rows = 262
        big = datagen.bf16_bits(rng.standard_normal((rows, cols + 1)).astype(np.float32))
        xt = bf16_dev(big)[:, 1:]
        ends = rng.integers(0, cols + 1, size=rows).astype(np.int32)
        ends[0] = cols
        say("block misaligned bf16", cols, k)
        got = host(rts.topk_rows(xt, k, row_ends=dev(ends)))
        assert_ids_equal(got, oracle.topk_rows(np.ascontiguousarray(big[:, 1:]), ends, k),
                         f"block misaligned bf16 {cols} {k}")


def test_block_rows_strided_and_misaligned(rts):
    # logits starting one element past a 16-byte boundary (element loads) and
    # an output wider than k (columns past k untouched)
    rng = np.random.default_rng(23)
    rows, cols, k = 270, 9000, 1100
    big = rng.standard_normal((rows, cols + 1)).astype(np.float32)
    xt = dev(big)[:, 1:]
    out = torch.full((rows, k + 5), 777, dtype=torch.int32, device="cuda")
    ends = rng.integers(0, cols + 1, size=rows).astype(np.int32)
    say("block misaligned")
    rts.topk_rows(xt, k, row_ends=dev(ends), out=out)
    got = host(out)
    assert (got[:, k:] == 777).all()
    assert_ids_equal(got[:, :k], oracle.topk_rows(np.ascontiguousarray(big[:, 1:]), ends, k),
                     "block misaligned")
