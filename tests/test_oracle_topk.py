"""Pins of the oracle's per-row top-K (oracle_topk_rows) to facts outside it.

* golden rows derived by hand from the pages' rule (tests/golden/topk_rows_small.json);
* a pure-Python brute force (tests/brute.py) on tiny random rows with every
  special value (NaN, +-inf, +-0, denormals, ties) and every kind of row end;
* closed forms: all-equal, ascending and descending rows, all-NaN rows,
  more +inf than K, K >= row length (the full order, checked against
  numpy's stable argsort);
* invariants against torch.topk on random rows (selected-score multiset,
  unique ids below the row end, -1 tails, untouched padding columns).
"""

import json
import math
import os

import numpy as np
import pytest

import brute
import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_rows():
    g = json.load(open(os.path.join(GOLDEN, "topk_rows_small.json")))
    rows = g["rows"]
    x = np.array([[float(v) for v in r["values"]] for r in rows], dtype=np.float32)
    ends = np.array([r["row_end"] for r in rows], dtype=np.int32)
    got = oracle.topk_rows(x, ends, g["k"])
    for i, r in enumerate(rows):
        assert got[i].tolist() == r["expected"], (i, r["why"])
    # The same rows in bf16 (every value is exact in bf16).
    got16 = oracle.topk_rows(datagen.bf16_bits(x), ends, g["k"])
    assert np.array_equal(got16, got)


SPECIALS = [0.0, -0.0, math.inf, -math.inf, math.nan, 1e-45, -1e-45, 1.0, -1.0, 2.0]


def _random_rows(rng, rows, cols, mode):
    if mode == "normal":
        x = rng.standard_normal((rows, cols)).astype(np.float32)
    elif mode == "ties":
        x = rng.integers(-3, 4, size=(rows, cols)).astype(np.float32)
    else:
        x = rng.choice(np.array(SPECIALS, dtype=np.float32), size=(rows, cols))
        mix = rng.random((rows, cols)) < 0.5
        x = np.where(mix, rng.integers(-2, 3, size=(rows, cols)).astype(np.float32), x)
    return x


@pytest.mark.parametrize("mode", ["normal", "ties", "specials"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_brute_force_tiny(mode, dtype):
    rng = np.random.default_rng(7 + len(mode) + (dtype == "bf16"))
    for trial in range(30):
        rows = int(rng.integers(1, 17))
        cols = int(rng.integers(1, 65))
        k = int(rng.integers(1, cols + 6))
        x = _random_rows(rng, rows, cols, mode)
        ends = rng.integers(-3, cols + 4, size=rows).astype(np.int32)
        if dtype == "bf16":
            xb = datagen.bf16_bits(x)
            got = oracle.topk_rows(xb, ends, k)
            vals = datagen.bf16_to_f32(xb)
        else:
            got = oracle.topk_rows(x, ends, k)
            vals = x
        for i in range(rows):
            exp = brute.topk_row([float(v) for v in vals[i]], int(ends[i]), k)
            assert got[i].tolist() == exp, (mode, dtype, trial, i)


def test_null_row_ends_means_full_rows():
    x = np.random.default_rng(3).standard_normal((5, 40)).astype(np.float32)
    a = oracle.topk_rows(x, None, 7)
    b = oracle.topk_rows(x, np.full(5, 40, np.int32), 7)
    assert np.array_equal(a, b)


def test_closed_forms():
    cols, k = 300, 64
    # all equal: the k lowest ids
    x = np.full((1, cols), 3.25, np.float32)
    assert oracle.topk_rows(x, None, k)[0].tolist() == list(range(k))
    # ascending: e-1, e-2, ...
    x = np.arange(cols, dtype=np.float32)[None]
    for e in (0, 1, k - 1, k, k + 1, cols):
        exp = list(range(e - 1, max(e - 1 - k, -1), -1))
        exp += [-1] * (k - len(exp))
        assert oracle.topk_rows(x, np.array([e], np.int32), k)[0].tolist() == exp, e
    # descending: 0..k-1
    x = -np.arange(cols, dtype=np.float32)[None]
    assert oracle.topk_rows(x, None, k)[0].tolist() == list(range(k))
    # all NaN: -1 everywhere
    x = np.full((1, cols), np.nan, np.float32)
    assert oracle.topk_rows(x, None, k)[0].tolist() == [-1] * k
    # more +inf than k: the first k +inf ids, ascending
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, cols)).astype(np.float32)
    pos = np.sort(rng.choice(cols, size=k + 20, replace=False))
    x[0, pos] = np.inf
    assert oracle.topk_rows(x, None, k)[0].tolist() == pos[:k].tolist()


def test_full_order_matches_stable_argsort():
    # k >= row length on distinct values: the whole row in descending order.
    rng = np.random.default_rng(5)
    x = rng.permutation(np.arange(-500, 500, dtype=np.float32) * 0.5)[None]
    got = oracle.topk_rows(x, None, 1000)[0]
    assert got.tolist() == np.argsort(-x[0], kind="stable").tolist()
    got = oracle.topk_rows(x, None, 1010)[0]
    assert got[:1000].tolist() == np.argsort(-x[0], kind="stable").tolist()
    assert got[1000:].tolist() == [-1] * 10


def test_signed_zero_and_infinities():
    x = np.array([[-0.0, 0.0, -0.0, 0.0, -np.inf, np.inf, np.nan]], np.float32)
    assert oracle.topk_rows(x, None, 7)[0].tolist() == [5, 1, 3, 0, 2, 4, -1]


def test_invariants_vs_torch_topk():
    torch = pytest.importorskip("torch")
    w = datagen.WORKLOADS["prefill"]
    x = datagen.logits(w, blocks=[0])[:256]
    ends = datagen.row_ends(w)[:256]
    k = w.k
    out = np.full((256, k + 9), 12345, np.int32)
    oracle.topk_rows(x, ends, k, out=out)
    assert (out[:, k:] == 12345).all(), "columns past k must stay untouched"
    got = out[:, :k]
    for i in range(0, 256, 17):
        e = int(ends[i])
        ids = got[i]
        assert (ids >= 0).all() and (ids < e).all()
        assert len(set(ids.tolist())) == k
        ref = torch.topk(torch.from_numpy(x[i, :e].copy()), k).values.numpy()
        assert np.array_equal(np.sort(x[i, ids]), np.sort(ref))
        # reported in descending score order
        assert (np.diff(x[i, ids]) <= 0).all()


def test_strided_input_and_output():
    rng = np.random.default_rng(9)
    big = rng.standard_normal((6, 50)).astype(np.float32)
    view = big[:, :37]            # ld = 50 > cols = 37
    ends = np.array([37, 10, 0, 36, 5, 37], np.int32)
    a = oracle.topk_rows(view, ends, 12)
    b = oracle.topk_rows(np.ascontiguousarray(view), ends, 12)
    assert np.array_equal(a, b)


def test_rejects_bad_arguments():
    x = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.topk_rows(x, None, 0)
