"""Pins of the oracle's emit_rows (a rank's owned physical KV rows of the
selected ids) to facts outside it:

* a hand-worked example of the definition (tests/golden/emit_rows_small.json);
* pure-Python brute force (tests/brute.py) on random tables, requests and ids,
  with out-of-range requests, blocks past the table and int32 wrap;
* closed form: with the identity block table (block q*nb + b, stride = block
  size) the physical row is req * nb * B + gid // W;
* partition: over all ranks the owned rows are exactly the selected ids whose
  block lies inside the table.
"""

import json
import os

import numpy as np
import pytest

import brute
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_emit_rows():
    gd = json.load(open(os.path.join(GOLDEN, "emit_rows_small.json")))
    for rank, exp in gd["expected"].items():
        rows_out, valid = oracle.emit_rows(np.array(gd["ids"]), gd["world"], int(rank),
                                           np.array(gd["req_id"]), np.array(gd["block_table"]),
                                           gd["block_size"], gd["stride_rows"])
        assert rows_out.tolist() == exp["rows_out"], rank
        assert valid.tolist() == exp["valid_out"], rank


@pytest.mark.parametrize("world,block_size,k,out_cols", [(8, 64, 64, 64), (3, 1, 40, 50), (1, 16, 32, 33),
                                                         (16, 128, 96, 96)])
def test_emit_rows_brute_force(world, block_size, k, out_cols):
    rng = np.random.default_rng(world * 31 + block_size + k)
    rows, nreq, cols = 23, 5, 7
    table = rng.integers(0, 1 << 20, size=(nreq, cols)).astype(np.int32)
    table[0, 0] = 0x7FFFFFF0                       # wraps once scaled
    req = rng.integers(-1, nreq + 1, size=rows).astype(np.int32)
    ids = np.empty((rows, k), np.int32)
    for t in range(rows):
        ids[t] = rng.permutation(world * block_size * (cols + 2) + k)[:k]
    ids[rng.random((rows, k)) < 0.1] = -1
    stride = int(rng.integers(1, 300))
    for rank in range(world):
        rows_out, valid = oracle.emit_rows(ids, world, rank, req, table, block_size, stride, out_cols)
        for t in range(rows):
            exp, cnt = brute.emit_rows_row(ids[t].tolist(), world, rank, int(req[t]), table.tolist(),
                                           block_size, stride, out_cols)
            assert rows_out[t].tolist() == exp, (rank, t)
            assert valid[t] == cnt


def test_emit_rows_identity_table_closed_form():
    world, B, nb, k, rows = 4, 16, 10, 64, 9
    nreq = 3
    table = np.arange(nreq * nb, dtype=np.int32).reshape(nreq, nb)
    rng = np.random.default_rng(3)
    req = rng.integers(0, nreq, size=rows).astype(np.int32)
    ids = np.stack([rng.permutation(world * B * nb)[:k] for _ in range(rows)]).astype(np.int32)
    for rank in range(world):
        rows_out, valid = oracle.emit_rows(ids, world, rank, req, table, B, B)
        for t in range(rows):
            own = [g for g in ids[t] if g % world == rank]
            assert valid[t] == len(own)
            assert rows_out[t, :len(own)].tolist() == [int(req[t]) * nb * B + g // world for g in own]
            assert (rows_out[t, len(own):] == -1).all()


def test_emit_rows_partition_over_ranks():
    world, B, cols, k, rows = 8, 32, 5, 128, 12
    rng = np.random.default_rng(8)
    table = np.stack([rng.permutation(1000)[:cols] for _ in range(4)]).astype(np.int32)
    req = rng.integers(0, 4, size=rows).astype(np.int32)
    ids = np.stack([rng.permutation(world * B * (cols + 1))[:k] for _ in range(rows)]).astype(np.int32)
    total = np.zeros(rows, np.int64)
    for rank in range(world):
        _, valid = oracle.emit_rows(ids, world, rank, req, table, B, B)
        total += valid
    inside = ((ids // world) // B < cols).sum(axis=1)
    assert np.array_equal(total, inside)


def test_emit_rows_rejects_bad_arguments():
    ids = np.zeros((2, 4), np.int32)
    with pytest.raises(Exception):
        oracle.emit_rows(ids, 2, 2, np.zeros(2), np.zeros((1, 1)), 4, 1)       # rank >= world
    with pytest.raises(Exception):
        oracle.emit_rows(ids, 2, 0, np.zeros(2), np.zeros((1, 1)), 4, 1, out_cols=3)
