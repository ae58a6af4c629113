"""GPU parity of pack_candidates, merge_select_rank_major, pack_pairs and
merge_select_pairs_rank_major against the CPU oracle (bit-exact ids, words and
saturation words), on random and constructed inputs.  The merge workload at
full size is in test_gpu_merge_workload.py.

Inputs of the merge selects are built by the oracle (or by hand), never by the
GPU path."""

import numpy as np
import pytest

import brute
import datagen
import oracle
from gpu_common import assert_ids_equal, bf16_dev, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rts():
    import row_top_select_amd
    return row_top_select_amd


def test_pack_random(rts):
    rng = np.random.default_rng(11)
    for n in (32, 64, 96, 384):
        rows, cols = 37, int(rng.integers(100, 140000))
        x = datagen.bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
        x[rng.random((rows, cols)) < 0.02] = 0x7FC0
        idx = rng.integers(-3, cols + 5, size=(rows, n)).astype(np.int32)
        ends = rng.integers(-1, cols + 10, size=rows).astype(np.int32)
        for use_ends in (True, False):
            say("pack", n, cols, use_ends)
            e = ends if use_ends else None
            got = host(rts.pack_candidates(bf16_dev(x), dev(idx), row_ends=None if e is None else dev(e)))
            exp = oracle.pack_candidates(x, idx, e)
            assert_ids_equal(got, exp, f"pack n={n}")


def _gathered(rng, world, rows, n, fill=0.9, ties=False):
    g = np.zeros((world, rows, n + n // 32), np.uint32)
    for r in range(world):
        for t in range(rows):
            locs = rng.choice(1 << 17, size=n, replace=False)
            if ties:
                b = (rng.integers(0, 6, size=n) + 0x3F80).astype(np.uint16)
            else:
                b = datagen.bf16_bits(rng.standard_normal(n).astype(np.float32))
            keep = rng.random(n) < fill
            o = np.where(b & 0x8000, ~b.astype(np.uint32) & 0xFFFF, b.astype(np.uint32) | 0x8000)
            w = (o << 16) | (0xFFFF - (locs & 0xFFFF))
            g[r, t, :n] = np.where(keep, w, 0)
            hi = ((locs >> 16) & 1) & keep
            for j in np.nonzero(hi)[0]:
                g[r, t, n + j // 32] |= np.uint32(1 << (j % 32))
    return g.view(np.int32)


@pytest.mark.parametrize("world,n,k,fill,ties", [
    (8, 384, 2048, 1.0, False), (8, 384, 2048, 0.6, False), (8, 384, 2048, 1.0, True),
    (4, 64, 100, 0.9, False), (1, 32, 32, 1.0, False), (16, 256, 1024, 0.95, True),
    (3, 96, 2048, 0.8, False), (8, 2048, 512, 1.0, False)])
def test_merge_packed_random(rts, world, n, k, fill, ties):
    rng = np.random.default_rng(world * 1000 + n + k)
    g = _gathered(rng, world, 40, n, fill, ties)
    say("merge packed", world, n, k, fill, ties)
    ids, sat = rts.merge_select_rank_major(dev(g), k)
    eids, esat = oracle.merge_select_rank_major(g, k)
    assert_ids_equal(host(ids), eids, "ids")
    assert np.array_equal(host(sat), esat), "sat_word"


@pytest.mark.parametrize("world,n,k", [(8, 384, 2048), (3, 96, 500), (16, 64, 1024), (5, 2048, 2048)])
def test_merge_packed_row_major(rts, world, n, k):
    # [R, W, n + n/32] holds the same words as [W, R, n + n/32]: same ids and sat_word.
    rng = np.random.default_rng(world + n + k)
    g = _gathered(rng, world, 29, n, 0.9, ties=bool(world % 2))
    say("merge packed row-major", world, n, k)
    ids, sat = rts.merge_select_row_major(dev(np.ascontiguousarray(g.transpose(1, 0, 2))), k)
    eids, esat = oracle.merge_select_rank_major(g, k)
    assert_ids_equal(host(ids), eids, "ids")
    assert np.array_equal(host(sat), esat), "sat_word"


@pytest.mark.parametrize("world,kc,k", [(8, 2048, 2048), (3, 100, 77), (2, 2500, 1024)])
def test_merge_pairs_row_major(rts, world, kc, k):
    rng = np.random.default_rng(world * 3 + kc + k)
    rows = 21
    p = np.zeros((world, rows, kc, 2), np.int32)
    p[..., 0] = rng.standard_normal((world, rows, kc)).astype(np.float32).view(np.int32)
    for t in range(rows):                                  # distinct ids within a row
        p[:, t, :, 1] = rng.permutation(world * kc * 4)[:world * kc].reshape(world, kc)
    p[..., 1][rng.random((world, rows, kc)) < 0.05] = -1
    say("merge pairs row-major", world, kc, k)
    rm = np.ascontiguousarray(p.transpose(1, 0, 2, 3).reshape(rows, world * kc, 2))
    got = host(rts.merge_select_pairs_row_major(dev(rm), k, world))
    assert_ids_equal(got, oracle.merge_select_pairs_rank_major(p, k), "pair ids")


def test_merge_packed_saturation_constructed(rts):
    # rank 1 holds every top score: its bit is set, and the output matches the oracle
    world, s, n, k, rows = 8, 2048, 96, 512, 16
    rng = np.random.default_rng(4)
    gl = rng.standard_normal((rows, world * s)).astype(np.float32)
    gl[:, 1::world] += 10.0
    gb = datagen.bf16_bits(gl)
    ranks = datagen.rank_slices(gb, world)
    packed = np.stack([oracle.pack_candidates(ranks[r], oracle.topk_rows(ranks[r], None, n))
                       for r in range(world)])
    say("saturation")
    ids, sat = rts.merge_select_rank_major(dev(packed), k)
    eids, esat = oracle.merge_select_rank_major(packed, k)
    assert_ids_equal(host(ids), eids, "ids")
    assert np.array_equal(host(sat), esat)
    assert ((host(sat).view(np.uint32) >> 16) == 0b10).all()


def test_merge_packed_duplicates_stay_in_bounds(rts):
    # repeated words are outside the contract: only in-range, deterministic output is required
    rng = np.random.default_rng(6)
    world, n, k, rows = 4, 64, 128, 8
    g = _gathered(rng, world, rows, n, 1.0, True)
    g[1] = g[0]
    say("duplicates")
    out = torch.full((rows, k), 12345, dtype=torch.int32, device="cuda")
    ids, sat = rts.merge_select_rank_major(dev(g), k, out=out)
    a = host(ids)
    ids2, _ = rts.merge_select_rank_major(dev(g), k)
    assert np.array_equal(a, host(ids2))
    assert ((a >= -1) & (a < (1 << 17) * world)).all()


def test_pairs_random(rts):
    rng = np.random.default_rng(21)
    for world, kc, k in ((8, 2048, 2048), (4, 512, 512), (3, 100, 64), (2, 64, 1000), (16, 256, 1024),
                         (16, 2048, 2048), (1, 2048, 512), (5, 1000, 2048)):
        rows = 30
        p = np.zeros((world, rows, kc, 2), np.int32)
        v = rng.standard_normal((world, rows, kc)).astype(np.float32)
        v[rng.random(v.shape) < 0.01] = np.nan
        v[rng.random(v.shape) < 0.01] = -0.0
        v[rng.random(v.shape) < 0.01] = 0.0
        v[rng.random(v.shape) < 0.05] = 1.5          # ties on the score
        p[..., 0] = v.view(np.int32)
        gid = np.stack([rng.permutation(1 << 20)[:kc * world].reshape(world, kc) for _ in range(rows)],
                       axis=1)
        p[..., 1] = gid
        p[..., 1][rng.random(v.shape) < 0.05] = -1
        say("pairs", world, kc, k)
        got = host(rts.merge_select_pairs_rank_major(dev(p), k))
        exp = oracle.merge_select_pairs_rank_major(p, k)
        assert_ids_equal(got, exp, f"pairs {world} {kc} {k}")


@pytest.mark.parametrize("regime", ["all_equal", "eight_values", "quantized", "few_valid"])
def test_pairs_tie_regimes(rts, regime):
    # Score ties that fall on the k-th key in every regime the select handles
    # differently: a tie set of up to 64, a larger one, a boundary bin too full
    # for the LDS list (all scores equal), and rows with at most k valid.
    rng = np.random.default_rng(77)
    for world, kc, k in ((8, 2048, 2048), (4, 512, 512), (3, 100, 64)):
        rows = 12
        if regime == "all_equal":
            v = np.full((world, rows, kc), 0.75, np.float32)
        elif regime == "eight_values":
            v = rng.integers(0, 8, (world, rows, kc)).astype(np.float32)
        elif regime == "quantized":
            v = (np.round(rng.standard_normal((world, rows, kc)) * 300) / 300).astype(np.float32)
        else:
            v = rng.standard_normal((world, rows, kc)).astype(np.float32)
        p = np.zeros((world, rows, kc, 2), np.int32)
        p[..., 0] = v.view(np.int32)
        p[..., 1] = np.stack([rng.permutation(1 << 20)[:kc * world].reshape(world, kc)
                              for _ in range(rows)], axis=1)
        if regime == "few_valid":
            p[..., 1][rng.random(v.shape) < 1.0 - 0.8 * k / (world * kc)] = -1
        say("pairs ties", regime, world, kc, k)
        got = host(rts.merge_select_pairs_rank_major(dev(p), k))
        assert_ids_equal(got, oracle.merge_select_pairs_rank_major(p, k), f"pairs {regime} {world} {kc} {k}")


def test_pack_pairs_random(rts):
    rng = np.random.default_rng(31)
    rows, cols, kc = 50, 5000, 256
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[rng.random((rows, cols)) < 0.01] = np.nan
    idx = rng.integers(-2, cols + 3, size=(rows, kc)).astype(np.int32)
    ends = rng.integers(0, cols + 1, size=rows).astype(np.int32)
    say("pack pairs")
    got = host(rts.pack_pairs(dev(x), dev(idx), 3, 8, row_ends=dev(ends)))
    exp = oracle.pack_pairs(x, idx, 3, 8, ends)
    assert np.array_equal(got, exp)


# ---------------------------------------------------------------------------
# Second round (rescue) of the packed merge
# ---------------------------------------------------------------------------

def _sat_words(rng, rows, world, n, k, g):
    """Valid masks with tau16 taken from the row's words, empty masks, and masks
    that round 1 never writes (too many bits, a bit at or above world)."""
    slots = (k - 1) // n
    out = np.zeros(rows, np.uint32)
    gu = g.view(np.uint32)
    for t in range(rows):
        words = gu[:, t, :n].ravel()
        words = words[words != 0]
        tau = int(words[rng.integers(0, words.size)]) >> 16 if words.size and t % 3 else \
            int(rng.integers(0, 1 << 16))
        kind = t % 6
        if kind == 0:
            mask = 0
        elif kind == 4:
            mask = (1 << min(world, slots + 1)) - 1 if slots < world else 0
        elif kind == 5:
            mask = 1 << world
        else:
            nb = int(rng.integers(1, min(slots, world) + 1))
            mask = sum(1 << int(r) for r in rng.choice(world, size=nb, replace=False))
        out[t] = ((mask << 16) | tau) & 0xFFFFFFFF
    return out.view(np.int32)


@pytest.mark.parametrize("world,n,k,fill,ties", [
    (8, 384, 2048, 1.0, False), (8, 384, 2048, 0.7, True), (4, 64, 256, 0.9, False),
    (2, 32, 64, 1.0, False), (16, 256, 1024, 0.95, True), (3, 96, 2048, 0.8, False),
    (5, 32, 512, 1.0, True),
    # 48 and 64 candidate registers per thread (one workgroup per row)
    (16, 1024, 2048, 0.9, False), (16, 128, 2048, 1.0, True)])
def test_rescue_random(rts, world, n, k, fill, ties):
    rng = np.random.default_rng(world * 7919 + n + k)
    rows, slots = 48, (k - 1) // n
    g = _gathered(rng, world, rows, n, fill, ties)
    recv = np.ascontiguousarray(_gathered(rng, slots, rows, k, fill, ties).transpose(1, 0, 2))
    sw = _sat_words(rng, rows, world, n, k, g)
    ids0 = rng.integers(-1, 1 << 20, size=(rows, k)).astype(np.int32)
    say("rescue random", world, n, k, fill, ties)
    out = dev(ids0)
    rts.merge_rescue_rank_major(dev(g), dev(recv), dev(sw), out)
    exp = oracle.merge_rescue_rank_major(g, recv, sw, ids0)
    assert_ids_equal(host(out), exp, "rescued ids")


def test_rescue_many_rows(rts):
    # More rows than the strided grid reads in one batch (512 workgroups x 512
    # sat_words): the rows that enter lie in every batch, the rest stay as given.
    rng = np.random.default_rng(99)
    world, n, k, rows = 2, 32, 64, 270000
    hot = np.unique(np.concatenate([rng.choice(rows, 150, replace=False),
                                    [0, 511, 512, 262143, 262144, 262145, rows - 1]]))
    g = np.zeros((world, rows, n + n // 32), np.int32)
    g[:, hot] = _gathered(rng, world, len(hot), n, 0.9)
    recv = np.zeros((rows, 1, k + k // 32), np.int32)
    recv[hot] = _gathered(rng, 1, len(hot), k, 0.9).transpose(1, 0, 2)
    sw = np.zeros(rows, np.uint32)
    sw[hot] = ((1 + (hot % 2)) << 16) | 0x8000            # rank 0 or rank 1 saturated
    sw = sw.view(np.int32)
    ids0 = np.tile(np.arange(k, dtype=np.int32), (rows, 1))
    say("rescue many rows", rows, len(hot))
    out = dev(ids0)
    rts.merge_rescue_rank_major(dev(g), dev(recv), dev(sw), out)
    got = host(out)
    exp_hot = oracle.merge_rescue_rank_major(g[:, hot], recv[hot], sw[hot], ids0[hot])
    assert_ids_equal(got[hot], exp_hot, "rescued rows")
    cold = np.ones(rows, bool)
    cold[hot] = False
    assert np.array_equal(got[cold], ids0[cold]), "rows with an empty mask changed"


def test_rescue_push_random(rts):
    rng = np.random.default_rng(5)
    world, n, k, rows = 8, 384, 2048, 61
    slots = (k - 1) // n
    g = _gathered(rng, world, rows, n, 1.0)
    sw = _sat_words(rng, rows, world, n, k, g)
    local = rng.integers(-2**31, 2**31, size=(world, rows, k + k // 32)).astype(np.int32)
    recv_h = np.full((rows, slots, k + k // 32), 12345, np.int32)
    recv_d = dev(recv_h)
    ld = dev(local)
    swd = dev(sw)
    for r in range(world):
        say("rescue push rank", r)
        rts.rescue_push(ld[r], r, world, n, swd, recv_d)
        oracle.rescue_push(local[r], r, world, n, sw, recv_h)
    assert np.array_equal(host(recv_d), recv_h)


def test_rescue_limits(rts):
    g = torch.zeros((16, 4, 33), dtype=torch.int32, device="cuda")
    sw = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = torch.zeros((4, 2048), dtype=torch.int32, device="cuda")
    recv = torch.zeros((4, 63, 2112), dtype=torch.int32, device="cuda")
    # 16 * 32 + 16 * 2048 candidate slots exceed what one workgroup holds
    with pytest.raises(rts.RtsError) as e:
        rts.merge_rescue_rank_major(g, recv, sw, out)
    assert e.value.status == rts.RTS_EUNSUPPORTED
    # n >= k: no receive slot, nothing to do
    g2 = torch.zeros((2, 4, 66), dtype=torch.int32, device="cuda")
    out2 = torch.full((4, 64), 9, dtype=torch.int32, device="cuda")
    rts.merge_rescue_rank_major(g2, torch.zeros((4, 0, 66), dtype=torch.int32, device="cuda"),
                                torch.full((4,), 0x10000, dtype=torch.int32, device="cuda"), out2)
    assert (host(out2) == 9).all()


# ---------------------------------------------------------------------------
# emit_rows: a rank's owned physical KV rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("world,block_size,k,out_cols", [
    (8, 64, 2048, 2048), (8, 64, 512, 600), (3, 1, 37, 37), (1, 16, 64, 64), (16, 128, 1, 5),
    (5, 7, 1000, 1024)])
def test_emit_rows_random(rts, world, block_size, k, out_cols):
    rng = np.random.default_rng(world * 17 + block_size + k)
    rows, nreq, cols = 67, 9, 11
    table = rng.integers(0, 1 << 21, size=(nreq, cols)).astype(np.int32)
    table[1, :3] = 0x7FFFFFF0                      # wraps once scaled
    req = rng.integers(-2, nreq + 2, size=rows).astype(np.int32)
    ids = np.empty((rows, k), np.int32)
    for t in range(rows):
        ids[t] = rng.permutation(world * block_size * (cols + 3) + k)[:k]
    ids[rng.random((rows, k)) < 0.1] = -1
    stride = int(rng.integers(1, 1000))
    ids_d, req_d, tab_d = dev(ids), dev(req), dev(table)
    for rank in sorted({0, world - 1, world // 2}):
        say("emit_rows", world, block_size, k, out_cols, rank)
        rows_out = torch.full((rows, out_cols), 12345, dtype=torch.int32, device="cuda")
        _, valid = rts.emit_rows(ids_d, world, rank, req_d, tab_d, block_size, stride,
                                 rows_out=rows_out)
        e_rows, e_valid = oracle.emit_rows(ids, world, rank, req, table, block_size, stride, out_cols)
        assert_ids_equal(host(rows_out), e_rows, "rows_out")
        assert np.array_equal(host(valid), e_valid), "valid_out"


def test_emit_rows_strided_table(rts):
    # A block table that is a column slice of a wider one (row stride > columns).
    rng = np.random.default_rng(2)
    world, B, k, rows = 4, 32, 256, 40
    wide = rng.integers(0, 5000, size=(6, 20)).astype(np.int32)
    req = rng.integers(0, 6, size=rows).astype(np.int32)
    ids = np.stack([rng.permutation(world * B * 14)[:k] for _ in range(rows)]).astype(np.int32)
    tab_d = dev(wide)[:, :12]
    assert tab_d.stride(0) == 20
    rows_out, valid = rts.emit_rows(dev(ids), world, 1, dev(req), tab_d, B, B)
    e_rows, e_valid = oracle.emit_rows(ids, world, 1, req, wide[:, :12], B, B)
    assert_ids_equal(host(rows_out), e_rows, "rows_out")
    assert np.array_equal(host(valid), e_valid)


# ---------------------------------------------------------------------------
# Owned rows straight from the packed selects (fused emit_rows)
# ---------------------------------------------------------------------------

def _table(rng, nreq=7, cols=40):
    t = rng.integers(0, 1 << 20, size=(nreq, cols)).astype(np.int32)
    t[0, 0] = 0x7FFFFFF0
    return t


@pytest.mark.parametrize("world,n,k,B", [(8, 384, 2048, 64), (3, 96, 500, 16), (16, 64, 1024, 32),
                                         (4, 2048, 1024, 128), (8, 64, 96, 8)])
def test_merge_select_rows_fused(rts, world, n, k, B):
    rng = np.random.default_rng(world * 5 + n + k)
    rows = 37
    g = _gathered(rng, world, rows, n, 0.9, ties=bool(world % 2))
    table = _table(rng)
    req = rng.integers(-1, table.shape[0] + 1, size=rows).astype(np.int32)
    eids, esat = oracle.merge_select_rank_major(g, k)
    g_d, req_d, tab_d = dev(g), dev(req), dev(table)
    stride = int(rng.integers(1, 500))
    for rank in sorted({0, world - 1}):
        say("fused rows", world, n, k, B, rank)
        ids = torch.empty((rows, k), dtype=torch.int32, device="cuda")
        sat = torch.empty((rows,), dtype=torch.int32, device="cuda")
        rows_out = torch.full((rows, k + 3), 777, dtype=torch.int32, device="cuda")
        _, valid, _, _ = rts.merge_select_rank_major_rows(g_d, k, rank, req_d, tab_d, B, stride,
                                                          rows_out=rows_out, out_ids=ids, sat_word=sat)
        e_rows, e_valid = oracle.emit_rows(eids, world, rank, req, table, B, stride, k + 3)
        assert_ids_equal(host(rows_out), e_rows, "rows_out")
        assert np.array_equal(host(valid), e_valid), "valid_out"
        assert_ids_equal(host(ids), eids, "ids")
        assert np.array_equal(host(sat), esat), "sat_word"
        # rows only: ids and sat_word not requested
        r2, v2, _, _ = rts.merge_select_rank_major_rows(g_d, k, rank, req_d, tab_d, B, stride)
        assert_ids_equal(host(r2), e_rows[:, :k], "rows_out without ids")
        assert np.array_equal(host(v2), e_valid)


def test_merge_rescue_rows_fused(rts):
    world, n, k, B = 8, 384, 2048, 64
    rng = np.random.default_rng(21)
    rows, slots = 40, (k - 1) // n
    g = _gathered(rng, world, rows, n, 1.0)
    recv = np.ascontiguousarray(_gathered(rng, slots, rows, k, 0.95).transpose(1, 0, 2))
    sw = _sat_words(rng, rows, world, n, k, g)
    table = _table(rng, cols=300)
    req = rng.integers(0, table.shape[0], size=rows).astype(np.int32)
    ids0 = rng.integers(-1, 1 << 20, size=(rows, k)).astype(np.int32)
    e_ids = oracle.merge_rescue_rank_major(g, recv, sw, ids0)
    entered = e_ids.tolist() != ids0.tolist()
    swu = sw.view(np.uint32)
    mask = swu >> 16
    enter = (mask != 0) & ((mask >> world) == 0) & (np.array([bin(int(m)).count("1") for m in mask]) <= slots)
    for rank in (0, 5):
        say("fused rescue rows", rank)
        rows_out = torch.full((rows, k), 55, dtype=torch.int32, device="cuda")
        valid = torch.full((rows,), 66, dtype=torch.int32, device="cuda")
        ids = dev(ids0)
        rts.merge_rescue_rank_major_rows(dev(g), dev(recv), dev(sw), k, rank, dev(req), dev(table), B, B,
                                         rows_out, valid, out_ids=ids)
        e_rows, e_valid = oracle.emit_rows(e_ids, world, rank, req, table, B, B)
        got_rows, got_valid = host(rows_out), host(valid)
        assert_ids_equal(got_rows[enter], e_rows[enter], "rescued rows_out")
        assert np.array_equal(got_valid[enter], e_valid[enter])
        assert (got_rows[~enter] == 55).all() and (got_valid[~enter] == 66).all(), "rows that stay were written"
        assert_ids_equal(host(ids), e_ids, "rescued ids")
    assert entered


@pytest.mark.parametrize("world,n,k,rescue", [(3, 96, 64, False), (8, 2048, 1024, False),
                                              (3, 32, 64, True), (8, 64, 192, True)])
def test_repeated_words_rows_stay_in_bounds(rts, world, n, k, rescue):
    # Repeated words inside one rank (the same local id in many slots) are
    # outside the contract: more than k candidates can tie with the k-th
    # composite.  In round 1 (block kernel: world 3, or world * ceil(n/64) >
    # 64) rank 0 then owns n > out_cols selected candidates; in the second
    # round its receive slot holds k copies.  The fused rows outputs must stop
    # at out_cols: the guard rows around rows_out and valid_out stay untouched.
    rng = np.random.default_rng(world * 31 + n + k)
    rows, B = 6, 16
    g = _gathered(rng, world, rows, n, 1.0)
    top = np.int32((0xFE00 << 16) | (0xFFFF - 5) - (1 << 32))   # a huge score, local id 5
    g[0, :, :n] = top                              # rank 0: n copies of one candidate
    g[0, :, n:] = 0
    table = _table(rng, cols=(1 << 17) // B + 1)
    req = rng.integers(0, table.shape[0], size=rows).astype(np.int32)
    out_cols = k + 3
    guard = 424242
    buf = torch.full(((rows + 2) * out_cols,), guard, dtype=torch.int32, device="cuda")
    rows_out = buf[out_cols:(rows + 1) * out_cols].view(rows, out_cols)
    vbuf = torch.full((rows + 2,), guard, dtype=torch.int32, device="cuda")
    valid = vbuf[1:rows + 1]
    g_d, req_d, tab_d = dev(g), dev(req), dev(table)
    say("repeated words rows", world, n, k, rescue)
    if not rescue:
        rts.merge_select_rank_major_rows(g_d, k, 0, req_d, tab_d, B, B, rows_out=rows_out,
                                         valid_out=valid)
    else:
        slots = (k - 1) // n
        recv = np.ascontiguousarray(_gathered(rng, slots, rows, k, 1.0).transpose(1, 0, 2))
        recv[:, 0, :k] = top                       # slot 0 (owned by rank 0): k copies
        recv[:, 0, k:] = 0
        sw = np.full(rows, (1 << 16) | 0x7F00, np.uint32).view(np.int32)   # rank 0 saturated
        rts.merge_rescue_rank_major_rows(g_d, dev(recv), dev(sw), k, 0, req_d, tab_d, B, B,
                                         rows_out, valid)
    b, v = host(buf).reshape(rows + 2, out_cols), host(vbuf)
    assert (b[0] == guard).all() and (b[-1] == guard).all(), "rows_out written out of bounds"
    assert v[0] == guard and v[-1] == guard, "valid_out written out of bounds"
    assert ((v[1:-1] >= 0) & (v[1:-1] <= out_cols)).all()
    # the first valid_out entries of each row are physical rows, then -1
    for t in range(rows):
        assert (b[t + 1, v[t + 1]:] == -1).all()
