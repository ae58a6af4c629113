"""The merge workload at full size on the GPU, every row against the oracle.

Workload: global 6710 x 131072 N(0,1) logits; rank r owns the columns
g % 8 == r, a contiguous [8, 6710, 16384] block.
  * packed merge: per rank a local top-384 of the bf16 logits, packed into
    B' words [8, 6710, 396] (rank-major, read in place), global top-2048;
  * pair merge: per rank a local top-2048 of the fp32 logits as (score, gid)
    pairs [8, 6710, 2048, 2], global top-2048;
  * the second round on the rank-skewed variant (most rows saturate round 1);
  * one rank's owned physical KV rows, separately and fused into the select.

The oracle runs the whole pipeline on its own (its local top-N, pack and
select) for all 6710 rows; the GPU selects are also run on the oracle's
packed buffers, so each step is checked on inputs that did not come from the
GPU.  The last test runs the producer and the select on two streams ordered by
an event (the kernels page's module docstring: the merges of a step are
stream-ordered).
"""

import numpy as np
import pytest

import datagen
import oracle
from gpu_common import assert_ids_equal, bf16_dev, dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

W, R, S, N, K = (datagen.MERGE_WORLD, datagen.MERGE_ROWS, datagen.MERGE_LOCAL_COLS,
                 datagen.MERGE_N, datagen.MERGE_K)
BLOCK = 64      # tokens per KV block of the synthetic block table
NREQ = 97       # requests; row t belongs to request t % 97


@pytest.fixture(scope="module")
def rts():
    import row_top_select_amd
    return row_top_select_amd


@pytest.fixture(scope="module")
def ranks():
    say("merge workload: generate")
    g32 = datagen.merge_global(threads=8)
    r32 = datagen.rank_slices(g32, W)
    del g32
    return r32, datagen.bf16_bits(r32)


@pytest.fixture(scope="module")
def o_packed(ranks):
    """The oracle's packed merge, every row: local top-384, words, ids, sat_word."""
    _, r16 = ranks
    say("merge workload: oracle local top-384 + pack + select")
    locs = np.stack([oracle.topk_rows(r16[r], None, N) for r in range(W)])
    packed = np.stack([oracle.pack_candidates(r16[r], locs[r]) for r in range(W)])
    ids, sat = oracle.merge_select_rank_major(packed, K)
    return locs, packed, ids, sat


@pytest.fixture(scope="module")
def o_pairs(ranks):
    """The oracle's pair merge, every row: local top-2048, pairs, ids."""
    r32, _ = ranks
    say("merge workload: oracle local top-2048 + pairs + select")
    locs = np.stack([oracle.topk_rows(r32[r], None, K) for r in range(W)])
    pairs = np.stack([oracle.pack_pairs(r32[r], locs[r], r, W) for r in range(W)])
    return locs, pairs, oracle.merge_select_pairs_rank_major(pairs, K)


def _tables():
    rng = np.random.default_rng(77)
    table = np.stack([rng.permutation(200000)[:300] for _ in range(NREQ)]).astype(np.int32)
    # local ids past 200 * 64 have no block in the short table and drop out
    return table, np.ascontiguousarray(table[:, :200])


def test_packed_merge_every_row(rts, ranks, o_packed):
    locs, packed, eids, esat = o_packed
    _, r16 = ranks
    say("packed merge: gpu")
    x16 = bf16_dev(r16)
    gathered = torch.empty((W, R, N + N // 32), dtype=torch.int32, device="cuda")
    gl = []
    for r in range(W):
        loc = rts.topk_rows(x16[r], N)
        gl.append(loc)
        rts.pack_candidates(x16[r], loc, out=gathered[r])
    ids, sat = rts.merge_select_rank_major(gathered, K)
    rm_ids, rm_sat = rts.merge_select_row_major(gathered.movedim(0, 1).contiguous(), K)
    del x16
    say("packed merge: compare", R, "rows")
    for r in range(W):
        assert_ids_equal(host(gl[r]), locs[r], f"local top-{N} of rank {r}")
    assert np.array_equal(host(gathered), packed), "packed words"
    assert_ids_equal(host(ids), eids, "merged ids")
    assert np.array_equal(host(sat), esat), "sat_word"
    assert torch.equal(rm_ids, ids) and torch.equal(rm_sat, sat), "row-major packed select"
    # round 1 is exact on this workload: no rank saturates
    assert ((esat.view(np.uint32) >> 16) == 0).mean() > 0.99


def test_packed_select_on_oracle_words(rts, o_packed):
    # The select alone, on the oracle's words: rank-major and row-major.
    _, packed, eids, esat = o_packed
    say("packed select on oracle words")
    g = dev(packed)
    ids, sat = rts.merge_select_rank_major(g, K)
    assert_ids_equal(host(ids), eids, "ids")
    assert np.array_equal(host(sat), esat), "sat_word"
    ids2, sat2 = rts.merge_select_row_major(dev(np.ascontiguousarray(packed.transpose(1, 0, 2))), K)
    assert_ids_equal(host(ids2), eids, "row-major ids")
    assert np.array_equal(host(sat2), esat), "row-major sat_word"


def test_pair_merge_every_row(rts, ranks, o_pairs):
    locs, pairs, epids = o_pairs
    r32, _ = ranks
    say("pair merge: gpu")
    x32 = dev(r32)
    gp = torch.empty((W, R, K, 2), dtype=torch.int32, device="cuda")
    for r in range(W):
        loc = rts.topk_rows(x32[r], K)
        assert_ids_equal(host(loc), locs[r], f"local top-{K} of rank {r}")
        rts.pack_pairs(x32[r], loc, r, W, out=gp[r])
    del x32
    pids = rts.merge_select_pairs_rank_major(gp, K)
    rm = rts.merge_select_pairs_row_major(gp.movedim(0, 1).reshape(R, W * K, 2).contiguous(), K, W)
    say("pair merge: compare", R, "rows")
    assert np.array_equal(host(gp), pairs), "pairs"
    assert_ids_equal(host(pids), epids, "pair ids")
    assert torch.equal(rm, pids), "row-major pair select"
    del gp, rm
    # the select alone, on the oracle's pairs
    assert_ids_equal(host(rts.merge_select_pairs_rank_major(dev(pairs), K)), epids,
                     "pair select on oracle pairs")


def test_emit_rows_every_row(rts, o_packed):
    # Every rank's owned rows of the selection, separately (emit_rows) and
    # fused into the select, against the oracle's emit_rows of its own ids.
    _, packed, eids, _ = o_packed
    req = (np.arange(R) % NREQ).astype(np.int32)
    g = dev(packed)
    ids, _ = rts.merge_select_rank_major(g, K, want_sat=False)
    req_d = dev(req)
    for tab in _tables():
        tab_d = dev(tab)
        total = torch.zeros(R, dtype=torch.int64, device="cuda")
        for rank in range(W):
            say("emit_rows rank", rank, tab.shape)
            e_rows, e_valid = oracle.emit_rows(eids, W, rank, req, tab, BLOCK, BLOCK)
            rows_out, valid = rts.emit_rows(ids, W, rank, req_d, tab_d, BLOCK, BLOCK)
            assert_ids_equal(host(rows_out), e_rows, "rows_out")
            assert np.array_equal(host(valid), e_valid), "valid_out"
            f_rows, f_valid, _, _ = rts.merge_select_rank_major_rows(g, K, rank, req_d, tab_d,
                                                                     BLOCK, BLOCK)
            assert_ids_equal(host(f_rows), e_rows, "fused rows_out")
            assert np.array_equal(host(f_valid), e_valid), "fused valid_out"
            total += valid.long()
        inside = (((ids // W) // BLOCK) < tab.shape[1]).sum(dim=1)
        assert torch.equal(total, inside.long()), "the ranks do not partition the selected ids"


def test_rescue_every_row(rts):
    # Rank-skewed workload: round 1, every rank's local top-2048 packed and
    # pushed, the second round; the oracle runs the same pipeline on all rows.
    say("rescue workload: generate")
    g32 = datagen.skew_ranks(datagen.merge_global(threads=8))
    r16 = datagen.bf16_bits(datagen.rank_slices(g32, W))
    del g32
    slots = (K - 1) // N
    say("rescue workload: oracle")
    o_gathered = np.stack([oracle.pack_candidates(r16[r], oracle.topk_rows(r16[r], None, N))
                           for r in range(W)])
    o_ids1, o_sat = oracle.merge_select_rank_major(o_gathered, K)
    o_recv = np.zeros((R, slots, K + K // 32), np.int32)
    o_local = []
    for r in range(W):
        o_local.append(oracle.pack_candidates(r16[r], oracle.topk_rows(r16[r], None, K)))
        oracle.rescue_push(o_local[r], r, W, N, o_sat, o_recv)
    o_ids2 = oracle.merge_rescue_rank_major(o_gathered, o_recv, o_sat, o_ids1)
    masks = o_sat.view(np.uint32) >> 16
    assert (masks != 0).mean() > 0.5, "the skewed workload should saturate most rows"

    say("rescue workload: gpu")
    x16 = bf16_dev(r16)
    gathered = torch.empty((W, R, N + N // 32), dtype=torch.int32, device="cuda")
    for r in range(W):
        rts.pack_candidates(x16[r], rts.topk_rows(x16[r], N), out=gathered[r])
    ids, sat = rts.merge_select_rank_major(gathered, K)
    assert_ids_equal(host(ids), o_ids1, "round-1 ids")
    assert np.array_equal(host(sat), o_sat), "sat_word"
    recv = torch.zeros((R, slots, K + K // 32), dtype=torch.int32, device="cuda")
    local = torch.empty((R, K + K // 32), dtype=torch.int32, device="cuda")
    for r in range(W):
        rts.pack_candidates(x16[r], rts.topk_rows(x16[r], K), out=local)
        assert np.array_equal(host(local), o_local[r]), f"rank {r}'s packed local top-{K}"
        rts.rescue_push(local, r, W, N, sat, recv)
    del x16
    assert np.array_equal(host(recv), o_recv), "receive buffer"
    rts.merge_rescue_rank_major(gathered, recv, sat, ids)
    say("rescue workload: compare", R, "rows")
    assert_ids_equal(host(ids), o_ids2, "rescued ids")
    # the same second round on the oracle's buffers, fused with one rank's rows
    table, _ = _tables()
    req = (np.arange(R) % NREQ).astype(np.int32)
    e_rows, e_valid = oracle.emit_rows(o_ids2, W, 2, req, table, BLOCK, BLOCK)
    o1_rows, o1_valid = oracle.emit_rows(o_ids1, W, 2, req, table, BLOCK, BLOCK)
    ids_d = dev(o_ids1)
    rows_out, valid, _, _ = rts.merge_select_rank_major_rows(dev(o_gathered), K, 2, dev(req),
                                                             dev(table), BLOCK, BLOCK)
    assert_ids_equal(host(rows_out), o1_rows, "round-1 fused rows")
    rts.merge_rescue_rank_major_rows(dev(o_gathered), dev(o_recv), dev(o_sat), K, 2, dev(req),
                                     dev(table), BLOCK, BLOCK, rows_out, valid, out_ids=ids_d)
    assert_ids_equal(host(ids_d), o_ids2, "rescued ids on oracle buffers")
    assert_ids_equal(host(rows_out), e_rows, "rescued fused rows")
    assert np.array_equal(host(valid), e_valid), "rescued valid_out"
    assert np.array_equal(e_valid[masks == 0], o1_valid[masks == 0])


def test_stream_ordered_producer_and_select(rts, ranks, o_packed):
    # The local top-384 and pack of every rank run on stream A; the select runs
    # on stream B after an event recorded on A, enqueued right away (before A
    # has finished).  The result must equal the oracle's on every row.
    _, r16 = ranks
    _, _, eids, esat = o_packed
    x16 = bf16_dev(r16)
    gathered = torch.zeros((W, R, N + N // 32), dtype=torch.int32, device="cuda")
    locs = torch.empty((W, R, N), dtype=torch.int32, device="cuda")
    ids = torch.full((R, K), -7, dtype=torch.int32, device="cuda")
    sat = torch.zeros((R,), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    done = torch.cuda.Event()
    say("stream-ordered merge")
    for trial in range(3):
        gathered.zero_()
        torch.cuda.synchronize()
        for r in range(W):
            rts.topk_rows(x16[r], N, out=locs[r], stream=a)
            rts.pack_candidates(x16[r], locs[r], out=gathered[r], stream=a)
        done.record(a)
        b.wait_event(done)
        rts.merge_select_rank_major(gathered, K, out=ids, sat_word=sat, stream=b)
        b.synchronize()
        assert_ids_equal(host(ids), eids, f"ids (trial {trial})")
        assert np.array_equal(host(sat), esat), f"sat_word (trial {trial})"
