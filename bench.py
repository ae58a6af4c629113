"""Benchmark of the row top-K select on one MI355X.

Headline workload: top-512 of every row of a 4096 x 102400 fp32 logit matrix
(N(0,1), seed 105) with causal row ends row_end[i] = 98305 + i, the pages'
"very long rows" synthetic control.  One step = one topk_rows call over the
whole matrix, inputs resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--all] [--copy-calib]
                  [--counters NAME]

--all adds a "secondary" object with the other workloads: tiny, prefill,
ties, long, decode, the 8K x 8K distribution ablation, the headline shape in
bf16, the packed and pair merges with their row-major comparison, the merge's
second round and the owned-rows output (warm back-to-back timings, plus
cold-cache medians for the selects).  --copy-calib only runs a plain 1 GiB
device copy (the reference point for rocprofv3 FETCH_SIZE / WRITE_SIZE
scaling).  --counters NAME only runs one workload's measured call three times,
for rocprofv3 --pmc runs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0                  # MI355X HBM3E
PAGES_ROWS_PER_S = 4096 / 499.9e-6     # best published rate on this workload (GB200, context)
COUNTERS = os.path.join(ROOT, "profiles", "topk_rows_verylong_counters.json")
KERNEL_SOURCES = ["row_top_select_amd/csrc/rts_topk_rows.hip",
                  "row_top_select_amd/csrc/rts_device.hpp",
                  "row_top_select_amd/csrc/rts_levels.hpp"]


def log(*a):
    """Progress on stderr (the JSON line alone goes to stdout)."""
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(ends, k, rows, elem=4) -> int:
    # logits inside [0, row_end) + row_ends + k int32 ids per row
    return int(ends.astype("int64").sum()) * elem + rows * 4 + rows * k * 4


def time_calls(fn, steps, warmup, torch, per_call=None):
    """Wall time of `steps` back-to-back calls after `warmup`, and the mean
    per-call time from HIP events on the launch stream.  With a list as
    `per_call`, an event is recorded between consecutive calls too (the calls
    stay back to back) and each call's own time is appended to it."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True)
           for _ in range(steps + 1 if per_call is not None else 2)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        fn()
        if per_call is not None:
            evs[i + 1].record(stream)
    evs[-1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if per_call is not None:
        per_call.extend(evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(steps))
    return wall, evs[0].elapsed_time(evs[-1]) / 1e3 / steps


def spread(ts):
    """Median, min, max and mean of per-call times, in microseconds."""
    v = sorted(ts)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"median_us": med * 1e6, "min_us": v[0] * 1e6, "max_us": v[-1] * 1e6,
            "mean_us": sum(v) / n * 1e6, "calls": n}


_SCRUB = None


def time_cold_graph(fn, torch, rounds=4, calls=20, warmup=25):
    """Per-call times of one call captured in a HIP graph and replayed with the
    caches cold: before each replay a 1 GiB read-modify-write (larger than L2
    and the 256 MB Infinity Cache) runs on the same stream, outside the two
    events around the replay.  `warmup` replays, then `rounds` x `calls` timed."""
    global _SCRUB
    if _SCRUB is None:
        _SCRUB = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(rounds):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(calls)]
        for e0, e1 in evs:
            _SCRUB.add_(1.0)
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        ts.extend(e0.elapsed_time(e1) / 1e3 for e0, e1 in evs)
    del g
    return ts


def time_cold(fn, calls, torch):
    """Median per-call time with the caches cold: a 1 GiB read-modify-write
    (larger than L2 and the 256 MB Infinity Cache) runs before each timed call,
    which alone sits between two events on the launch stream."""
    global _SCRUB
    if _SCRUB is None:
        _SCRUB = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fn()
    ts = []
    for _ in range(calls):
        _SCRUB.add_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_graph(fn, steps, torch):
    """Per-call time of ``fn`` replayed from a HIP graph of ``steps`` calls: for
    kernels of a few microseconds, where launching from Python one call at a
    time would be what is measured."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                       # warm, outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / 1e3 / steps


def cpu_baseline(x_sample, ends_sample, k, total_rows_note):
    import oracle
    t0 = time.perf_counter()
    ids = oracle.topk_rows(x_sample, ends_sample, k)
    dt = time.perf_counter() - t0
    n = x_sample.shape[0]
    what = (f"all {n} rows" if n == total_rows_note else
            f"{n} of {total_rows_note} rows (rows 0..{n - 1})")
    return ids, {
        "value": n / dt,
        "unit": "rows/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"{what} of the same workload (same data and row ends), one run, {dt:.2f} s wall; "
                  f"host CPU {cpu_model()}; the plain full-sort oracle (each row's valid entries "
                  f"sorted with qsort, C -O2, OpenMP over rows), not a tuned CPU selector",
    }


def _median_runs(fn, runs=3):
    ts = []
    for i in range(runs + 1):                 # the first run warms up
        t0 = time.perf_counter()
        fn()
        if i:
            ts.append(time.perf_counter() - t0)
    ts.sort()
    return ts[len(ts) // 2]


def oracle_times(datagen):
    """The oracle (test infrastructure, CPU only) on every workload, on all of
    the host's threads (tiny and prefill also on one): wall-clock median of 3
    runs after 1 warm-up.  For the merges it times the select alone, on the
    oracle's own packed words and pairs of the merge workload."""
    import numpy as np
    import oracle
    cores = oracle.max_threads()
    res = {"cores": cores, "cpu": cpu_model(), "workloads": {}}
    for name in ("tiny", "prefill", "ties", "long", "decode", "robust", "robust_plus100",
                 "robust_scale1e8"):
        w = datagen.WORKLOADS[name]
        x = datagen.logits(w, threads=8)
        ends = datagen.row_ends(w)
        entry = {"shape": [w.rows, w.cols], "k": w.k}
        for threads in ((1, cores) if name in ("tiny", "prefill") else (cores,)):
            t = _median_runs(lambda: oracle.topk_rows(x, ends, w.k, nthreads=threads))
            entry[f"ms_{threads}_threads"] = t * 1e3
            entry[f"rows_per_s_{threads}_threads"] = w.rows / t
        res["workloads"][name] = entry
        log(f"oracle {name}: {entry}")
        del x
    W, N, K = datagen.MERGE_WORLD, datagen.MERGE_N, datagen.MERGE_K
    ranks32 = datagen.rank_slices(datagen.merge_global(threads=8), W)
    ranks16 = datagen.bf16_bits(ranks32)
    packed = np.stack([oracle.pack_candidates(ranks16[r], oracle.topk_rows(ranks16[r], None, N))
                       for r in range(W)])
    del ranks16
    t = _median_runs(lambda: oracle.merge_select_rank_major(packed, K))
    res["workloads"]["merge_packed_select"] = {"shape": list(packed.shape), "k": K,
                                               f"ms_{cores}_threads": t * 1e3,
                                               f"rows_per_s_{cores}_threads": packed.shape[1] / t}
    del packed
    pairs = np.stack([oracle.pack_pairs(ranks32[r], oracle.topk_rows(ranks32[r], None, K), r, W)
                      for r in range(W)])
    del ranks32
    t = _median_runs(lambda: oracle.merge_select_pairs_rank_major(pairs, K))
    res["workloads"]["merge_pairs_select"] = {"shape": list(pairs.shape), "k": K,
                                              f"ms_{cores}_threads": t * 1e3,
                                              f"rows_per_s_{cores}_threads": pairs.shape[1] / t}
    return res


def secondary(torch, rts, datagen, steps, warmup):
    import numpy as np
    res = {}
    # The measured configs, the pages' distribution ablation (8K x 8K: normal,
    # +100, *1e-8) and the headline shape in bf16.
    for name in ("tiny", "prefill", "ties", "long", "decode", "robust", "robust_plus100",
                 "robust_scale1e8", "verylong_bf16"):
        bf16 = name.endswith("_bf16")
        w = datagen.WORKLOADS[name[:-5] if bf16 else name]
        x_np = datagen.logits(w, threads=8)
        if bf16:
            x = torch.from_numpy(datagen.bf16_bits(x_np).view(np.int16)).cuda().view(torch.bfloat16)
        else:
            x = torch.from_numpy(x_np).cuda()
        del x_np
        ends_np = datagen.row_ends(w)
        ends = torch.from_numpy(ends_np).cuda()
        out = torch.empty((w.rows, w.k), dtype=torch.int32, device="cuda")
        ws_n = rts.topk_rows_workspace_size(x.dtype, w.rows, w.cols, w.k)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
        call = lambda: rts.topk_rows(x, w.k, row_ends=ends, out=out, workspace=ws if ws_n else None)
        _, t = time_calls(call, steps, warmup, torch)
        t_cold = time_cold(call, 9, torch)
        b = algorithmic_bytes(ends_np, w.k, w.rows, elem=2 if bf16 else 4)
        log(f"{name}: {t * 1e6:.1f} us warm, {t_cold * 1e6:.1f} us cold")
        res[name] = {"shape": [w.rows, w.cols], "k": w.k, "dtype": "bf16" if bf16 else "f32",
                     "us_per_call": t * 1e6, "rows_per_s": w.rows / t,
                     "algorithmic_GBps": b / t / 1e9, "cold_us_per_call": t_cold * 1e6,
                     "cold_algorithmic_GBps": b / t_cold / 1e9}
        del x
    # Packed merge (config of 8 simulated ranks) and the pair merge.
    W, R, S, N, K = (datagen.MERGE_WORLD, datagen.MERGE_ROWS, datagen.MERGE_LOCAL_COLS,
                     datagen.MERGE_N, datagen.MERGE_K)
    g = datagen.merge_global()
    ranks32 = datagen.rank_slices(g, W)
    del g
    x16 = torch.from_numpy(datagen.bf16_bits(ranks32).view(np.int16)).cuda().view(torch.bfloat16)
    gathered = torch.empty((W, R, N + N // 32), dtype=torch.int32, device="cuda")
    locs = [rts.topk_rows(x16[r], N) for r in range(W)]
    _, t_local = time_calls(lambda: rts.topk_rows(x16[0], N, out=locs[0]), steps, warmup, torch)
    _, t_pack = time_calls(lambda: rts.pack_candidates(x16[0], locs[0], out=gathered[0]), steps,
                           warmup, torch)
    for r in range(1, W):
        rts.pack_candidates(x16[r], locs[r], out=gathered[r])
    ids = torch.empty((R, K), dtype=torch.int32, device="cuda")
    sat = torch.empty((R,), dtype=torch.int32, device="cuda")
    _, t_sel = time_calls(lambda: rts.merge_select_rank_major(gathered, K, out=ids, sat_word=sat),
                          steps, warmup, torch)
    t_sel_cold = time_cold(lambda: rts.merge_select_rank_major(gathered, K, out=ids, sat_word=sat), 9,
                           torch)
    sel_bytes = W * R * (N + N // 32) * 4 + R * K * 4 + R * 4
    # The same words reordered row-major [R, W, n + n/32] (the dim-1 gather's
    # layout): the reorder copy, and the select reading that layout.
    grm = torch.empty((R, W, N + N // 32), dtype=torch.int32, device="cuda")
    _, t_copy = time_calls(lambda: grm.copy_(gathered.movedim(0, 1)), steps, warmup, torch)
    ids_rm = torch.empty_like(ids)
    sat_rm = torch.empty_like(sat)
    _, t_sel_rm = time_calls(lambda: rts.merge_select_row_major(grm, K, out=ids_rm, sat_word=sat_rm),
                             steps, warmup, torch)
    same = bool(torch.equal(ids_rm, ids) and torch.equal(sat_rm, sat))
    del grm, ids_rm, sat_rm
    # One rank's owned physical KV rows of the selection (64-token blocks, a
    # block table of 97 requests x 256 blocks).
    gen = torch.Generator().manual_seed(7)
    table = torch.stack([torch.randperm(1 << 18, generator=gen)[:256] for _ in range(97)]) \
        .to(torch.int32).cuda()
    req = (torch.arange(R, dtype=torch.int32) % 97).cuda()
    rows_out = torch.empty((R, K), dtype=torch.int32, device="cuda")
    valid = torch.empty((R,), dtype=torch.int32, device="cuda")
    _, t_emit = time_calls(lambda: rts.emit_rows(ids, W, 3, req, table, 64, 64, rows_out=rows_out,
                                                 valid_out=valid), steps, warmup, torch)
    emit_bytes = R * K * 4 * 2 + R * 8
    # The same rows straight from the select (no ids written or re-read).
    _, t_fused = time_calls(lambda: rts.merge_select_rank_major_rows(gathered, K, 3, req, table, 64, 64,
                                                                     rows_out=rows_out, valid_out=valid),
                            steps, warmup, torch)
    res["emit_rows"] = {"shape": [R, K], "world": W, "block_size": 64, "us_per_call": t_emit * 1e6,
                        "owned_rows_per_row": float(valid.float().mean()),
                        "algorithmic_GBps": emit_bytes / t_emit / 1e9,
                        "select_plus_emit_rows_us": (t_sel + t_emit) * 1e6,
                        "fused_select_rows_us": t_fused * 1e6}
    del rows_out, valid
    log(f"merge packed select {t_sel * 1e6:.1f} us, emit_rows {t_emit * 1e6:.1f} us")
    res["merge_packed"] = {"shape": [W, R, N + N // 32], "k": K,
                           "select_us": t_sel * 1e6, "select_rows_per_s": R / t_sel,
                           "select_algorithmic_GBps": sel_bytes / t_sel / 1e9,
                           "select_cold_us": t_sel_cold * 1e6,
                           "row_major_select_us": t_sel_rm * 1e6,
                           "reorder_copy_us": t_copy * 1e6,
                           "reorder_copy_plus_row_major_select_us": (t_copy + t_sel_rm) * 1e6,
                           "row_major_ids_identical": same,
                           "local_top384_bf16_us_per_rank": t_local * 1e6,
                           "pack_us_per_rank": t_pack * 1e6}
    # Second round.  On this workload no row saturates, so the rescue reads one
    # sat_word per row; on the rank-skewed variant most rows go through it.
    slots = (K - 1) // N
    recv = torch.zeros((R, slots, K + K // 32), dtype=torch.int32, device="cuda")
    t_fast = time_graph(lambda: rts.merge_rescue_rank_major(gathered, recv, sat, ids), 200, torch)
    del x16
    gs = datagen.skew_ranks(datagen.merge_global())
    x16 = torch.from_numpy(datagen.bf16_bits(datagen.rank_slices(gs, W)).view(np.int16)).cuda() \
        .view(torch.bfloat16)
    del gs
    for r in range(W):
        rts.pack_candidates(x16[r], rts.topk_rows(x16[r], N, out=locs[r]), out=gathered[r])
    rts.merge_select_rank_major(gathered, K, out=ids, sat_word=sat)
    local = torch.empty((R, K + K // 32), dtype=torch.int32, device="cuda")
    lk = torch.empty((R, K), dtype=torch.int32, device="cuda")
    for r in range(W):
        rts.pack_candidates(x16[r], rts.topk_rows(x16[r], K, out=lk), out=local)
        rts.rescue_push(local, r, W, N, sat, recv)
    t_push = time_graph(lambda: rts.rescue_push(local, W - 1, W, N, sat, recv), 100, torch)
    _, t_resc = time_calls(lambda: rts.merge_rescue_rank_major(gathered, recv, sat, ids), steps,
                           warmup, torch)
    n_sat = int(((sat.cpu().numpy().view(np.uint32) >> 16) != 0).sum())
    log(f"rescue {t_resc * 1e6:.1f} us")
    res["merge_rescue"] = {"shape": [W, R, N + N // 32], "recv": [R, slots, K + K // 32], "k": K,
                           "no_saturated_rows_us": t_fast * 1e6,
                           "rank_skewed_rows_saturated": n_sat,
                           "rank_skewed_rescue_us": t_resc * 1e6,
                           "rank_skewed_rescued_rows_per_s": n_sat / t_resc,
                           "rank_skewed_push_us_per_rank": t_push * 1e6}
    del x16, local, lk, recv
    x32 = torch.from_numpy(ranks32).cuda()
    pairs = torch.empty((W, R, K, 2), dtype=torch.int32, device="cuda")
    for r in range(W):
        rts.pack_pairs(x32[r], rts.topk_rows(x32[r], K), r, W, out=pairs[r])
    # A rank's local top-2048 (the pair merge's producer), fp32 and bf16.
    lk2 = torch.empty((R, K), dtype=torch.int32, device="cuda")
    _, t_l32 = time_calls(lambda: rts.topk_rows(x32[0], K, out=lk2), steps, warmup, torch)
    x16 = torch.from_numpy(datagen.bf16_bits(ranks32[0]).view(np.int16)).cuda().view(torch.bfloat16)
    del ranks32
    _, t_l16 = time_calls(lambda: rts.topk_rows(x16, K, out=lk2), steps, warmup, torch)
    del x16, lk2
    log(f"local top-2048 per rank: f32 {t_l32 * 1e6:.1f} us, bf16 {t_l16 * 1e6:.1f} us")
    pid = torch.empty((R, K), dtype=torch.int32, device="cuda")
    _, t_pairs = time_calls(lambda: rts.merge_select_pairs_rank_major(pairs, K, out=pid), steps,
                            warmup, torch)
    t_pairs_cold = time_cold(lambda: rts.merge_select_pairs_rank_major(pairs, K, out=pid), 9, torch)
    pb = W * R * K * 8 + R * K * 4
    del x32
    prm = torch.empty((R, W * K, 2), dtype=torch.int32, device="cuda")
    _, t_pcopy = time_calls(lambda: prm.view(R, W, K, 2).copy_(pairs.movedim(0, 1)), steps, warmup,
                            torch)
    pid_rm = torch.empty_like(pid)
    _, t_pairs_rm = time_calls(lambda: rts.merge_select_pairs_row_major(prm, K, W, out=pid_rm), steps,
                               warmup, torch)
    log(f"pair select {t_pairs * 1e6:.1f} us")
    res["merge_pairs"] = {"shape": [W, R, K, 2], "k": K, "select_us": t_pairs * 1e6,
                          "select_rows_per_s": R / t_pairs,
                          "select_algorithmic_GBps": pb / t_pairs / 1e9,
                          "select_cold_us": t_pairs_cold * 1e6,
                          "row_major_select_us": t_pairs_rm * 1e6,
                          "reorder_copy_us": t_pcopy * 1e6,
                          "reorder_copy_plus_row_major_select_us": (t_pcopy + t_pairs_rm) * 1e6,
                          "row_major_ids_identical": bool(torch.equal(pid_rm, pid)),
                          "local_top2048_f32_us_per_rank": t_l32 * 1e6,
                          "local_top2048_bf16_us_per_rank": t_l16 * 1e6}
    return res


COUNTER_WORKLOADS = ("tiny", "prefill", "ties", "long", "decode", "robust", "robust_plus100",
                     "robust_scale1e8", "verylong", "verylong_bf16", "merge_packed", "merge_pairs",
                     "local_top384_bf16", "local_top2048_f32", "local_top2048_bf16")


def counters_run(name, torch, rts, datagen, calls=3):
    """Only the measured call of one workload, `calls` times (for rocprofv3 --pmc runs)."""
    import numpy as np
    if name.startswith("local_top"):
        # one rank of the merge workload: [6710, 16384]
        k = int(name[len("local_top"):].split("_")[0])
        g = datagen.merge_global()
        r0 = np.ascontiguousarray(g[:, 0::datagen.MERGE_WORLD])
        del g
        if name.endswith("_bf16"):
            x = torch.from_numpy(datagen.bf16_bits(r0).view(np.int16)).cuda().view(torch.bfloat16)
        else:
            x = torch.from_numpy(r0).cuda()
        out = torch.empty((r0.shape[0], k), dtype=torch.int32, device="cuda")
        op = lambda: rts.topk_rows(x, k, out=out)
    elif name in ("merge_packed", "merge_pairs"):
        W, R, N, K = datagen.MERGE_WORLD, datagen.MERGE_ROWS, datagen.MERGE_N, datagen.MERGE_K
        g = datagen.merge_global()
        ranks32 = datagen.rank_slices(g, W)
        del g
        if name == "merge_packed":
            x = torch.from_numpy(datagen.bf16_bits(ranks32).view(np.int16)).cuda().view(torch.bfloat16)
            buf = torch.empty((W, R, N + N // 32), dtype=torch.int32, device="cuda")
            for r in range(W):
                rts.pack_candidates(x[r], rts.topk_rows(x[r], N), out=buf[r])
            op = lambda: rts.merge_select_rank_major(buf, K, out=ids, sat_word=sat)
            sat = torch.empty((R,), dtype=torch.int32, device="cuda")
        else:
            x = torch.from_numpy(ranks32).cuda()
            buf = torch.empty((W, R, K, 2), dtype=torch.int32, device="cuda")
            for r in range(W):
                rts.pack_pairs(x[r], rts.topk_rows(x[r], K), r, W, out=buf[r])
            op = lambda: rts.merge_select_pairs_rank_major(buf, K, out=ids)
        ids = torch.empty((R, K), dtype=torch.int32, device="cuda")
        del x
    else:
        bf16 = name.endswith("_bf16")
        w = datagen.WORKLOADS[name[:-5] if bf16 else name]
        x_np = datagen.logits(w, threads=8)
        if bf16:
            x = torch.from_numpy(datagen.bf16_bits(x_np).view(np.int16)).cuda().view(torch.bfloat16)
        else:
            x = torch.from_numpy(x_np).cuda()
        ends = torch.from_numpy(datagen.row_ends(w)).cuda()
        out = torch.empty((w.rows, w.k), dtype=torch.int32, device="cuda")
        ws_n = rts.topk_rows_workspace_size(x.dtype, w.rows, w.cols, w.k)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
        op = lambda: rts.topk_rows(x, w.k, row_ends=ends, out=out, workspace=ws if ws_n else None)
    torch.cuda.synchronize()
    for _ in range(calls):
        op()
    torch.cuda.synchronize()
    print(json.dumps({"counters_workload": name, "calls": calls}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--counters", choices=COUNTER_WORKLOADS,
                    help="only run one workload's measured call 3 times (for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}); rows shard across GPUs with no exchange, so run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calib:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "calls": 3}))
        return

    import datagen
    import row_top_select_amd as rts

    if args.counters:
        counters_run(args.counters, torch, rts, datagen)
        return

    w = datagen.WORKLOADS["verylong"]
    x_np = datagen.logits(w, threads=8)
    ends_np = datagen.row_ends(w)
    x = torch.from_numpy(x_np).cuda()
    ends = torch.from_numpy(ends_np).cuda()
    out = torch.empty((w.rows, w.k), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def step():
        rts.topk_rows(x, w.k, row_ends=ends, out=out, workspace=None)

    per_call = []
    wall, t_kernel = time_calls(step, args.steps, args.warmup, torch, per_call=per_call)
    ms_per_step = wall / args.steps * 1e3
    value = w.rows * args.steps / wall
    abytes = algorithmic_bytes(ends_np, w.k, w.rows)
    achieved = abytes / t_kernel / 1e9

    traffic = None
    if os.path.exists(COUNTERS):
        c = json.load(open(COUNTERS))
        if c.get("kernel_source_hash") == kernel_source_hash():
            traffic = c.get("hbm_bytes_per_launch")

    result = {
        "metric": "rows/s and achieved HBM GB/s, top-512 select at 4096×102400 fp32",
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": value / PAGES_ROWS_PER_S,
        "vs_baseline_note": "ratio to 4096 rows / 499.9 us, the best published figure on this "
                            "workload (DeepSelect on one GB200): context, another machine",
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "topk512_rows4096_cols102400_f32_causal", "rows": w.rows,
                   "cols": w.cols, "k": w.k, "row_ends": "98305+i", "distribution": "N(0,1)",
                   "seed": w.seed},
        "us_per_call": t_kernel * 1e6,
        "per_call": spread(per_call),
        "achieved_GBps": achieved,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes": abytes},
    }
    # The pages' protocol: one call in a graph, replayed with cold caches
    # (4 rounds x 20 calls after 25 warm-up replays); reported beside the
    # warm back-to-back figures above, which `value` is.
    cold = spread(time_cold_graph(step, torch))
    cold["algorithmic_GBps_at_median"] = abytes / (cold["median_us"] * 1e-6) / 1e9
    result["cold_graph_replay"] = cold
    if not args.no_cpu:
        # The whole workload is a few seconds of oracle time on the host's cores.
        ids, cpu = cpu_baseline(x_np, ends_np, w.k, w.rows)
        result["cpu_baseline"] = cpu
        result["parity_rows_equal"] = bool(np.array_equal(out.cpu().numpy(), ids))
    if args.all:
        del x
        torch.cuda.empty_cache()
        result["secondary"] = secondary(torch, rts, datagen, max(5, args.steps // 5), 2)
        if not args.no_cpu:
            result["secondary"]["cpu_oracle"] = oracle_times(datagen)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
