"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
selection arithmetic.  Every matrix is generated in blocks of 1024 rows, block
``b`` from ``numpy.random.Generator(PCG64(SeedSequence([seed, b])))``, so any
subset of row blocks can be regenerated on its own (the benchmark's CPU sample
and the full-size parity samples rely on that).

Workloads (shapes and distributions of the pages' synthetic controls: normal
random fp32 logits, top-k 512, causal row bounds ``row_end[i] = cols - rows + i + 1``):

=========  ====  ============================  ==================  ====
name       seed  shape / values                row_ends            K
=========  ====  ============================  ==================  ====
tiny       101   64 x 8192, N(0,1)             all 8192            512
prefill    102   4096 x 8192, N(0,1)           4097 + i            512
ties       103   4096 x 8192, integers [0,63]  4097 + i            512
long       104   2048 x 51200, N(0,1) with     49153 + i           512
                 0.1% +inf, 0.1% -inf, 0.05% NaN
verylong   105   4096 x 102400, N(0,1)         98305 + i           512
decode     106   64 x 102400, N(0,1)           all 102400          512
merge      107   global 6710 x 131072 N(0,1);  none                2048
                 rank r owns columns g % 8 == r
merge_     107   merge + 4.0 on the tokens of  none                2048
 skew            t % 7 ranks of row t (the
                 rescue round's input)
robust     108   8192 x 8192, N(0,1)           i + 1               512
robust_    108   the same values + 100         i + 1               512
 plus100
robust_    108   the same values * 1e-8        i + 1               512
 scale1e8
=========  ====  ============================  ==================  ====

The three ``robust`` workloads are the pages' distribution ablation at 8K
queries x 8K keys (one base matrix, shifted or scaled in fp32).  The headline
shape in bf16 is ``verylong`` rounded with ``bf16_bits``.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK_ROWS = 1024


def rng(seed: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, block])))


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    rows: int
    cols: int
    k: int
    kind: str          # "normal", "ties", "specials", "plus100", "scale1e8"
    causal: bool       # row_end[i] = cols - rows + i + 1, else full rows


WORKLOADS = {
    "tiny": Workload("tiny", 101, 64, 8192, 512, "normal", False),
    "prefill": Workload("prefill", 102, 4096, 8192, 512, "normal", True),
    "ties": Workload("ties", 103, 4096, 8192, 512, "ties", True),
    "long": Workload("long", 104, 2048, 51200, 512, "specials", True),
    "verylong": Workload("verylong", 105, 4096, 102400, 512, "normal", True),
    "decode": Workload("decode", 106, 64, 102400, 512, "normal", False),
    "robust": Workload("robust", 108, 8192, 8192, 512, "normal", True),
    "robust_plus100": Workload("robust_plus100", 108, 8192, 8192, 512, "plus100", True),
    "robust_scale1e8": Workload("robust_scale1e8", 108, 8192, 8192, 512, "scale1e8", True),
}

MERGE_SEED = 107
MERGE_ROWS = 6710
MERGE_WORLD = 8
MERGE_LOCAL_COLS = 16384          # 131072 / 8
MERGE_N = 384                     # local top-N of the packed merge
MERGE_K = 2048


def _fill_block(w: Workload, b: int) -> np.ndarray:
    r0 = b * BLOCK_ROWS
    nr = min(BLOCK_ROWS, w.rows - r0)
    g = rng(w.seed, b)
    if w.kind == "ties":
        return g.integers(0, 64, size=(nr, w.cols)).astype(np.float32)
    x = g.standard_normal(size=(nr, w.cols), dtype=np.float32)
    if w.kind == "specials":
        u = g.random(size=(nr, w.cols), dtype=np.float32)
        x[u < 0.001] = np.inf
        x[(u >= 0.001) & (u < 0.002)] = -np.inf
        x[(u >= 0.002) & (u < 0.0025)] = np.nan
    elif w.kind == "plus100":
        x += np.float32(100.0)
    elif w.kind == "scale1e8":
        x *= np.float32(1e-8)
    return x


def row_ends(w: Workload) -> np.ndarray:
    i = np.arange(w.rows, dtype=np.int64)
    if w.causal:
        return (w.cols - w.rows + i + 1).astype(np.int32)
    return np.full(w.rows, w.cols, dtype=np.int32)


def logits(w: Workload, blocks=None, threads: int = 4) -> np.ndarray:
    """fp32 [rows, cols] for ``w`` (or only the listed 1024-row blocks, stacked)."""
    nblocks = (w.rows + BLOCK_ROWS - 1) // BLOCK_ROWS
    blocks = list(range(nblocks)) if blocks is None else list(blocks)
    sizes = [min(BLOCK_ROWS, w.rows - b * BLOCK_ROWS) for b in blocks]
    out = np.empty((sum(sizes), w.cols), dtype=np.float32)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)

    def work(t):
        out[offs[t]:offs[t + 1]] = _fill_block(w, blocks[t])

    if threads > 1 and len(blocks) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(len(blocks))))
    else:
        for t in range(len(blocks)):
            work(t)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_u.size, step):
        c = flat_u[i:i + step]
        # uint32 arithmetic: no non-NaN pattern can carry past bit 31
        r = ((c + np.uint32(0x7FFF) + ((c >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
        nan = (c & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r[nan] = ((c[nan] >> 16) | np.uint32(0x0040)).astype(np.uint16)
        flat_o[i:i + step] = r
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def merge_global(rows: int = MERGE_ROWS, blocks=None, cols: int = MERGE_WORLD * MERGE_LOCAL_COLS,
                 seed: int = MERGE_SEED, threads: int = 4) -> np.ndarray:
    """Global fp32 logits [rows, cols] of the merge workload (row blocks of 1024)."""
    w = Workload("merge", seed, rows, cols, MERGE_K, "normal", False)
    return logits(w, blocks=blocks, threads=threads)


MERGE_SKEW_SHIFT = 4.0


def skew_ranks(g: np.ndarray, world: int = MERGE_WORLD, shift: float = MERGE_SKEW_SHIFT) -> np.ndarray:
    """Rank-skewed variant of global logits [R, world * S], in place: in row t
    the m = t % 7 ranks (t + 3 j) % world, j < m, get ``shift`` added to every
    token they own, so their local top lists outrank everyone else's and the
    rows with 1 <= m <= 5 saturate round 1 of the packed merge."""
    for t in range(g.shape[0]):
        for j in range(t % 7):
            g[t, (t + 3 * j) % world::world] += np.float32(shift)
    return g


def rank_slices(g: np.ndarray, world: int = MERGE_WORLD) -> np.ndarray:
    """[R, world * S] -> contiguous [world, R, S]: rank r owns global column c iff c % world == r."""
    return np.ascontiguousarray(np.stack([g[:, r::world] for r in range(world)]))
