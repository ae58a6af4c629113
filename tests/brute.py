"""Pure-Python brute force for tiny inputs, written independently of oracle/.

Each function restates a definition from the pages with Python tuple sorts and
explicit loops; the oracle tests compare the C oracle against these.
"""

import math
import struct


def f32_of_bits(u):
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bits_of_f32(v):
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bf16_value(b):
    return f32_of_bits((b & 0xFFFF) << 16)


def order_key(v, ident):
    """Sort key for (score desc, -0 below +0, id asc)."""
    return (-v, 1 if math.copysign(1.0, v) < 0 and v == 0 else 0, ident)


def topk_row(values, end, k):
    """values: list of Python floats (NaN allowed); returns k ids (-1 padded)."""
    e = max(0, min(end, len(values)))
    cands = [(order_key(values[j], j), j) for j in range(e) if not math.isnan(values[j])]
    cands.sort()
    ids = [j for _, j in cands[:k]]
    return ids + [-1] * (k - len(ids))


def ord16(b):
    b &= 0xFFFF
    return (~b & 0xFFFF) if b & 0x8000 else (b | 0x8000)


def pack_row(bf16_row, local_ids, end, n):
    """One B' row (n words + n/32 plane words) as Python ints (uint32 values)."""
    lim = min(end, len(bf16_row), 1 << 17)
    words = [0] * n
    plane = [0] * (n // 32)
    for j in range(n):
        loc = local_ids[j]
        if 0 <= loc < lim:
            b = bf16_row[loc]
            if (b & 0x7FFF) <= 0x7F80:
                words[j] = (ord16(b) << 16) | (0xFFFF - (loc & 0xFFFF))
                if (loc >> 16) & 1:
                    plane[j // 32] |= 1 << (j % 32)
    return words + plane


def merge_row(gathered_row, world, n, k):
    """gathered_row[r] = list of n + n/32 uint32 words of rank r for one row.

    Returns (ids in candidate order + -1 tail, sat_word as uint32)."""
    cands = []
    for r in range(world):
        row = gathered_row[r]
        for j in range(n):
            w = row[j] & 0xFFFFFFFF
            if w == 0:
                continue
            hi = (row[n + j // 32] >> (j % 32)) & 1
            local = (0xFFFF - (w & 0xFFFF)) | (hi << 16)
            gid = local * world + r
            cands.append(((-(w >> 16), gid, r * n + j), gid, w >> 16, r * n + j))
    cands.sort()
    chosen = cands[:k]
    tau = chosen[-1][2] if len(cands) >= k else 0
    by_pos = sorted((pos, gid) for _, gid, _, pos in chosen)
    ids = [gid for _, gid in by_pos] + [-1] * (k - len(chosen))
    mask = 0
    for r in range(world):
        row = gathered_row[r]
        if all((row[j] & 0xFFFFFFFF) != 0 and ((row[j] & 0xFFFFFFFF) >> 16) > tau for j in range(n)):
            mask |= 1 << r
    if bin(mask).count("1") > (k - 1) // n:
        mask = 0
    return ids, ((mask << 16) | tau) & 0xFFFFFFFF


def merge_pairs_row(pairs_row, world, kc, k):
    """pairs_row[r][j] = (score bits, gid).  Returns ids in candidate order + -1 tail."""
    cands = []
    for r in range(world):
        for j in range(kc):
            sbits, gid = pairs_row[r][j]
            v = f32_of_bits(sbits)
            if gid < 0 or math.isnan(v):
                continue
            cands.append((order_key(v, gid) + (r * kc + j,), gid, r * kc + j))
    cands.sort()
    chosen = sorted((pos, gid) for _, gid, pos in cands[:k])
    return [gid for _, gid in chosen] + [-1] * (k - len(chosen))


def _decode(words, plane_base, j, rank, world):
    """(ord16, gid) of slot j of a packed list; plane words start at plane_base."""
    w = words[j] & 0xFFFFFFFF
    hi = (words[plane_base + j // 32] >> (j % 32)) & 1
    return w >> 16, ((0xFFFF - (w & 0xFFFF)) | (hi << 16)) * world + rank


def push_row(recv_row, local_row, rank, world, n, k, sat_word):
    """In place: rank's packed local top-k into its slot when the row is rescued."""
    mask = (sat_word & 0xFFFFFFFF) >> 16
    if mask == 0 or mask >> world or bin(mask).count("1") > (k - 1) // n:
        return
    if (mask >> rank) & 1:
        recv_row[bin(mask & ((1 << rank) - 1)).count("1")] = list(local_row)


def rescue_row(gathered_row, recv_row, world, n, k, sat_word, ids_row):
    """Second round of the packed merge for one row.

    gathered_row[r]: rank r's n + n/32 round-1 words; recv_row[s]: receive slot
    s (k + k/32 words, owned by the s-th saturated rank).  Returns the row's
    ids: unchanged unless the mask is nonzero, below 1 << world and has at most
    (k-1)//n bits."""
    sw = sat_word & 0xFFFFFFFF
    mask, tau = sw >> 16, sw & 0xFFFF
    if mask == 0 or mask >> world or bin(mask).count("1") > (k - 1) // n:
        return list(ids_row)
    cands = []
    for r in range(world):
        if (mask >> r) & 1:
            continue
        for j in range(n):
            if gathered_row[r][j] & 0xFFFFFFFF == 0:
                continue
            o, gid = _decode(gathered_row[r], n, j, r, world)
            if o >= tau:
                cands.append((-o, gid, r * n + j))
    owners = [r for r in range(world) if (mask >> r) & 1]
    for s, r in enumerate(owners):
        for j in range(k):
            if recv_row[s][j] & 0xFFFFFFFF == 0:
                continue
            o, gid = _decode(recv_row[s], k, j, r, world)
            cands.append((-o, gid, world * n + s * k + j))
    cands.sort()
    chosen = sorted((pos, gid) for _, gid, pos in cands[:k])
    return [gid for _, gid in chosen] + [-1] * (k - len(chosen))


def emit_rows_row(ids_row, world, dcp_rank, req, table, block_size, stride_rows, out_cols):
    """One row of a rank's owned physical KV rows: (rows list padded with -1, count).
    ``table`` is the list of block-table rows (lists of block ids)."""
    out = []
    if 0 <= req < len(table):
        for gid in ids_row:
            if gid < 0 or gid % world != dcp_rank:
                continue
            local = gid // world
            b, off = divmod(local, block_size)
            if b < len(table[req]):
                v = (table[req][b] * stride_rows + off) & 0xFFFFFFFF
                out.append(v - (1 << 32) if v >= 1 << 31 else v)
    return out + [-1] * (out_cols - len(out)), len(out)
