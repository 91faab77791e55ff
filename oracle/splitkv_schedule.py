"""Split-KV schedule, written as a plain sequential walk.

TEST INFRASTRUCTURE ONLY: the tests compare the device-built schedule with
this one bit for bit.  It shares no code with the HIP library.

topnet.top, "Was ist FlashMLA?", section "MLA-Metadaten abrufen" says the
decode needs metadata computed once from cache_seqlens and the number of query
rows per KV head, returned as `tile_scheduler_metadata` and `num_splits`, and
reused by every layer.  The pages say nothing about what the two hold; this is
the schedule this project defines for them:

  * a *unit* is one sequence (dense) or one (sequence, query token) pair
    (sparse, since each query token has its own index list);
  * unit u has n_u >= 1 blocks of 64 keys: ceil(L_b / 64) for dense, and for
    sparse ceil(E / 64) where E is one past the last index entry that lies
    in [0, L_b) (0 if none); a unit with no keys still gets one block so that
    its output (zero, lse = -inf) is written by someone;
  * every unit costs c0 extra (loading its queries and writing its result);
  * lay the units end to end on a line of cost positions: unit u starts at
    C_u = sum over v < u of (n_v + c0); its block j sits at C_u + c0 + j;
  * with P parts, T = ceil(total / P) (at least 1) and block (u, j) belongs to
    part floor(position / T).

The device arrays:
  tile_metadata = header[8] + P rows of 8 int32 + U int32
    header = [P, T, c0, U, total_blocks, 0x4D4C4131, 0, 0]
    row p  = [u_first, j_first, u_last, j_end, split_of_u_first,
              L_first, n_first, 0]
             (j_end is one past the last block of u_last in the part;
              L_first is cache_seqlens of u_first's sequence and n_first its
              block count n_{u_first}, carried so that a part can start its
              first unit without reading them; an empty part is
              [-1, 0, -1, 0, 0, 0, 0, 0])
    then n_u for every unit
  num_splits = U + 1 int32 prefix sums of k_u, the number of parts unit u
               is spread over.
"""
from __future__ import annotations

import numpy as np

PAGE = 64
MAGIC = 0x4D4C4131
HEADER = 8
ROW = 8


def unit_blocks_dense(seqlens) -> np.ndarray:
    return np.array([max(1, (int(L) + PAGE - 1) // PAGE) for L in seqlens], dtype=np.int64)


def unit_blocks_sparse(seqlens, indices) -> np.ndarray:
    b_, s_q, topk = indices.shape
    out = []
    for b in range(b_):
        L = int(seqlens[b])
        for s in range(s_q):
            last = -1
            for j in range(topk):
                t = int(indices[b, s, j])
                if 0 <= t < L:
                    last = j
            E = last + 1
            out.append(max(1, (E + PAGE - 1) // PAGE))
    return np.array(out, dtype=np.int64)


def schedule(n_blocks, num_parts: int, c0: int, unit_len=None):
    """Return (tile_metadata int32 array, num_splits int32 array).
    unit_len[u] is the cache length of unit u's sequence (0 if not given)."""
    n_blocks = [int(x) for x in n_blocks]
    U = len(n_blocks)
    P = int(num_parts)
    total = sum(n + c0 for n in n_blocks)
    T = max(1, -(-total // P)) if total > 0 else 1

    members = [[] for _ in range(P)]     # (u, j) pairs per part, in order
    pos = 0
    parts_of_unit = []
    for u, n in enumerate(n_blocks):
        pos += c0
        seen = []
        for j in range(n):
            p = pos // T
            members[p].append((u, j))
            if not seen or seen[-1] != p:
                seen.append(p)
            pos += 1
        parts_of_unit.append(seen)

    num_splits = np.zeros(U + 1, dtype=np.int32)
    for u in range(U):
        num_splits[u + 1] = num_splits[u] + len(parts_of_unit[u])

    md = np.zeros(HEADER + ROW * P + U, dtype=np.int32)
    md[HEADER + ROW * P:] = n_blocks
    md[:HEADER] = [P, T, c0, U, sum(n_blocks), MAGIC, 0, 0]
    for p in range(P):
        r = md[HEADER + ROW * p: HEADER + ROW * (p + 1)]
        if not members[p]:
            r[:] = [-1, 0, -1, 0, 0, 0, 0, 0]
            continue
        u0, j0 = members[p][0]
        u1, j1 = members[p][-1]
        split = parts_of_unit[u0].index(p)
        L0 = int(unit_len[u0]) if unit_len is not None else 0
        r[:] = [u0, j0, u1, j1 + 1, split, L0, n_blocks[u0], 0]
    return md, num_splits


def check_schedule(md, num_splits, n_blocks):
    """Validity of any schedule in this format: every (unit, block) is covered
    exactly once, parts are contiguous and in order, split indices and
    num_splits agree.  Raises AssertionError on a violation."""
    P, T, c0, U, total, magic = (int(v) for v in md[:6])
    assert magic == MAGIC and U == len(n_blocks) and total == int(sum(n_blocks))
    assert list(md[HEADER + ROW * P:]) == [int(x) for x in n_blocks]
    cover = {}
    split_seen = {}
    last = (-1, -1)
    for p in range(P):
        u0, j0, u1, j1, sp = (int(v) for v in md[HEADER + ROW * p: HEADER + ROW * p + 5])
        if u0 < 0:
            continue
        assert u0 <= u1
        assert int(md[HEADER + ROW * p + 6]) == int(n_blocks[u0])
        for u in range(u0, u1 + 1):
            jb = j0 if u == u0 else 0
            je = j1 if u == u1 else int(n_blocks[u])
            assert 0 <= jb < je <= n_blocks[u]
            assert (u, jb) > last
            for j in range(jb, je):
                assert (u, j) not in cover
                cover[(u, j)] = p
            last = (u, je - 1)
            idx = sp if u == u0 else 0
            split_seen.setdefault(u, []).append(idx)
    for u in range(U):
        for j in range(int(n_blocks[u])):
            assert (u, j) in cover, (u, j)
        k = int(num_splits[u + 1]) - int(num_splits[u])
        assert split_seen[u] == list(range(k)), (u, split_seen[u], k)
    return True
