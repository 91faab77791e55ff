"""Host-side checks of the split-KV schedule definition (CPU only)."""
import numpy as np
import pytest

import mla_inputs as gen
from oracle import splitkv_schedule as S


def test_single_part_covers_everything():
    md, ns = S.schedule([3, 1, 5], 1, 2)
    assert list(md[:6]) == [1, 15, 2, 3, 9, S.MAGIC]
    assert list(md[8:13]) == [0, 0, 2, 5, 0]
    assert list(ns) == [0, 1, 2, 3]
    S.check_schedule(md, ns, [3, 1, 5])


def test_hand_worked_split():
    # units of 4 and 2 blocks, c0 = 1 -> total 8, P = 4, T = 2
    # positions: u0 overhead 0, blocks 1..4; u1 overhead 5, blocks 6..7
    # parts: p0 {u0b0}, p1 {u0b1,u0b2}, p2 {u0b3}, p3 {u1b0,u1b1}
    md, ns = S.schedule([4, 2], 4, 1)
    assert md[1] == 2
    rows = md[8:8 + 32].reshape(4, 8)[:, :5].tolist()
    assert rows == [[0, 0, 0, 1, 0], [0, 1, 0, 3, 1], [0, 3, 0, 4, 2], [1, 0, 1, 2, 0]]
    assert list(ns) == [0, 3, 4]


def test_empty_parts_and_units():
    md, ns = S.schedule([1, 1], 16, 2)
    S.check_schedule(md, ns, [1, 1])
    rows = md[8:8 + 128].reshape(16, 8)
    assert (rows[:, 0] >= 0).sum() == 2
    md, ns = S.schedule([], 8, 2)
    assert list(ns) == [0] and np.all(md[8:8 + 64:8] == -1)


@pytest.mark.parametrize("seed", range(30))
def test_random_schedules_valid_and_balanced(seed):
    rng = np.random.default_rng(seed)
    U = int(rng.integers(1, 200))
    n = [int(x) for x in rng.integers(1, 300, size=U)]
    P = int(rng.choice([1, 7, 8, 64, 256, 1024]))
    c0 = int(rng.integers(0, 4))
    md, ns = S.schedule(n, P, c0)
    S.check_schedule(md, ns, n)
    T = int(md[1])
    rows = md[8:8 + 8 * P].reshape(P, 8)
    for p in range(P):
        u0, j0, u1, j1 = rows[p, :4]
        if u0 < 0:
            continue
        blocks = sum((j1 if u == u1 else n[u]) - (j0 if u == u0 else 0) for u in range(u0, u1 + 1))
        pieces = u1 - u0 + 1
        assert blocks <= T
        assert blocks + c0 * pieces <= T + c0


def test_sparse_unit_blocks():
    idx = np.full((2, 2, 200), -1, dtype=np.int32)
    idx[0, 0, :5] = 3
    idx[0, 0, 150] = 7        # last valid at entry 150 -> 151 entries -> 3 blocks
    idx[0, 1, 199] = 1000     # out of range for L=50 -> no valid entry -> 1 block
    idx[1, 0, :64] = 1
    idx[1, 1, 64] = 0         # entry 64 valid -> 65 entries -> 2 blocks
    n = S.unit_blocks_sparse([50, 10], idx)
    assert list(n) == [3, 1, 1, 2]


def test_dense_unit_blocks():
    assert list(S.unit_blocks_dense([0, 1, 64, 65, 8192])) == [1, 1, 1, 2, 128]
