"""Pins of the oracle's grouping of slots by expert and its byte counts.

Grouping (the deduplicating kernel "groups the pass's tokens by expert", Lan,
Section 1) is pinned by brute force over every valid id array of a small case
against an independent formulation (a sort of (id, slot) pairs) plus structural
invariants; bytes by their closed forms n m w and X(n) w (Section 1, "Bytes").
"""
import itertools

import numpy as np

import oracle


def _check_grouping(ids, N):
    st, count, offset, sbe, distinct, U = oracle.route_group(ids, N)
    flat = ids.reshape(-1)
    nm = flat.size
    valid = [s for s in range(nm) if 0 <= flat[s] < N]
    # independent formulation: sort (id, slot) pairs
    want = [s for _, s in sorted((int(flat[s]), s) for s in valid)]
    assert list(sbe[:len(want)]) == want
    assert all(v == -1 for v in sbe[len(want):])
    assert offset[0] == 0 and offset[N] == len(valid)
    for e in range(N):
        assert count[e] == sum(1 for s in valid if flat[s] == e)
        assert offset[e + 1] - offset[e] == count[e]
        assert all(flat[s] == e for s in sbe[offset[e]:offset[e + 1]])
    present = sorted(set(int(flat[s]) for s in valid))
    assert U == len(present)
    assert list(distinct[:U]) == present and all(v == -1 for v in distinct[U:])
    return st, U


def test_grouping_brute_force_all_valid_arrays():
    N, m, n = 4, 2, 3
    pairs = [p for p in itertools.permutations(range(N), m)]  # ordered, distinct within a token
    total_u = 0
    for rows in itertools.product(pairs, repeat=n):
        ids = np.array(rows, np.int32)
        st, U = _check_grouping(ids, N)
        assert st == oracle.OR_OK
        assert m <= U <= min(n * m, N)
        total_u += U
    # mean union under uniform independent sets: N (1 - q^n), q = 1 - m/N
    assert total_u * 2 == len(pairs) ** n * 7  # 4 (1 - (1/2)^3) = 7/2


def test_grouping_invalid_ids():
    N = 5
    ids = np.array([[0, 7], [3, -1], [2, 2]], np.int32)
    st, U = _check_grouping(ids, N)
    assert st == oracle.OR_E_IDS and U == 3
    st, U = _check_grouping(np.array([[1, 1]], np.int32), N)
    assert st == oracle.OR_E_IDS and U == 1


def test_grouping_random_larger():
    rng = np.random.default_rng(0)
    for N, m, n in [(64, 6, 8), (128, 8, 32), (8, 2, 8)]:
        for _ in range(20):
            ids = np.stack([rng.choice(N, m, replace=False) for _ in range(n)]).astype(np.int32)
            st, U = _check_grouping(ids, N)
            assert st == oracle.OR_OK and m <= U <= min(n * m, N)
            assert U / (n * m) >= 1 / n  # distinct share in [1/n, 1]


def test_bytes_closed_forms():
    rng = np.random.default_rng(1)
    N, m, d, d_ff = 64, 6, 2048, 1408
    w = 3 * d * d_ff * 2
    assert w == 17_301_504
    for n in range(1, 9):
        ids = np.stack([rng.choice(N, m, replace=False) for _ in range(n)]).astype(np.int32)
        slot = oracle.bytes_requested(0, N, m, d, d_ff, 2, ids)
        dedup = oracle.bytes_requested(1, N, m, d, d_ff, 2, ids)
        assert slot == n * m * w
        assert dedup == len(set(ids.reshape(-1).tolist())) * w
        assert slot - dedup >= 0  # Eq. (3)
        assert dedup >= m * w      # (B.9)
    bad = np.array([[0, 64, 1, 2, 3, 4]], np.int32)
    assert oracle.bytes_requested(0, N, m, d, d_ff, 2, bad) == oracle.OR_E_IDS
