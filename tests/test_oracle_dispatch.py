"""Pins for the oracle's dispatch plan (histogram, scan, stable placement)."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def brute_plan(idx, E):
    """Walk experts in order and, inside one expert, tokens in order,
    handing out consecutive row numbers."""
    T, k = len(idx), len(idx[0])
    counts = [0] * E
    row_of_slot = [[None] * k for _ in range(T)]
    token_of_row = []
    offsets = [0]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t][j] == e:
                    row_of_slot[t][j] = len(token_of_row)
                    token_of_row.append(t)
                    counts[e] += 1
        offsets.append(len(token_of_row))
    return counts, offsets, row_of_slot, token_of_row


@pytest.mark.parametrize("T,E,k,seed", [(1, 4, 2, 0), (37, 8, 4, 1), (64, 16, 3, 2), (50, 5, 5, 3)])
def test_plan_matches_brute_force(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, rs, tr = O.dispatch_plan(idx, E)
    bc, bo, brs, btr = brute_plan(idx.tolist(), E)
    assert counts.tolist() == bc
    assert offsets.tolist() == bo
    assert rs.tolist() == brs
    assert tr.tolist() == btr


def test_invariants_and_empty_experts():
    rng = np.random.default_rng(7)
    T, E, k = 500, 12, 4
    # Experts 3 and 9 never chosen.
    allowed = np.array([e for e in range(E) if e not in (3, 9)])
    idx = np.stack([rng.permutation(allowed)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, rs, tr = O.dispatch_plan(idx, E)
    assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
    assert counts[3] == 0 and counts[9] == 0
    assert offsets[3] == offsets[4] and offsets[9] == offsets[10]
    assert (np.diff(offsets) == counts).all()
    for t in range(T):
        for j in range(k):
            r = rs[t, j]
            assert tr[r] == t
            e = idx[t, j]
            assert offsets[e] <= r < offsets[e + 1]
    for e in range(E):
        seg = tr[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()  # strictly increasing tokens inside an expert


def test_single_expert_is_identity_order():
    idx = np.zeros((9, 1), dtype=np.int32)
    counts, offsets, rs, tr = O.dispatch_plan(idx, 1)
    assert tr.tolist() == list(range(9)) and rs[:, 0].tolist() == list(range(9))


def test_out_of_range_rejected():
    with pytest.raises(ValueError):
        O.dispatch_plan(np.array([[0, 4]], dtype=np.int32), 4)


def test_gather_rows():
    x = np.arange(12.0).reshape(4, 3)
    xp = O.gather_rows(x, np.array([2, 0, 2, 3]))
    np.testing.assert_array_equal(xp, x[[2, 0, 2, 3]])
