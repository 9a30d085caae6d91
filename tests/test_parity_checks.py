"""The GPU tests' selection check (tests/parity.py) on the CPU: rows that the
oracle itself produced pass, valid alternatives at a near-tie pass, and
every kind of wrong row -- planted into a copy of the oracle's own rows --
is refused.  Each query keeps its top-k blocks ("Optimizing Mixture of
Block Attention", summary page, "Definizione del Compito"); with the
forced own block that is the top-(k-1) of the past blocks by the
router-score equation ("Architettura del Modello Statistico")."""
import numpy as np
import pytest

import oracle
import parity


def _tied_case(K=4, B=4, nblk=12, H=1, d=8, seed=3):
    """Blocks 1, 2 and 3 share one centroid (exact ties for every query);
    block 0 has a much larger mean along q, so the routed sets are {0 and two
    of 1..3} for the early rows."""
    g = np.random.default_rng(seed)
    T = B * nblk
    q = np.abs(g.standard_normal((T, H, d))).astype(np.float32) + 0.5
    k = g.standard_normal((T, H, d)).astype(np.float32) * 0.1 - 1.0
    k[0:B] += 3.0
    for j in (2, 3):
        k[j * B:(j + 1) * B] = k[B:2 * B]
    cu = [0, T]
    cent = oracle.centroids(k, B, cu)
    idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    return q, cent, idx, ex, cu


def test_oracle_rows_pass_and_nothing_differs():
    q, cent, idx, ex, cu = _tied_case()
    d = parity.check_selection(idx, idx, ex, q, cent, 4, 4, cu)
    assert len(d) == 0


def test_a_different_choice_among_tied_blocks_is_valid():
    K, B = 4, 4
    q, cent, idx, ex, cu = _tied_case(K=K, B=B)
    # query block 4 (tokens 16..19): past blocks 0..3; 1, 2, 3 tie for the
    # two slots after block 0, and the oracle takes the lower ids 1, 2
    t = 17
    assert idx[t, 0].tolist() == [0, 1, 2, 4] and ex[t, 0]
    gpu = idx.copy()
    gpu[t, 0] = [0, 1, 3, 4]
    d = parity.check_selection(gpu, idx, ex, q, cent, B, K, cu)
    assert d.tolist() == [t]


@pytest.mark.parametrize("row,why", [
    ([0, 1, 4, -1], "one routed block dropped"),
    ([0, 1, 1, 4], "a block twice"),
    ([0, -1059061760, 1, 4], "garbage id"),
    ([0, 1, 2, 3], "own block missing"),
    ([0, 1, 2, 5], "future block"),
    ([1, 0, 2, 4], "not ascending"),
    ([0, 1, 2, 4][::-1], "descending"),
    ([1, 2, 3, 4], "the best block swapped for a tied one"),
])
def test_wrong_rows_at_a_near_tie_are_refused(row, why):
    K, B = 4, 4
    q, cent, idx, ex, cu = _tied_case(K=K, B=B)
    t = 17
    assert ex[t, 0]
    gpu = idx.copy()
    gpu[t, 0] = row
    with pytest.raises(AssertionError, match="not a valid"):
        parity.check_selection(gpu, idx, ex, q, cent, B, K, cu, what=why)


def test_any_change_to_a_row_without_a_near_tie_is_refused():
    g = np.random.default_rng(5)
    T, H, d, B, K = 256, 2, 16, 16, 4
    q = g.standard_normal((T, H, d)).astype(np.float32)
    k = g.standard_normal((T, H, d)).astype(np.float32)
    cu = [0, T]
    cent = oracle.centroids(k, B, cu)
    idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    r = np.argwhere(~ex & (np.arange(T)[:, None] // B >= K + 2))[0]
    gpu = idx.copy()
    row = gpu[r[0], r[1]]
    i = r[0] // B
    row[0] = next(j for j in range(i) if j not in row)   # swap in an unselected block
    gpu[r[0], r[1]] = np.sort(row[:K - 1]).tolist() + [i]
    with pytest.raises(AssertionError, match="without a near-tie"):
        parity.check_selection(gpu, idx, ex, q, cent, B, K, cu)


def test_selection_errors_tolerance_edges():
    # past scores; k = 3 -> a = 2nd best = 10.0, b = 3rd best = 10.0 - 5e-5
    s = np.array([20.0, 10.0, 10.0 - 5e-5, 1.0])
    assert parity.selection_errors([0, 1, 4], s, 4, 3) == []
    # b's block instead of a's: within tau = 1e-4 of a -> still valid
    assert parity.selection_errors([0, 2, 4], s, 4, 3) == []
    # a block far below a is not
    assert parity.selection_errors([0, 3, 4], s, 4, 3)
    # fewer past blocks than slots: all of them, in order, then padding
    assert parity.selection_errors([0, 1, 2, -1], s, 2, 4) == []
    assert parity.selection_errors([0, 2, -1, -1], s, 2, 4)
    assert parity.selection_errors([0, 1, 2, 5], s, 2, 4)
