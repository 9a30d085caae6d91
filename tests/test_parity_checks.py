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


# ------------------------------------------------- BLASST kept selections ----
# The GPU tests' check of a BLASST forward's kept selection
# (tests/test_blasst_gpu.py: _check_kept_format, _keep_of) on the CPU: the
# oracle's own decisions written as a kept selection pass, and planted
# mistakes are refused ("BLASST", summary page, "Meccanismo di Pruning": the
# first block visited is never skipped; skipped blocks leave the row).
def _kept_case(lam=0.3, seed=71):
    import test_blasst_gpu as tbl
    g = np.random.default_rng(seed)
    B, K, H, d = 4, 4, 2, 8
    cu = [0, 30, 30, 61]
    T = cu[-1]
    q, k, v = (g.standard_normal((T, H, d)).astype(np.float32) for _ in range(3))
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    *_, keep = oracle.attend_blasst(q, k, v, idx, B, K, cu, lam, return_keep=True)
    kept = np.full(idx.shape, -1, np.int32)
    for r in np.ndindex(idx.shape[:2]):
        sel = [j for j, kk in zip(idx[r], keep[r]) if kk and j >= 0]
        kept[r][:len(sel)] = sel
    return tbl, idx, keep, kept


def test_blasst_kept_from_the_oracle_passes_and_maps_back():
    tbl, idx, keep, kept = _kept_case()
    assert not keep[idx >= 0].all()              # something was skipped
    tbl._check_kept_format(kept, idx)
    assert np.array_equal(tbl._keep_of(kept, idx), keep)


@pytest.mark.parametrize("mistake", ["first_dropped", "not_ascending", "hole", "foreign_block",
                                     "duplicate"])
def test_blasst_kept_planted_mistakes_are_refused(mistake):
    tbl, idx, keep, kept = _kept_case()
    bad = kept.copy()
    K = idx.shape[-1]
    n = (bad >= 0).sum(-1)
    rows = np.argwhere((n >= 2) & (n < K))       # room for a hole after the last block
    assert len(rows)
    t, h = rows[len(rows) // 2]
    m = int(n[t, h])
    row = bad[t, h]
    if mistake == "first_dropped":
        row[:m - 1] = row[1:m].copy()
        row[m - 1] = -1
    elif mistake == "not_ascending":
        row[0], row[1] = row[1], row[0]
    elif mistake == "hole":
        row[m] = row[m - 1]
        row[m - 1] = -1
    elif mistake == "foreign_block":
        listed = set(idx[t, h].tolist())
        row[m - 1] = next(j for j in range(1000, 2000) if j not in listed)
    elif mistake == "duplicate":
        row[1] = row[0]
    with pytest.raises(AssertionError):
        tbl._check_kept_format(bad, idx)
