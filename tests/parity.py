"""Parity procedure shared by the GPU tests (and checked itself on the CPU).

Selection (P3, P5).  A GPU row of block ids equal to the oracle's passes.  A
row that differs passes only where the oracle marks the query a near-tie
(its (k-1)-th and k-th past scores within 1e-5 relative) and the row is a
valid tolerant top-(k-1) of the oracle's fp64 scores: own block present, no
future block, ascending, unique, -1 padded to k, min(k, i+1) blocks, every
selected past block scoring >= a - tau and every unselected one <= b + tau,
tau = 1e-5 max(|a|, |b|).  Each query keeps its top-k blocks ("Optimizing
Mixture of Block Attention", summary page, "Definizione del Compito"), scored
by the router-score equation ("Architettura del Modello Statistico").

Output (P4).  O and LSE are compared with the oracle's attention on the same
selection: the oracle's own rows where the selections agree, and the oracle
fed the GPU's row (``oracle.attend_rows``) where they differ, so that like is
compared with like.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

import oracle

NEAR_TIE_REL = 1e-5


def selection_errors(row: Sequence[int], scores: np.ndarray, i: int, K: int) -> List[str]:
    """Why ``row`` (k block ids of a query in block i) is not a valid
    tolerant top-(k-1) of the past-block scores ``scores[:i]``; [] if valid."""
    row = [int(x) for x in row]
    err = []
    if len(row) != K:
        return [f"row has {len(row)} entries, expected {K}"]
    m = min(K - 1, i)
    sel = row[: m + 1]
    pad = row[m + 1:]
    if any(x != -1 for x in pad):
        err.append(f"padding {pad} is not all -1")
    if any(x < 0 for x in sel):
        err.append(f"negative id among the first {m + 1} entries {sel}")
    if any(b <= a for a, b in zip(sel, sel[1:])):
        err.append(f"{sel} is not strictly ascending")
    if i not in sel:
        err.append(f"own block {i} missing")
    if any(x > i for x in sel):
        err.append(f"future block in {sel}")
    if err:
        return err
    past = [x for x in sel if x != i]
    if len(past) != m:
        return [f"{len(past)} past blocks, expected {m}"]
    if i < K:
        if past != list(range(i)):
            err.append(f"all {i} past blocks must be kept, got {past}")
        return err
    s = np.asarray(scores[:i], dtype=np.float64)
    order = sorted(range(i), key=lambda j: (-s[j], j))
    a, b = s[order[K - 2]], s[order[K - 1]]
    tau = NEAR_TIE_REL * max(abs(a), abs(b))
    chosen = set(past)
    for j in past:
        if s[j] < a - tau:
            err.append(f"selected block {j} scores {s[j]!r} < a - tau = {a - tau!r}")
    for j in range(i):
        if j not in chosen and s[j] > b + tau:
            err.append(f"unselected block {j} scores {s[j]!r} > b + tau = {b + tau!r}")
    return err


def _own_block(rows: np.ndarray, H: int, B: int, cu: Sequence[int]) -> np.ndarray:
    t = rows // H
    cu = np.asarray(cu, dtype=np.int64)
    s = np.searchsorted(cu, t, side="right") - 1
    return ((t - cu[s]) // B).astype(np.int64)


def check_selection(gpu: np.ndarray, ref: np.ndarray, exempt: np.ndarray, q, cent, B: int,
                    K: int, cu: Sequence[int], rows: Optional[np.ndarray] = None,
                    what: str = "") -> np.ndarray:
    """P3 on every given row.  gpu / ref: [nrows, K] (rows = their global
    token*H + head ids, all rows when None); exempt: [nrows].  Returns the
    global ids of the rows that differ (each checked valid)."""
    H = q.shape[-2]
    gpu = np.asarray(gpu).reshape(-1, K)
    ref = np.asarray(ref).reshape(-1, K)
    exempt = np.asarray(exempt).reshape(-1)
    if rows is None:
        rows = np.arange(gpu.shape[0], dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    diff = np.any(gpu != ref, axis=-1)
    bad = diff & ~exempt
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows differ from the oracle without a "
                           f"near-tie (first row {int(rows[np.argmax(bad)])}: gpu "
                           f"{gpu[np.argmax(bad)].tolist()} oracle {ref[np.argmax(bad)].tolist()})")
    drows = rows[diff]
    if len(drows):
        sc = oracle.route_scores(q, cent, B, cu, drows)
        own = _own_block(drows, H, B, cu)
        for n, (r, i) in enumerate(zip(drows, own)):
            e = selection_errors(gpu[diff][n], sc[n], int(i), K)
            assert not e, f"{what}: near-tie row {int(r)} is not a valid top-(k-1): {e}"
    return drows


def outputs_on_gpu_selection(q, k, v, gpu_idx_full: np.ndarray, B: int, K: int, cu,
                             drows: np.ndarray, scale: float = 0.0):
    """The oracle's (o, lse) of the rows ``drows`` attending the GPU's own
    selection (gpu_idx_full: [T, H, K])."""
    return oracle.attend_rows(q, k, v, gpu_idx_full, B, K, cu, drows, scale=scale)
