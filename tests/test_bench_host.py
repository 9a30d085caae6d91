"""Host-side pieces of bench.py (CPU): the attended-pair count that prices
the BLASST backward, against the workload FLOP count for a full selection
and against a direct count for a selection with blocks dropped; the
refusal of more than one GPU."""
import subprocess
import sys

import numpy as np
import torch

import bench
import oracle
import workloads


def _direct_pairs(kept, cu, B):
    """(query, key) pairs of a selection counted row by row."""
    T, H, K = kept.shape
    n = 0
    for a, b in zip(cu[:-1], cu[1:]):
        for t in range(a, b):
            i = (t - a) // B
            for h in range(H):
                row = kept[t, h]
                n += B * int(np.sum((row >= 0) & (row < i)))
                if np.any(row == i):
                    n += (t - a) - i * B + 1
    return n


def test_attended_keys_of_a_full_selection_match_the_workload_flops():
    for name, seq in (("C1", None), ("C2", 2048)):
        s = workloads.spec(name)
        if seq:
            s = s.scaled(seq)
        x = workloads.make(s)
        cu = workloads.segments(s)
        idx, *_ = oracle.route(x["q"], oracle.centroids(x["k"], s.block_size, cu), s.block_size,
                               s.top_k, cu)
        keys = bench._attended_keys(torch.from_numpy(idx), cu, s.block_size)
        assert keys == workloads.eff_flops(s)["total"] // (4 * s.head_dim)
        assert keys == _direct_pairs(idx, cu, s.block_size)


def test_attended_keys_with_dropped_blocks():
    """Kept selections as the BLASST forward writes them: past blocks and
    own blocks dropped, rows compacted and -1 padded, ragged sequences."""
    B, K, H = 8, 4, 2
    cu = [0, 37, 37, 100]
    T = cu[-1]
    g = np.random.default_rng(3)
    kept = np.full((T, H, K), -1, np.int32)
    for a, b in zip(cu[:-1], cu[1:]):
        for t in range(a, b):
            i = (t - a) // B
            for h in range(H):
                past = sorted(g.choice(i, size=min(K - 1, i), replace=False).tolist()) if i else []
                sel = [j for j in past if g.random() < 0.6] + ([i] if g.random() < 0.7 else [])
                kept[t, h, :len(sel)] = sel
    assert bench._attended_keys(torch.from_numpy(kept), cu, B) == _direct_pairs(kept, cu, B)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout
