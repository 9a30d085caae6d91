"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own loops: each compares it with a
library routine (torch conv1d / mean / scaled_dot_product_attention, numpy
matmul + stable argsort), a closed form, a hand-worked example
(tests/golden), or an invariant that a dropped term, wrong sign, wrong index
or transposed operand would break.

Source: "Optimizing Mixture of Block Attention" summary page -- task
definition ("Definizione del Compito"), router-score equation
("Architettura del Modello Statistico"), key convolution ("Appendice B").
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, dtype=np.float32):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape).astype(dtype)


def _bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a).to(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------- conv ----
def _conv_ref64(k, w, cu):
    """Library conv1d in fp64, per sequence (weights flipped: torch's conv1d
    correlates, the page's form convolves k_{t-l} with w_l)."""
    T, H, d = k.shape
    W = w.shape[-1]
    out = np.zeros((T, H, d), dtype=np.float64)
    wt = torch.from_numpy(w[:, :, ::-1].copy()).double().reshape(H * d, 1, W)
    for s in range(len(cu) - 1):
        x = torch.from_numpy(k[cu[s]:cu[s + 1]]).double().reshape(-1, H * d).T[None]
        x = F.pad(x, (W - 1, 0))
        y = F.conv1d(x, wt, groups=H * d)[0].T.reshape(-1, H, d)
        out[cu[s]:cu[s + 1]] = y.numpy()
    return out


@pytest.mark.parametrize("W", [1, 3, 4, 8])
def test_conv_plain_matches_library_conv1d(W):
    T, H, d = 70, 3, 8
    k = _rand((T, H, d), 1)
    w = _rand((H, d, W), 2) * np.float32(1 / math.sqrt(W))
    cu = [0, 70]
    ours = oracle.key_conv(k, w, cu, mode=0, round_bf16=False)
    ref = _conv_ref64(k, w, cu)
    # fp32 fmaf chain of W taps: relative error <= W * 2^-24 of sum |w x|
    bound = (W + 1) * 2.0 ** -24 * _conv_ref64(np.abs(k), np.abs(w), cu)
    assert np.all(np.abs(ours - ref) <= bound + 1e-30)


def test_conv_plain_bf16_rounding_matches_fp64_rounding():
    T, H, d, W = 400, 4, 16, 3
    k = _bf16(_rand((T, H, d), 3))
    w = _rand((H, d, W), 4) * np.float32(1 / math.sqrt(W))
    cu = [0, T]
    ours = oracle.key_conv(k, w, cu, mode=0, round_bf16=True)
    ref = _bf16(_conv_ref64(k, w, cu).astype(np.float32))
    same = ours == ref
    assert same.mean() > 0.999
    # where they differ it is by one bf16 step at a rounding boundary
    diff = np.abs(ours - ref)[~same]
    assert np.all(diff <= np.abs(ref[~same]) * 2.0 ** -7 + 1e-30)
    # outputs are bf16 values
    assert np.array_equal(ours, _bf16(ours))


def test_conv_special_cases():
    T, H, d, W = 20, 2, 4, 4
    k = _bf16(_rand((T, H, d), 5))
    cu = [0, T]
    # identity filter (tap 0 = current token) reproduces k exactly
    w = np.zeros((H, d, W), np.float32)
    w[:, :, 0] = 1
    assert np.array_equal(oracle.key_conv(k, w, cu), k)
    # e_l shifts by l with zero fill at the sequence start
    for l in range(W):
        w = np.zeros((H, d, W), np.float32)
        w[:, :, l] = 1
        out = oracle.key_conv(k, w, cu)
        assert np.array_equal(out[l:], k[:T - l])
        assert np.all(out[:l] == 0)
    # W = 1 is a per-channel scale
    w1 = _rand((H, d, 1), 6)
    out = oracle.key_conv(k, w1, cu, round_bf16=False)
    assert np.array_equal(out, (k * w1[None, :, :, 0]).astype(np.float32))


def test_conv_varlen_equals_separate_sequences():
    H, d, W = 2, 8, 3
    lens = [5, 17, 1, 9]
    cu = list(np.cumsum([0] + lens))
    k = _bf16(_rand((cu[-1], H, d), 7))
    w = _rand((H, d, W), 8)
    whole = oracle.key_conv(k, w, cu)
    for s in range(len(lens)):
        part = oracle.key_conv(k[cu[s]:cu[s + 1]], w, [0, lens[s]])
        assert np.array_equal(whole[cu[s]:cu[s + 1]], part)


def test_conv_silu_residual_matches_library():
    T, H, d, W = 50, 2, 8, 5
    k = _rand((T, H, d), 9)
    w = _rand((H, d, W), 10) * np.float32(0.5)
    cu = [0, T]
    ours = oracle.key_conv(k, w, cu, mode=1, round_bf16=False)
    conv = torch.from_numpy(_conv_ref64(k, w, cu))
    ref = (torch.from_numpy(k).double() + F.silu(conv)).numpy()
    assert np.allclose(ours, ref, rtol=2e-6, atol=2e-6)
    # zero filter -> k' = k exactly
    w0 = np.zeros_like(w)
    assert np.array_equal(oracle.key_conv(k, w0, cu, mode=1, round_bf16=False), k)


# ----------------------------------------------------------- centroids ----
def test_centroids_match_library_mean():
    H, d, B = 3, 8, 16
    lens = [64, 40, 16, 7]             # includes partial last blocks
    cu = list(np.cumsum([0] + lens))
    k = _bf16(_rand((cu[-1], H, d), 11))
    cent = oracle.centroids(k, B, cu)
    rows = []
    for s, L in enumerate(lens):
        for j in range((L + B - 1) // B):
            a, b = cu[s] + j * B, min(cu[s] + (j + 1) * B, cu[s + 1])
            rows.append(torch.from_numpy(k[a:b]).double().mean(dim=0).float().numpy())
    ref = np.stack(rows)
    assert cent.shape == ref.shape
    assert np.array_equal(cent, ref)
    assert oracle.total_blocks(cu, B) == len(rows)


def test_centroid_of_constant_block_is_that_key():
    H, d, B = 1, 4, 8
    k = np.zeros((16, H, d), np.float32)
    k[:8] = np.array([0.1, -3.5, 7.25, 1e-3], np.float32)
    k[8:] = _rand((8, H, d), 12)
    cent = oracle.centroids(k, B, [0, 16])
    assert np.array_equal(cent[0, 0], k[0, 0])


# ------------------------------------------------------------- routing ----
def _route_brute(q, cent, B, K, cu):
    """Full fp64 score matrix (matmul), causal mask, stable argsort."""
    T, H, d = q.shape
    idx = np.full((T, H, K), -1, np.int32)
    boff = 0
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        n = (L + B - 1) // B
        for h in range(H):
            S = q[cu[s]:cu[s + 1], h].astype(np.float64) @ cent[boff:boff + n, h].astype(np.float64).T
            for tl in range(L):
                i = tl // B
                past = S[tl, :i]
                order = np.argsort(-past, kind="stable")[:min(K - 1, i)]
                row = sorted(order.tolist() + [i])
                idx[cu[s] + tl, h, :len(row)] = row
        boff += n
    return idx


@pytest.mark.parametrize("B,K,lens", [(4, 3, [64]), (8, 2, [40, 24]),
                                      (4, 16, [32]), (16, 4, [100, 3, 50])])
def test_route_matches_bruteforce(B, K, lens):
    H, d = 2, 8
    cu = list(np.cumsum([0] + lens))
    q = _bf16(_rand((cu[-1], H, d), 13))
    k = _bf16(_rand((cu[-1], H, d), 14))
    cent = oracle.centroids(k, B, cu)
    idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    assert np.array_equal(idx, _route_brute(q, cent, B, K, cu))


def test_route_invariants():
    H, d, B, K = 2, 8, 4, 5
    lens = [61, 30]
    cu = list(np.cumsum([0] + lens))
    q = _rand((cu[-1], H, d), 15)
    k = _rand((cu[-1], H, d), 16)
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    for s, L in enumerate(lens):
        for tl in range(L):
            i = tl // B
            for h in range(H):
                row = idx[cu[s] + tl, h]
                valid = row[row >= 0]
                assert i in valid                         # own block kept
                assert np.all(valid <= i)                 # no future block
                assert len(valid) == min(K, i + 1)        # |S| = min(k, i+1)
                assert np.all(np.diff(valid) > 0)         # ascending, distinct
                assert np.all(row[len(valid):] == -1)     # -1 padding at end


def test_route_ties_go_to_lower_index():
    # q = ones; block j's keys chosen so several blocks have equal sums.
    B, K, d = 2, 3, 2
    T = 10
    q = np.ones((T, 1, d), np.float32)
    blocks = [[1, 1], [2, 0], [0, 2], [1, 1], [5, 5]]   # sums: 2,2,2,2,10
    k = np.zeros((T, 1, d), np.float32)
    for j, (a, b) in enumerate(blocks):
        k[2 * j, 0] = [a, 0]
        k[2 * j + 1, 0] = [0, b]
    cent = oracle.centroids(k, B, [0, T])
    idx, ga, gb, ex = oracle.route(q, cent, B, K, [0, T])
    # query block 4 (t=8,9): past blocks 0..3 all score 1 -> take 0 and 1
    assert idx[8, 0].tolist() == [0, 1, 4]
    assert idx[9, 0].tolist() == [0, 1, 4]
    assert ex[8, 0] and ga[8, 0] == gb[8, 0]
    # query block 3: past 0..2 tie -> 0, 1
    assert idx[6, 0].tolist() == [0, 1, 3]


def _route_one_query(scores, K):
    """The oracle's routing of one query whose past-block scores are exactly
    ``scores`` (B = 1, q = e_0 and centroid j = (scores[j], 0): every score is
    one exact product)."""
    n = len(scores)
    T = n + 1
    q = np.zeros((T, 1, 2), np.float32)
    q[:, 0, 0] = 1.0
    cent = np.zeros((T, 1, 2), np.float32)
    cent[:n, 0, 0] = np.asarray(scores, np.float32)
    assert np.array_equal(cent[:n, 0, 0].astype(np.float64), np.asarray(scores, np.float64))
    idx, ga, gb, ex = oracle.route(q, cent, 1, K, [0, T])
    return idx[n, 0].tolist(), float(ga[n, 0]), float(gb[n, 0]), bool(ex[n, 0])


# (k-1)-th best a = 100000 (or -100000) against the k-th best b: the near-tie
# record is |a - b| <= 1e-5 max(|a|, |b|) on those two ranks only
@pytest.mark.parametrize("a,b,exempt", [
    (100000.0, 99999.5, True),        # 0.5e-5 relative
    (100000.0, 99999.125, True),      # 0.875e-5
    (100000.0, 99998.875, False),     # 1.125e-5
    (100000.0, 99998.0, False),       # 2e-5
    (-100000.0, -100000.5, True),     # negative scores, 0.5e-5 of |b|
    (-100000.0, -100002.0, False),    # 2e-5
    (3.0, 3.0, True),                 # an exact tie
])
def test_route_near_tie_gap_threshold(a, b, exempt):
    K = 4                              # k-1 = 3 routed slots: ranks 3 and 4
    # past scores in scrambled block order: two clear winners, a, b, a clear loser
    top = abs(a) * 3
    scores = [b, top, a - 50000 if a > 0 else a - 50000, top * 2, a]
    order = sorted(range(5), key=lambda j: (-scores[j], j))
    assert [scores[j] for j in order[2:4]] == [a, b]
    row, ga, gb, ex = _route_one_query(scores, K)
    assert row == sorted(order[:3]) + [5]
    assert ga == a and gb == b
    assert ex == exempt


def test_route_near_tie_uses_ranks_k_minus_1_and_k():
    """Only the gap between the (k-1)-th and k-th best past scores counts:
    a near-equal pair at ranks (k-2, k-1) or (k, k+1) is no near-tie."""
    K = 4
    # ranks: 1st 300000, 2nd 100000.5, 3rd (k-1) 100000, 4th (k) 90000, 5th 89999.5
    scores = [89999.5, 100000.0, 300000.0, 90000.0, 100000.5]
    row, ga, gb, ex = _route_one_query(scores, K)
    assert row == [1, 2, 4, 5]
    assert (ga, gb) == (100000.0, 90000.0)
    assert not ex
    # moving the near-equal pair onto ranks (k-1, k) makes it one
    scores = [89999.5, 100000.5, 300000.0, 100000.0, 200000.0]
    row, ga, gb, ex = _route_one_query(scores, K)
    assert row == [1, 2, 4, 5]
    assert (ga, gb) == (100000.5, 100000.0)
    assert ex
    # and with k = 2 the pair is the best and second-best score (2.2e-6 apart)
    row, ga, gb, ex = _route_one_query([7.0, 7.0 + 2.0 ** -16, 1.0], 2)
    assert row == [1, 3] and (ga, gb) == (7.0 + 2.0 ** -16, 7.0) and ex


def test_route_top_k_at_least_blocks_selects_all_past():
    H, d, B = 1, 4, 4
    T = 32
    q = _rand((T, H, d), 17)
    k = _rand((T, H, d), 18)
    idx, *_ = oracle.route(q, oracle.centroids(k, B, [0, T]), B, 8, [0, T])
    for t in range(T):
        i = t // B
        assert idx[t, 0, :i + 1].tolist() == list(range(i + 1))


# ----------------------------------------------------------- attention ----
def _mask_from_idx(idx_row_sets, L, B):
    m = np.zeros((L, L), bool)
    for t in range(L):
        i = t // B
        for j in idx_row_sets[t]:
            if j < 0:
                continue
            if j < i:
                m[t, j * B:min((j + 1) * B, L)] = True
        m[t, i * B:t + 1] = True
    return m


def test_attend_dense_when_topk_covers_all_blocks():
    H, d, B, T = 2, 16, 8, 48
    q, k, v = (_rand((T, H, d), s) for s in (19, 20, 21))
    cu = [0, T]
    K = T // B
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    o, lse = oracle.attend(q, k, v, idx, B, K, cu)
    tq, tk, tv = (torch.from_numpy(x).double().permute(1, 0, 2)[None] for x in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2)
    assert np.allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    S = (tq @ tk.transpose(-1, -2))[0] / math.sqrt(d)
    S = S.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -math.inf)
    assert np.allclose(lse, torch.logsumexp(S, -1).T.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("B,K", [(4, 3), (8, 2), (4, 1)])
def test_attend_matches_masked_sdpa(B, K):
    H, d, T = 2, 8, 40
    q, k, v = (_bf16(_rand((T, H, d), s)) for s in (22, 23, 24))
    cu = [0, T]
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    scale = 0.37
    o, lse = oracle.attend(q, k, v, idx, B, K, cu, scale=scale)
    for h in range(H):
        m = torch.from_numpy(_mask_from_idx([idx[t, h].tolist() for t in range(T)], T, B))
        tq, tk, tv = (torch.from_numpy(x[:, h]).double() for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                             attn_mask=m[None], scale=scale)[0]
        assert np.allclose(o[:, h], ref.numpy(), rtol=1e-12, atol=1e-12)
        S = (tq @ tk.T * scale).masked_fill(~m, -math.inf)
        assert np.allclose(lse[:, h], torch.logsumexp(S, -1).numpy(), rtol=1e-12, atol=1e-12)


def test_attend_v_ones_gives_ones_and_v_identity_gives_probabilities():
    H, d, B, K = 1, 32, 4, 3
    T = 32                                          # T <= d so V = I fits
    q, k = _rand((T, H, d), 25), _rand((T, H, d), 26)
    cu = [0, T]
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    o, _ = oracle.attend(q, k, np.ones((T, H, d), np.float32), idx, B, K, cu)
    assert np.allclose(o, 1.0, rtol=0, atol=1e-14)
    eye = np.eye(T, d, dtype=np.float32)[:, None, :]
    p, _ = oracle.attend(q, k, eye, idx, B, K, cu)
    p = p[:, 0, :T]
    assert np.allclose(p.sum(-1), 1.0, atol=1e-14)
    support = _mask_from_idx([idx[t, 0].tolist() for t in range(T)], T, B)
    assert np.all(p[~support] == 0)
    assert np.all(p[support] > 0)


def test_attend_single_block_is_dense_causal():
    H, d, T = 1, 8, 24
    B = 32                                           # one (partial) block
    q, k, v = (_rand((T, H, d), s) for s in (27, 28, 29))
    idx, *_ = oracle.route(q, oracle.centroids(k, B, [0, T]), B, 2, [0, T])
    o, _ = oracle.attend(q, k, v, idx, B, 2, [0, T])
    tq, tk, tv = (torch.from_numpy(x).double().permute(1, 0, 2)[None] for x in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0].permute(1, 0, 2)
    assert np.allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------- golden + whole pass ----
def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "hand_worked_B2_d2.json")))
    arr = lambda key: np.array(g[key], np.float32)[:, None, :]
    k, q, v = arr("k"), arr("q"), arr("v")
    B, K, cu = g["B"], g["top_k"], [0, 6]
    cent = oracle.centroids(k, B, cu)
    assert np.array_equal(cent[:, 0], np.array(g["centroids"], np.float32))
    idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    assert idx[:, 0].tolist() == g["idx"]
    assert ex[:, 0].tolist() == g["exempt"]
    o, lse = oracle.attend(q, k, v, idx, B, K, cu, scale=math.log(2.0))
    num = np.array(g["o_num"], np.float64)
    assert np.allclose(o[:, 0, 0], num[:, 0] / num[:, 1], rtol=1e-14, atol=1e-14)
    assert np.allclose(o[:, 0, 1], 1.0, rtol=1e-14)
    assert np.allclose(lse[:, 0], np.log(np.array(g["lse_of"], np.float64)), rtol=1e-14)
    kc = oracle.key_conv(k, np.array(g["conv_w"], np.float32)[None], cu)
    assert np.array_equal(kc[:, 0], np.array(g["k_conv"], np.float32))


def test_forward_heads_batches_and_sequences_are_independent():
    H, d, B, K, W = 3, 8, 4, 3, 3
    lens = [24, 13, 32]
    cu = list(np.cumsum([0] + lens))
    q, k, v = (_bf16(_rand((cu[-1], H, d), s)) for s in (30, 31, 32))
    w = _rand((H, d, W), 33)
    full = oracle.forward(q, k, v, B, K, cu, conv_w=w)
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        for h in range(H):
            part = oracle.forward(q[sl, h:h + 1], k[sl, h:h + 1], v[sl, h:h + 1],
                                  B, K, [0, lens[s]], conv_w=w[h:h + 1])
            assert np.array_equal(full["idx"][sl, h:h + 1], part["idx"])
            assert np.array_equal(full["o"][sl, h:h + 1], part["o"])
    again = oracle.forward(q, k, v, B, K, cu, conv_w=w, nthreads=1)
    assert np.array_equal(full["o"], again["o"]) and np.array_equal(full["idx"], again["idx"])


# ----------------------------------------------------------- workloads ----
def test_workload_generator_is_seeded_and_shaped():
    s = workloads.spec("C1")
    a, b = workloads.make(s), workloads.make(s)
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["v"], b["v"])
    assert a["q"].shape == (1, 1024, 1, 64) and a["q"].dtype == torch.float32
    s5 = workloads.spec("C5").scaled(1024)
    x = workloads.make(s5)
    assert x["q"].shape == (1024, 16, 128) and x["q"].dtype == torch.bfloat16
    assert x["cu_seqlens"][0] == 0 and x["cu_seqlens"][-1] == 1024
    assert x["conv_w"].shape == (16, 128, 4)


def test_effective_flops_match_counts_from_oracle_idx():
    s = workloads.Spec("t", 7, 2, 200, 2, 8, 16, 4, "f32")
    x = workloads.make(s)
    cu = workloads.segments(s)
    idx, *_ = oracle.route(x["q"], oracle.centroids(x["k"], s.block_size, cu),
                           s.block_size, s.top_k, cu)
    keys = 0
    for b in range(s.batch):
        for tl in range(s.seq):
            i = tl // s.block_size
            for h in range(s.heads):
                row = idx[b * s.seq + tl, h]
                keys += s.block_size * int(np.sum((row >= 0) & (row < i)))
                keys += tl - i * s.block_size + 1
    assert workloads.eff_flops(s)["total"] == 4 * s.head_dim * keys
    pairs = int(np.sum((idx >= 0) & (idx < (np.arange(s.seq) // s.block_size)[None, :, None, None].repeat(2, 0).reshape(-1, 1, 1))))
    assert workloads.routed_pairs(s) == pairs


def test_row_subsets_equal_full_runs():
    H, d, B, K = 2, 8, 4, 3
    lens = [37, 0, 20]
    cu = list(np.cumsum([0] + lens))
    q, k, v = (_bf16(_rand((cu[-1], H, d), s)) for s in (34, 35, 36))
    cent = oracle.centroids(k, B, cu)
    idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    o, lse = oracle.attend(q, k, v, idx, B, K, cu)
    rows = np.array([0, 5, 17, 2 * 36 + 1, 2 * 37, 2 * 56 + 1])
    ri, rga, rgb, rex = oracle.route_rows(q, cent, B, K, cu, rows)
    assert np.array_equal(ri, idx.reshape(-1, K)[rows])
    assert np.array_equal(rex, ex.reshape(-1)[rows])
    ro, rl = oracle.attend_rows(q, k, v, idx, B, K, cu, rows)
    assert np.array_equal(ro, o.reshape(-1, d)[rows])
    assert np.array_equal(rl, lse.reshape(-1)[rows])


# ------------------------------------------------------------ backward ----
# "Backward Pass: Ricalcolo (Algoritmo 5)": gradients of the attention over
# the selected blocks, for a fixed selection.  Pinned against the library's
# own autograd of masked attention, central differences of the (separately
# pinned) forward, and closed-form invariants.
def _bwd_case(seed, T=40, H=2, d=8, cu=(0, 17, 40)):
    q, k, v, do = (_bf16(_rand((T, H, d), seed + i)) for i in range(4))
    return q, k, v, do, list(cu)


@pytest.mark.parametrize("B,K", [(4, 3), (8, 2), (4, 1), (8, 5)])
def test_attend_bwd_matches_autograd_of_masked_sdpa(B, K):
    q, k, v, do, cu = _bwd_case(40)
    T, H, d = q.shape
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    scale = 0.41
    dq, dk, dv = oracle.attend_bwd(q, k, v, idx, do, B, K, cu, scale=scale)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        L = b - a
        for h in range(H):
            m = torch.from_numpy(_mask_from_idx([idx[t, h].tolist() for t in range(a, b)], L, B))
            tq, tk, tv = (torch.from_numpy(x[a:b, h]).double().requires_grad_() for x in (q, k, v))
            o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=m[None],
                                               scale=scale)[0]
            o.backward(torch.from_numpy(do[a:b, h]).double())
            for ours, ref in ((dq, tq), (dk, tk), (dv, tv)):
                assert np.allclose(ours[a:b, h], ref.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_attend_bwd_matches_central_differences():
    B, K = 4, 3
    q, k, v, do, cu = _bwd_case(50, T=24, H=1, d=4, cu=(0, 24))
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    grads = dict(zip("qkv", oracle.attend_bwd(q, k, v, idx, do, B, K, cu)))
    base = {"q": q, "k": k, "v": v}

    def loss(x):
        o, _ = oracle.attend(x["q"], x["k"], x["v"], idx, B, K, cu)
        return float(np.sum(o * do.astype(np.float64)))

    g = np.random.default_rng(5)
    for name in "qkv":
        for _ in range(12):
            t, c = int(g.integers(0, 24)), int(g.integers(0, 4))
            xp = {n: a.copy() for n, a in base.items()}
            xm = {n: a.copy() for n, a in base.items()}
            xp[name][t, 0, c] += np.float32(1e-3)
            xm[name][t, 0, c] -= np.float32(1e-3)
            step = float(xp[name][t, 0, c]) - float(xm[name][t, 0, c])
            fd = (loss(xp) - loss(xm)) / step
            assert abs(fd - grads[name][t, 0, c]) <= 1e-5 * max(1.0, abs(fd)), (name, t, c)


def test_attend_bwd_invariants():
    B, K = 4, 3
    q, k, v, do, cu = _bwd_case(60)
    T, H, d = q.shape
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    dq, dk, dv = oracle.attend_bwd(q, k, v, idx, do, B, K, cu)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        # each row's probabilities sum to one: sum_u dv_u = sum_t dO_t
        assert np.allclose(dv[a:b].sum(0), do[a:b].astype(np.float64).sum(0), atol=1e-12)
        # each row's dS sums to zero: sum_u dk_u = 0
        assert np.allclose(dk[a:b].sum(0), 0.0, atol=1e-12)
    # dO = 0: every gradient vanishes
    z = oracle.attend_bwd(q, k, v, idx, np.zeros_like(do), B, K, cu)
    assert all(np.all(x == 0.0) for x in z)
    # equal value rows make O independent of q and k
    vc = np.broadcast_to(v[:1], v.shape).copy()
    dq1, dk1, dv1 = oracle.attend_bwd(q, k, vc, idx, do, B, K, cu)
    assert np.abs(dq1).max() < 1e-12 and np.abs(dk1).max() < 1e-12
    # the first token of a sequence sees only itself (P = 1, dS = 0)
    assert np.all(dq[0] == 0.0) and np.all(dq[17] == 0.0)


def test_attend_bwd_subsets_equal_full_runs():
    B, K = 4, 3
    q, k, v, do, cu = _bwd_case(70)
    T, H, d = q.shape
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    full = oracle.attend_bwd(q, k, v, idx, do, B, K, cu)
    g = np.random.default_rng(3)
    qsel = g.random((T, H)) < 0.3
    nb = oracle.total_blocks(cu, B)
    kbsel = g.random((nb, H)) < 0.3
    sub = oracle.attend_bwd(q, k, v, idx, do, B, K, cu, qsel=qsel, kbsel=kbsel)
    assert np.array_equal(sub[0][qsel], full[0][qsel])
    assert np.isnan(sub[0][~qsel]).all()
    boff = np.concatenate([[0], np.cumsum([-(-(cu[s + 1] - cu[s]) // B) for s in range(len(cu) - 1)])])
    for t in range(T):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        gblk = boff[s] + (t - cu[s]) // B
        for h in range(H):
            for x, f in ((sub[1], full[1]), (sub[2], full[2])):
                if kbsel[gblk, h]:
                    assert np.array_equal(x[t, h], f[t, h])
                else:
                    assert np.isnan(x[t, h]).all()


# ------------------------------------------------------- conv backward ----
def _conv_autograd64(k, w, g, cu, mode):
    """Library autograd of the key conv in fp64 (per-sequence conv1d with
    flipped weights and left padding, plus k + silu(conv) for mode 1)."""
    T, H, d = k.shape
    W = w.shape[-1]
    wt = torch.from_numpy(w[:, :, ::-1].copy()).double().reshape(H * d, 1, W).requires_grad_()
    kt = torch.from_numpy(k).double().requires_grad_()
    outs = []
    for s in range(len(cu) - 1):
        x = kt[cu[s]:cu[s + 1]].reshape(-1, H * d).T[None]
        y = F.conv1d(F.pad(x, (W - 1, 0)), wt, groups=H * d)[0].T.reshape(-1, H, d)
        if mode == 1:
            y = kt[cu[s]:cu[s + 1]] + F.silu(y)
        outs.append(y)
    out = torch.cat(outs)
    out.backward(torch.from_numpy(g).double())
    dw = wt.grad.reshape(H, d, W).numpy()[:, :, ::-1]
    return kt.grad.numpy(), dw


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("W", [1, 3, 4])
def test_conv_bwd_matches_autograd_conv1d(mode, W):
    T, H, d = 60, 2, 8
    cu = [0, 1, 25, 60]
    k = _bf16(_rand((T, H, d), 81))
    g = _bf16(_rand((T, H, d), 82))
    w = _rand((H, d, W), 83) * np.float32(1 / math.sqrt(W))
    dk, dw = oracle.key_conv_bwd(k, w, g, cu, mode)
    rk, rw = _conv_autograd64(k, w, g, cu, mode)
    assert np.allclose(dk, rk, rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, rw, rtol=1e-12, atol=1e-12)


def test_conv_bwd_matches_central_differences():
    T, H, d, W = 12, 1, 2, 3
    cu = [0, 12]
    k = _rand((T, H, d), 84)
    g = _rand((T, H, d), 85)
    w = _rand((H, d, W), 86)
    for mode in (0, 1):
        dk, dw = oracle.key_conv_bwd(k, w, g, cu, mode)

        def loss(kk, ww):
            # the conv in fp64 through the library (the oracle's own forward
            # rounds to fp32 by design, too coarse for differences)
            x = torch.from_numpy(kk[:, 0].T.copy()).double()[None]
            wt = torch.from_numpy(ww[0, :, ::-1].copy()).double()[:, None]
            y = F.conv1d(F.pad(x, (W - 1, 0)), wt, groups=d)[0].T
            if mode == 1:
                y = torch.from_numpy(kk[:, 0]).double() + F.silu(y)
            return float((y * torch.from_numpy(g[:, 0]).double()).sum())

        for (t, c) in [(0, 0), (5, 1), (11, 0)]:
            kp, km = k.copy(), k.copy()
            kp[t, 0, c] += np.float32(1e-3)
            km[t, 0, c] -= np.float32(1e-3)
            fd = (loss(kp, w) - loss(km, w)) / (float(kp[t, 0, c]) - float(km[t, 0, c]))
            assert abs(fd - dk[t, 0, c]) <= 1e-5 * max(1.0, abs(fd))
        for (c, l) in [(0, 0), (1, 2)]:
            wp, wm = w.copy(), w.copy()
            wp[0, c, l] += np.float32(1e-3)
            wm[0, c, l] -= np.float32(1e-3)
            fd = (loss(k, wp) - loss(k, wm)) / (float(wp[0, c, l]) - float(wm[0, c, l]))
            assert abs(fd - dw[0, c, l]) <= 1e-5 * max(1.0, abs(fd))


def test_conv_bwd_identity_filter_passes_gradient_through():
    T, H, d, W = 20, 2, 4, 3
    cu = [0, 7, 20]
    k, g = _rand((T, H, d), 87), _rand((T, H, d), 88)
    w = np.zeros((H, d, W), np.float32)
    w[:, :, 0] = 1.0                                   # k' = k
    dk, dw = oracle.key_conv_bwd(k, w, g, cu, 0)
    assert np.array_equal(dk, g.astype(np.float64))
    # dw_l = sum_t g_t k_{t-l} within each sequence
    ref = np.zeros((H, d, W))
    for s in range(2):
        a, b = cu[s], cu[s + 1]
        for l in range(W):
            ref[:, :, l] += (g[a + l:b].astype(np.float64) * k[a:b - l]).sum(0)
    assert np.allclose(dw, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- BLASST ----
# "BLASST: Dynamic BLocked Attention Sparsity via Softmax Thresholding",
# section "Meccanismo di Pruning": blocks visited in order with a running
# maximum M; a block whose maximum m~ has m~ - M < ln(lambda) is skipped.
def _blasst_case(seed, T=48, H=2, d=8, B=4, K=4):
    q, k, v = (_bf16(_rand((T, H, d), seed + i)) for i in range(3))
    cu = [0, 20, T]
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    return q, k, v, idx, cu, B, K


def test_blasst_with_lambda_zero_is_plain_attention():
    q, k, v, idx, cu, B, K = _blasst_case(60)
    o, lse = oracle.attend(q, k, v, idx, B, K, cu)
    ob, lb, near = oracle.attend_blasst(q, k, v, idx, B, K, cu, 0.0)
    assert np.array_equal(o, ob) and np.array_equal(lse, lb) and not near.any()


def test_blasst_keep_mask_matches_masked_sdpa():
    """Explicit per-slot keep choices: the attention over the kept blocks
    equals the library's SDPA with that boolean mask (fp64)."""
    q, k, v, idx, cu, B, K = _blasst_case(61)
    T, H, d = q.shape
    g = np.random.default_rng(5)
    keep = g.random(idx.shape) < 0.6
    ob, lb, _ = oracle.attend_blasst(q, k, v, idx, B, K, cu, 0.0, keep=keep)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        L = s1 - s0
        for h in range(H):
            m = np.zeros((L, L), bool)
            for tl in range(L):
                i = tl // B
                row, kp = idx[s0 + tl, h], keep[s0 + tl, h]
                own_kept = True
                for p in range(K):
                    j = row[p]
                    if j == i:
                        own_kept = bool(kp[p])
                    elif 0 <= j < i and kp[p]:
                        m[tl, j * B:min((j + 1) * B, L)] = True
                if own_kept:
                    m[tl, i * B:tl + 1] = True
            qq, kk, vv = (torch.from_numpy(x[s0:s1, h]).double()[None] for x in (q, k, v))
            ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=torch.from_numpy(m)[None])
            rows = m.any(1)
            assert np.allclose(ob[s0:s1, h][rows], ref[0].numpy()[rows], atol=1e-12)


def test_blasst_crafted_skips():
    """One head, blocks of 2 keys, d = 2, q = (1, 0) and scale 1: a key's
    score is its first coordinate.  Block maxima, in visiting order, are
    1, 3, 2.5, 0.5 (past) and the own block's; with lambda = e^-1 a block is
    skipped when its maximum is more than 1 below the running maximum."""
    B, K = 2, 5
    firsts = [[1.0, 0.0], [3.0, -1.0], [2.5, 2.0], [0.5, 0.0], [2.2, 9.0]]   # block 4 = own
    T = 10
    q = np.zeros((T, 1, 2), np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((T, 1, 2), np.float32)
    for j, (a, b) in enumerate(firsts):
        k[2 * j, 0, 0], k[2 * j + 1, 0, 0] = a, b
    v = _rand((T, 1, 2), 62)
    idx = np.full((T, 1, K), -1, np.int32)
    idx[8] = [[0, 1, 2, 3, 4]]                   # query t = 8 (own block 4, keys u <= 8)
    idx[:8] = [[0, -1, -1, -1, -1]]
    idx[9] = idx[8]
    o, lse, near = oracle.attend_blasst(q, k, v, idx, B, K, [0, T], math.exp(-1.0), scale=1.0)
    # t = 8: block 0 (max 1) kept, M = 1; block 1 (3) kept, M = 3; block 2
    # (2.5) kept; block 3 (0.5 < 3 - 1) skipped; own block: key 8 only
    # (score 2.2 >= 2) kept
    keys = [0, 1, 2, 3, 4, 5, 8]
    z = k[keys, 0, 0].astype(np.float64)
    p = np.exp(z - z.max())
    assert np.allclose(o[8, 0], (p[:, None] * v[keys, 0]).sum(0) / p.sum(), atol=1e-14)
    assert abs(lse[8, 0] - (z.max() + math.log(p.sum()))) < 1e-14
    # t = 9: own block keys 8, 9 (max 9) raise the maximum: still kept, block 3 still skipped
    keys9 = keys + [9]
    z9 = k[keys9, 0, 0].astype(np.float64)
    p9 = np.exp(z9 - z9.max())
    assert np.allclose(o[9, 0], (p9[:, None] * v[keys9, 0]).sum(0) / p9.sum(), atol=1e-14)
    # a threshold exactly at a decision is flagged as near (block 3 is the
    # 4th visited: bit 3), and the flipped decision keeps it
    o2, _, near2 = oracle.attend_blasst(q, k, v, idx, B, K, [0, T], math.exp(-2.5), scale=1.0)
    assert near2[8, 0] == 1 << 3 and near[8, 0] == 0      # block 3: 0.5 - 3 = -2.5
    flip = np.zeros((T, 1), np.uint64)
    flip[8, 0] = 1 << 3
    o3, _, _ = oracle.attend_blasst(q, k, v, idx, B, K, [0, T], math.exp(-2.5), scale=1.0,
                                    flip=flip)
    kept = [keys, keys[:6] + [6, 7, 8]]
    z3 = k[kept[1], 0, 0].astype(np.float64)
    p3 = np.exp(z3 - z3.max())
    ref2 = (p3[:, None] * v[kept[1], 0]).sum(0) / p3.sum()
    # at exactly -2.5 the rule keeps block 3 (not below the threshold): the
    # flip skips it
    assert np.allclose(o2[8, 0], ref2, atol=1e-14) and np.allclose(o3[8, 0], o[8, 0], atol=1e-14)


def test_blasst_first_block_kept_and_v_ones():
    q, k, v, idx, cu, B, K = _blasst_case(63)
    ones = np.ones_like(v)
    for lam in (0.3, 0.9, 1.0):
        o, lse, _ = oracle.attend_blasst(q, k, ones, idx, B, K, cu, lam)
        assert np.allclose(o, 1.0, atol=1e-12)
    # lambda = 1: every attended block after the first raises the running max
    o1, l1, _ = oracle.attend_blasst(q, k, v, idx, B, K, cu, 1.0)
    o0, l0 = oracle.attend(q, k, v, idx, B, K, cu)
    assert not np.allclose(o1, o0)             # something was skipped
    assert np.all(l1 <= l0 + 1e-12)            # dropping keys only lowers the LSE


# ------------------------------------------------------- BLASST backward ----
# The BLASST page's sparsity-aware training needs the gradient of the
# skipped softmax: for fixed decisions it is the gradient of attention over
# the kept blocks' keys (the decisions are piecewise constant, as the router
# is).  Pinned against autograd of the library's masked SDPA, central
# differences of the keep-mask forward (pinned above against SDPA), the
# all-kept case and the decisions of the crafted case.
def _blasst_mask(idx, keep, s0, s1, h, B, K):
    L = s1 - s0
    m = np.zeros((L, L), bool)
    for tl in range(L):
        i = tl // B
        row, kp = idx[s0 + tl, h], keep[s0 + tl, h]
        own_kept = True
        for p in range(K):
            j = row[p]
            if j == i:
                own_kept = bool(kp[p])
            elif 0 <= j < i and kp[p]:
                m[tl, j * B:min((j + 1) * B, L)] = True
        if own_kept:
            m[tl, i * B:tl + 1] = True
    return m


def test_blasst_bwd_all_kept_is_plain_backward():
    q, k, v, idx, cu, B, K = _blasst_case(64)
    do = _bf16(_rand(q.shape, 65))
    plain = oracle.attend_bwd(q, k, v, idx, do, B, K, cu)
    kept = oracle.attend_bwd(q, k, v, idx, do, B, K, cu, keep=np.ones(idx.shape, bool))
    assert all(np.array_equal(a, b) for a, b in zip(plain, kept))


@pytest.mark.parametrize("seed", [66, 67])
def test_blasst_bwd_matches_autograd_of_masked_sdpa(seed):
    """Random keep choices (own blocks dropped in some rows); rows whose
    every block is dropped have no keys and a zero dq."""
    q, k, v, idx, cu, B, K = _blasst_case(seed)
    T, H, d = q.shape
    do = _bf16(_rand(q.shape, seed + 10))
    keep = np.random.default_rng(seed).random(idx.shape) < 0.6
    own_dropped = 0
    scale = 0.37
    dq, dk, dv = oracle.attend_bwd(q, k, v, idx, do, B, K, cu, scale=scale, keep=keep)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        for h in range(H):
            m = _blasst_mask(idx, keep, s0, s1, h, B, K)
            own_dropped += int(sum(not m[t, t] for t in range(s1 - s0)))
            rows = m.any(1)
            tq, tk, tv = (torch.from_numpy(x[s0:s1, h]).double().requires_grad_() for x in (q, k, v))
            mm = torch.from_numpy(m)
            o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mm[None],
                                               scale=scale)[0]
            # keyless rows come out NaN from SDPA; they carry no gradient
            o = torch.where(torch.from_numpy(rows)[:, None], o, torch.zeros_like(o))
            o.backward(torch.from_numpy(do[s0:s1, h]).double())
            for ours, ref in ((dq, tq), (dk, tk), (dv, tv)):
                g = ref.grad.numpy()
                assert np.allclose(ours[s0:s1, h], np.nan_to_num(g, nan=0.0), rtol=1e-10, atol=1e-12)
            assert np.all(dq[s0:s1, h][~rows] == 0.0)
    assert own_dropped > 0


def test_blasst_bwd_matches_central_differences():
    B, K = 4, 3
    q, k, v, do, cu = _bwd_case(80, T=24, H=1, d=4, cu=(0, 24))
    idx, *_ = oracle.route(q, oracle.centroids(k, B, cu), B, K, cu)
    keep = np.random.default_rng(8).random(idx.shape) < 0.7
    keep[:, :, 0] = True                       # no row without keys
    grads = dict(zip("qkv", oracle.attend_bwd(q, k, v, idx, do, B, K, cu, keep=keep)))
    base = {"q": q, "k": k, "v": v}

    def loss(x):
        o, _, _ = oracle.attend_blasst(x["q"], x["k"], x["v"], idx, B, K, cu, 0.0, keep=keep)
        return float(np.sum(o * do.astype(np.float64)))

    g = np.random.default_rng(6)
    for name in "qkv":
        for _ in range(12):
            t, c = int(g.integers(0, 24)), int(g.integers(0, 4))
            xp = {n: a.copy() for n, a in base.items()}
            xm = {n: a.copy() for n, a in base.items()}
            xp[name][t, 0, c] += np.float32(1e-3)
            xm[name][t, 0, c] -= np.float32(1e-3)
            step = float(xp[name][t, 0, c]) - float(xm[name][t, 0, c])
            fd = (loss(xp) - loss(xm)) / step
            assert abs(fd - grads[name][t, 0, c]) <= 1e-5 * max(1.0, abs(fd)), (name, t, c)


def test_blasst_decisions_output():
    """The decisions attend_blasst reports, on the crafted case of
    test_blasst_crafted_skips (block 3 skipped for t = 8 and 9), and on a
    random case where feeding them back as keep reproduces O and LSE."""
    B, K = 2, 5
    firsts = [[1.0, 0.0], [3.0, -1.0], [2.5, 2.0], [0.5, 0.0], [2.2, 9.0]]
    T = 10
    q = np.zeros((T, 1, 2), np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((T, 1, 2), np.float32)
    for j, (a, b) in enumerate(firsts):
        k[2 * j, 0, 0], k[2 * j + 1, 0, 0] = a, b
    v = _rand((T, 1, 2), 62)
    idx = np.full((T, 1, K), -1, np.int32)
    idx[8] = [[0, 1, 2, 3, 4]]
    idx[:8] = [[0, -1, -1, -1, -1]]
    idx[9] = idx[8]
    *_, kp = oracle.attend_blasst(q, k, v, idx, B, K, [0, T], math.exp(-1.0), scale=1.0,
                                  return_keep=True)
    assert kp[8, 0].tolist() == [True, True, True, False, True] == kp[9, 0].tolist()
    assert kp[0, 0].tolist() == [True, False, False, False, False]
    # random: the decisions fed back reproduce the rule's result exactly
    q, k, v, idx, cu, B, K = _blasst_case(68)
    o, lse, _, kp = oracle.attend_blasst(q, k, v, idx, B, K, cu, 0.2, return_keep=True)
    assert not kp[idx >= 0].all() and not kp[idx < 0].any()
    o2, l2, _ = oracle.attend_blasst(q, k, v, idx, B, K, cu, 0.0, keep=kp)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
