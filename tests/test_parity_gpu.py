"""GPU parity: the HIP MoBA forward against the CPU oracle.

Bars (fixed before the kernels were written):
  * key conv (plain) and centroids: bit-exact;
  * block selection: identical rows; a row may differ only where the
    oracle's (k-1)-th and k-th past scores are within 1e-5 relative
    (near-tie), and then it must still be a valid tolerant top-(k-1) of the
    oracle's fp64 scores (tests/parity.py checks every such row);
  * O: max |err| <= 2e-2 and mean |err| <= 2e-3 for bf16, max |err| <= 1e-4
    for fp32; LSE: <= 1e-3 (bf16) / 1e-5 (fp32) -- against the oracle's
    attention on the same selection (the GPU's own row where it differs);
  * the router claims an exact selection, so every test also asserts that
    no row differs at all (after the checks above have run).
Inputs are the seeded synthetic workloads (same generator on both sides).
Oracle results never come from the GPU: where the attention stage is tested
alone, it is fed the oracle's own selection.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def moba():
    import block_sparse_long_key_amd as m
    return m


def _np(t):
    return t.detach().float().cpu().numpy()


def _tol(dtype):
    return (2e-2, 2e-3, 1e-3) if dtype == "bf16" else (1e-4, 1e-4, 1e-5)


def _flat(x, H):
    a = _np(x)
    return a.reshape(-1, H, a.shape[-1])


def _check_o(o_gpu, lse_gpu, o_ref, lse_ref, dtype, rows=None, what="", out_round=False):
    """O and LSE against the oracle.  out_round: the max bar counts only the
    error beyond the rounding of each output to bf16 itself (half an ulp of
    |O_ref|), which no bf16 result can avoid and which the absolute bar
    leaves out once |O| grows past 1 (sharp softmax scales)."""
    mx, mean, ltol = _tol(dtype)
    o = _np(o_gpu).reshape(o_ref.shape[0], -1, o_ref.shape[-1]) if rows is None else o_gpu
    err = np.abs(o.astype(np.float64) - o_ref)
    if out_round:
        half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 1e-30))) - 8)
        over = (err - half_ulp).max()
        assert over <= mx, f"{what} max |O err| beyond the output rounding {over:.3e} > {mx}"
    else:
        assert err.max() <= mx, f"{what} max |O err| {err.max():.3e} > {mx}"
    assert err.mean() <= mean, f"{what} mean |O err| {err.mean():.3e} > {mean}"
    if lse_gpu is not None:
        l = _np(lse_gpu).reshape(lse_ref.shape) if rows is None else lse_gpu
        lerr = np.abs(l.astype(np.float64) - lse_ref)
        assert lerr.max() <= ltol, f"{what} max |LSE err| {lerr.max():.3e} > {ltol}"


def _check_sel(gidx, ref_idx, exempt, q, cent, B, K, cu, rows=None, what=""):
    """P3 on every given row (see tests/parity.py); returns the global ids
    of the rows that differ from the oracle (each a valid near-tie row)."""
    return parity.check_selection(gidx, ref_idx, exempt, q, cent, B, K, cu, rows=rows, what=what)


def _assert_exact(drows, what):
    assert len(drows) == 0, (f"{what}: {len(drows)} near-tie rows differ from the oracle "
                             f"(valid, but the router claims an exact selection)")


def _verify_forward(o, lse, idx, ref, q, kc, v, B, K, cu, dtype, what, scale=0.0, out_round=False):
    """Whole-array check of one forward: selection (P3) on every row, O and
    LSE (P4) on every row against the oracle's attention on the same
    selection (the GPU's own row where the selections differ), then
    exactness of the selection."""
    H, d = ref["o"].shape[-2], ref["o"].shape[-1]
    T = ref["o"].shape[0]
    gi = idx.cpu().numpy().reshape(-1, K)
    drows = _check_sel(gi, ref["idx"], ref["exempt"], q, ref["cent"], B, K, cu, what=what)
    o_ref = ref["o"].reshape(-1, d)
    lse_ref = ref["lse"].reshape(-1)
    if len(drows):
        o_ref, lse_ref = o_ref.copy(), lse_ref.copy()
        ro, rl = parity.outputs_on_gpu_selection(q, kc, v, gi.reshape(T, H, K), B, K, cu, drows,
                                                 scale=scale)
        o_ref[drows], lse_ref[drows] = ro, rl
    _check_o(_np(o).reshape(-1, d), None if lse is None else _np(lse).reshape(-1), o_ref, lse_ref,
             dtype, rows=True, what=what, out_round=out_round)
    _assert_exact(drows, what)


SMALL = {
    "C1": workloads.spec("C1"),
    "C2": workloads.spec("C2"),
    "C3s": workloads.spec("C3").scaled(4096),
    "C4s": workloads.spec("C4").scaled(8192),
    "C5s": workloads.spec("C5").scaled(8192),
    "Hs": workloads.spec("H").scaled(8192),
}


@pytest.fixture(scope="module")
def cases():
    cache = {}

    def get(name):
        if name not in cache:
            s = SMALL[name]
            print(f"[case {name}] {s}", flush=True)
            x = workloads.make(s)
            cu = workloads.segments(s)
            ref = oracle.forward(x["q"], x["k"], x["v"], s.block_size, s.top_k, cu,
                                 conv_w=x["conv_w"], round_bf16=(s.dtype == "bf16"))
            cache[name] = (s, x, cu, ref)
        return cache[name]
    return get


def _gpu_inputs(s, x):
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(DEV)
    return q, k, v, w, x["cu_seqlens"]


@pytest.mark.parametrize("name", ["C3s", "C5s"])
def test_key_conv_bitexact(cases, name):
    s, x, cu, ref = cases(name)
    q, k, v, w, cus = _gpu_inputs(s, x)
    kk, cent = moba().moba_key_conv(k, w, s.block_size, "plain", cus, with_centroids=True)
    torch.cuda.synchronize()
    assert np.array_equal(_flat(kk, s.heads), ref["k_conv"])
    assert np.array_equal(_np(cent), ref["cent"])
    kk2 = moba().moba_key_conv(k, w, s.block_size, "plain", cus)
    assert torch.equal(kk, kk2)


@pytest.mark.parametrize("name", list(SMALL))
def test_centroids_bitexact(cases, name):
    s, x, cu, ref = cases(name)
    q, k, v, w, cus = _gpu_inputs(s, x)
    if w is not None:
        k = moba().moba_key_conv(k, w, s.block_size, "plain", cus)
    cent = moba().moba_centroids(k, s.block_size, cus)
    torch.cuda.synchronize()
    assert np.array_equal(_np(cent), ref["cent"])


@pytest.mark.parametrize("name", list(SMALL))
def test_route_matches_oracle(cases, name):
    s, x, cu, ref = cases(name)
    q, k, v, w, cus = _gpu_inputs(s, x)
    cent = torch.from_numpy(ref["cent"]).to(DEV)
    idx = moba().moba_route_topk(q, cent, s.block_size, s.top_k, cus)
    torch.cuda.synchronize()
    drows = _check_sel(idx.cpu().numpy(), ref["idx"], ref["exempt"], x["q"], ref["cent"],
                       s.block_size, s.top_k, cu, what=name)
    print(f"[{name}] rows differing: {len(drows)}; near-tie rows: {int(ref['exempt'].sum())}")
    # the router re-scores near-ties in fp64 in the oracle's order: no row may differ
    _assert_exact(drows, name)


@pytest.mark.parametrize("name", list(SMALL))
def test_attention_on_oracle_selection(cases, name):
    s, x, cu, ref = cases(name)
    q, k, v, w, cus = _gpu_inputs(s, x)
    kk = torch.from_numpy(ref["k_conv"]).to(s.torch_dtype).to(DEV).reshape(k.shape)
    idx = torch.from_numpy(ref["idx"]).to(DEV).reshape(q.shape[:-1] + (s.top_k,))
    o, lse = moba().moba_attn_fwd(q, kk, v, idx, s.block_size, s.top_k, cu_seqlens=cus)
    torch.cuda.synchronize()
    _check_o(o, lse, ref["o"], ref["lse"], s.dtype, what=name)


@pytest.mark.parametrize("name", list(SMALL))
def test_full_forward_matches_oracle(cases, name):
    s, x, cu, ref = cases(name)
    q, k, v, w, cus = _gpu_inputs(s, x)
    o, lse, idx, kk = moba().moba_fwd(q, k, v, s.block_size, s.top_k, conv_w=w, cu_seqlens=cus)
    torch.cuda.synchronize()
    _verify_forward(o, lse, idx, ref, x["q"], ref["k_conv"], x["v"], s.block_size, s.top_k, cu,
                    s.dtype, name)


def test_deterministic_bitwise(cases):
    s, x, cu, ref = cases("Hs")
    q, k, v, w, cus = _gpu_inputs(s, x)
    a = moba().moba_fwd(q, k, v, s.block_size, s.top_k)
    b = moba().moba_fwd(q, k, v, s.block_size, s.top_k)
    c = moba().fwd(q, k, v, s.block_size, s.top_k)         # (o, lse, idx)
    torch.cuda.synchronize()
    for x1, x2 in zip(a, b):
        assert torch.equal(x1, x2)
    assert len(c) == 3
    for x1, x3 in zip(a, c):
        assert torch.equal(x1, x3)


# ------------------------------------------------------------ edge cases --
def _run_case(seqlens, H, d, B, K, dtype, seed, conv_w_width=0, scale=None, v_ones=False):
    tokens = sum(seqlens)
    g = torch.Generator().manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.randn((tokens, H, d), generator=g).to(dt)
    k = torch.randn((tokens, H, d), generator=g).to(dt)
    v = torch.ones((tokens, H, d)).to(dt) if v_ones else torch.randn((tokens, H, d), generator=g).to(dt)
    w = None
    if conv_w_width:
        w = torch.randn((H, d, conv_w_width), generator=g) / math.sqrt(conv_w_width)
    cu = [0]
    for L in seqlens:
        cu.append(cu[-1] + L)
    ref = oracle.forward(q, k, v, B, K, cu, conv_w=w, round_bf16=(dtype == "bf16"),
                         scale=scale or 0.0)
    gq, gk, gv = (t.to(DEV) for t in (q, k, v))
    gw = None if w is None else w.to(DEV)
    o, lse, idx, kk = moba().moba_fwd(gq, gk, gv, B, K, conv_w=gw, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    if conv_w_width:
        assert np.array_equal(_np(kk), ref["k_conv"]), "k' differs from the oracle's"
    _verify_forward(o, lse, idx, ref, q, ref["k_conv"], v, B, K, cu, dtype,
                    f"edge {seqlens[:8]} B{B} K{K} {dtype}", scale=scale or 0.0)
    return o, lse, idx, ref


@pytest.mark.parametrize("period,seq,B,K", [(3, 4096, 64, 8), (5, 8192, 64, 16), (40, 8192, 64, 8)])
def test_route_exact_ties(period, seq, B, K):
    """Keys that repeat block by block with a period give bit-identical
    centroids, so each query sees classes of exactly tied scores and the
    lower block index must win.  Period 3 makes tie classes of up to ~n/3
    blocks: more than fit the router's candidate window, so both the in-kernel
    fp64 re-selection and the separate re-selection kernel are exercised."""
    H, d = 2, 64
    print(f"[ties period {period} seq {seq} B{B} K{K}]", flush=True)
    g = torch.Generator().manual_seed(1000 + period)
    q = torch.randn((seq, H, d), generator=g).to(torch.bfloat16)
    base = torch.randn((period * B, H, d), generator=g).to(torch.bfloat16)
    nblk = seq // B
    k = torch.cat([base[(j % period) * B:(j % period + 1) * B] for j in range(nblk)])
    cu = [0, seq]
    cent = oracle.centroids(k, B, cu)
    ref_idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    idx = moba().moba_route_topk(q.to(DEV), torch.from_numpy(cent).to(DEV), B, K, cu)
    torch.cuda.synchronize()
    got = idx.cpu().numpy().reshape(ref_idx.shape)
    drows = _check_sel(got, ref_idx, ex, q, cent, B, K, cu, what=f"ties period {period}")
    print(f"[ties period {period}] rows differing: {len(drows)}; near-tie rows: {int(ex.sum())}")
    assert ex.sum() > 0
    _assert_exact(drows, f"ties period {period}")


def test_route_one_lane_holds_the_top_k():
    """Blocks whose id mod 16 is below 4 score highest, so one of the four
    lanes that share a query holds the whole top-k: more than the lane keeps,
    which must be detected and re-selected exactly."""
    H, d, B, K, seq = 2, 64, 64, 8, 4096
    print(f"[lane overflow B{B} K{K}]", flush=True)
    g = torch.Generator().manual_seed(77)
    q = (torch.randn((seq, H, d), generator=g) * 0.1 + 1.0).to(torch.bfloat16)
    k = torch.randn((seq, H, d), generator=g) * 0.1
    blk = torch.arange(seq) // B
    k += torch.where((blk % 16) < 4, 1.0, -1.0)[:, None, None]
    k = k.to(torch.bfloat16)
    cu = [0, seq]
    cent = oracle.centroids(k, B, cu)
    ref_idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    idx = moba().moba_route_topk(q.to(DEV), torch.from_numpy(cent).to(DEV), B, K, cu)
    torch.cuda.synchronize()
    got = idx.cpu().numpy().reshape(ref_idx.shape)
    # the construction does put all k-1 routed blocks of late rows in one
    # lane (a lane scores the blocks j with the same (j mod 16) / 4)
    late = ref_idx[B * 40:, :, :K - 1]
    assert np.all((late % 16) < 4)
    _assert_exact(_check_sel(got, ref_idx, ex, q, cent, B, K, cu, what="lane overflow"),
                  "lane overflow")


@pytest.mark.parametrize("seq,B,K", [(65536, 64, 8), (65536, 64, 16), (40000, 64, 6)])
def test_route_long_scan_every_row(seq, B, K):
    """A 1024-block sequence: block ids take 10 key bits, so a few percent of
    the rows are flagged and most of them go through the fix kernel's fp64
    re-scoring of their best 2k-4 blocks against the bound on all others
    (k = 6 is the smallest k with room for that).  Every row must equal the
    oracle's selection."""
    H, d = 1, 64
    print(f"[long scan seq {seq} B{B} K{K}]", flush=True)
    g = torch.Generator().manual_seed(seq + K)
    q = torch.randn((seq, H, d), generator=g).to(torch.bfloat16)
    k = torch.randn((seq, H, d), generator=g).to(torch.bfloat16)
    cu = [0, seq]
    cent = oracle.centroids(k, B, cu)
    ref_idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    idx = moba().moba_route_topk(q.to(DEV), torch.from_numpy(cent).to(DEV), B, K, cu)
    torch.cuda.synchronize()
    got = idx.cpu().numpy().reshape(ref_idx.shape)
    drows = _check_sel(got, ref_idx, ex, q, cent, B, K, cu, what=f"long scan K{K}")
    print(f"[long scan K{K}] rows differing: {len(drows)}; near-tie rows: {int(ex.sum())}")
    _assert_exact(drows, f"long scan K{K}")


@pytest.mark.parametrize("K", [6, 7, 8, 16])
def test_route_all_scores_tied_in_the_first_blocks(K):
    """Every query scores every past block equally (all key blocks share one
    centroid; a third of the query rows are zero): the oracle keeps the k-1
    lowest block ids.  The first query blocks (i <= 16) have fewer past
    blocks than the router's candidate lists hold, so its masked ids beyond
    i and its fp64 re-scoring of the best 2k-4 blocks meet here; every row
    must equal the oracle's."""
    H, d, B, seq = 3, 64, 64, 64 * 40
    print(f"[all tied K{K}]", flush=True)
    g = torch.Generator().manual_seed(500 + K)
    q = torch.randn((seq, H, d), generator=g)
    q[::3] = 0.0
    q = q.to(torch.bfloat16)
    k = torch.randn((B, H, d), generator=g).repeat(seq // B, 1, 1).to(torch.bfloat16)
    cu = [0, seq]
    cent = oracle.centroids(k, B, cu)
    ref_idx, ga, gb, ex = oracle.route(q, cent, B, K, cu)
    assert np.all(ref_idx[B * K:, :, :K - 1] == np.arange(K - 1))
    idx = moba().moba_route_topk(q.to(DEV), torch.from_numpy(cent).to(DEV), B, K, cu)
    torch.cuda.synchronize()
    got = idx.cpu().numpy().reshape(ref_idx.shape)
    drows = _check_sel(got, ref_idx, ex, q, cent, B, K, cu, what=f"all tied K{K}")
    _assert_exact(drows, f"all tied K{K}")


@pytest.mark.parametrize("seqlens,H,d,B,K,dtype", [
    ([1000], 2, 64, 64, 4, "bf16"),           # ragged tail (1000 = 15*64 + 40)
    ([130, 1, 64, 300], 3, 64, 128, 8, "bf16"),  # short / single-token sequences
    ([777, 0, 513], 2, 128, 128, 3, "bf16"),  # empty sequence in a varlen batch, d=128
    ([2048], 2, 64, 64, 1, "bf16"),           # k = 1: own block only
    ([1024], 2, 64, 128, 32, "bf16"),         # k >= n: dense causal
    ([640], 2, 64, 64, 32, "f32"),            # fp32, k > blocks
    ([1000], 1, 128, 64, 5, "f32"),           # fp32, d = 128, ragged
    ([4096], 1, 64, 64, 32, "bf16"),          # maximum k
    ([(53 * i) % 257 for i in range(64)], 2, 64, 64, 4, "bf16"),  # 64 sequences (one launch table), one empty
    ([(53 * i) % 257 for i in range(200)], 2, 64, 64, 4, "bf16"),  # 200 sequences: 4 groups of <= 64
    ([(29 * i) % 150 for i in range(70)], 1, 128, 64, 3, "f32"),    # 70 sequences, fp32, d = 128
    # fp32 at d = 128 attends 64-key sub-blocks of larger blocks
    ([700, 330], 2, 128, 128, 6, "f32"),      # B = 128, ragged, two sequences
    ([1100], 1, 128, 128, 16, "f32"),         # B = 128, k = 16: 32 expanded slots
    ([1000], 1, 128, 128, 1, "f32"),          # B = 128, k = 1: own block split in two
    ([1500], 1, 128, 256, 8, "f32"),          # B = 256: 4 sub-blocks per block
])
def test_edge_cases(seqlens, H, d, B, K, dtype):
    print(f"[edge {seqlens} H{H} d{d} B{B} K{K} {dtype}]", flush=True)
    _run_case(seqlens, H, d, B, K, dtype, seed=sum(seqlens) + K)


def test_many_sequences_with_key_conv():
    """130 varlen sequences with the key conv: k', centroids, selection and
    output of the whole forward equal the oracle's (the call runs as groups
    of at most 64 sequences)."""
    seqlens = [(71 * i) % 400 for i in range(130)]
    print(f"[many seqs conv] {len(seqlens)} sequences", flush=True)
    _run_case(seqlens, 2, 64, 64, 5, "bf16", seed=77, conv_w_width=3)


def test_v_ones_gives_ones():
    o, lse, idx, ref = _run_case([1500], 2, 64, 64, 4, "bf16", seed=11, v_ones=True)
    assert torch.all(o == 1.0)


@pytest.mark.parametrize("name,width", [("C3s", 3), ("Hs", 5)])
def test_conv_silu_residual_bitexact(name, width):
    """The page's k + SiLU(conv) form: k' bit-equal to the oracle's fp64
    evaluation rounded to fp32 and then to bf16 (the kernel's fast path is
    used only where its error bound proves the same rounding), and the
    centroids of k' too."""
    import dataclasses
    s = dataclasses.replace(SMALL[name], conv_width=width, conv_mode="silu_residual")
    x = workloads.make(s)
    cu = workloads.segments(s)
    ref = oracle.key_conv(x["k"], x["conv_w"], cu, mode=1, round_bf16=True)
    kk, cent = moba().moba_key_conv(x["k"].to(DEV), x["conv_w"].to(DEV), s.block_size,
                                    "silu_residual", x["cu_seqlens"], with_centroids=True)
    torch.cuda.synchronize()
    got = _flat(kk, s.heads)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"
    assert np.array_equal(_np(cent), oracle.centroids(ref, s.block_size, cu))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["plain", "silu_residual"])
@pytest.mark.parametrize("width", range(1, 9))
def test_key_conv_every_width_bitexact(width, mode, dtype):
    """Every filter width the kernels are built for (1..8), both forms and
    both I/O dtypes, on two ragged sequences with partial last blocks: k'
    and its centroids bit-equal to the oracle."""
    g = torch.Generator().manual_seed(100 + 10 * width + (mode == "plain"))
    T, H, d, B = 700, 2, 64, 64
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = (torch.randn((T, H, d), generator=g) * 2.0).to(dt)
    w = torch.randn((H, d, width), generator=g) * (1.0 / width) ** 0.5
    cu = [0, 300, T]
    print(f"[conv W={width} {mode} {dtype}]", flush=True)
    ref = oracle.key_conv(k.float(), w, cu, mode=0 if mode == "plain" else 1,
                          round_bf16=dtype == "bf16")
    kk, cent = moba().moba_key_conv(k.to(DEV), w.to(DEV), B, mode, cu, with_centroids=True)
    torch.cuda.synchronize()
    got = _flat(kk, H)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"
    assert np.array_equal(_np(cent), oracle.centroids(ref, B, cu))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("width", [1, 2, 3, 4, 5])
def test_key_conv_wide_rows_bitexact(width, dtype):
    """Token rows of 2048 channels (16 heads x d = 128), where plain convs of
    up to 4 taps and the pooling run 8 channels per thread: k' and the
    centroids bit-equal to the oracle (width 5 takes the 4-channel path on
    the same rows); pooling alone too."""
    g = torch.Generator().manual_seed(200 + width)
    T, H, d = 600, 16, 128
    B = 128 if dtype == "bf16" else 64          # (fp32 at d = 128 takes B = 64)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = (torch.randn((T, H, d), generator=g) * 2.0).to(dt)
    w = torch.randn((H, d, width), generator=g) * (1.0 / width) ** 0.5
    cu = [0, 250, T]
    print(f"[wide conv W={width} {dtype}]", flush=True)
    ref = oracle.key_conv(k.float(), w, cu, mode=0, round_bf16=dtype == "bf16")
    kk, cent = moba().moba_key_conv(k.to(DEV), w.to(DEV), B, "plain", cu, with_centroids=True)
    c0 = moba().moba_centroids(k.to(DEV), B, cu)
    torch.cuda.synchronize()
    got = _flat(kk, H)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} elements differ"
    assert np.array_equal(_np(cent), oracle.centroids(ref, B, cu))
    assert np.array_equal(_np(c0), oracle.centroids(k.float(), B, cu))


def test_conv_silu_residual_fp32_bitexact():
    """fp32 I/O: k' equals the oracle's fp64 formula rounded to fp32."""
    g = torch.Generator().manual_seed(31)
    T, H, d, W = 1500, 2, 64, 4
    k = torch.randn((T, H, d), generator=g) * 3.0
    w = torch.randn((H, d, W), generator=g)
    cu = [0, 700, T]
    ref = oracle.key_conv(k, w, cu, mode=1, round_bf16=False)
    kk = moba().moba_key_conv(k.to(DEV), w.to(DEV), 64, "silu_residual", cu)
    torch.cuda.synchronize()
    assert np.array_equal(_flat(kk, H), ref)


def test_scale_override_and_null_lse():
    o, lse, idx, ref = _run_case([700], 2, 64, 64, 3, "bf16", seed=5, scale=0.3)
    s = workloads.Spec("t", 1, 1, 700, 2, 64, 64, 3, "bf16")
    q = torch.from_numpy(np.zeros((700, 2, 64), np.float32)).to(torch.bfloat16).to(DEV)
    o2, lse2 = moba().moba_attn_fwd(q, q, q, idx, 64, 3, return_lse=False, cu_seqlens=[0, 700])
    torch.cuda.synchronize()
    assert lse2 is None and torch.all(o2 == 0)


# ------------------------------------------------------------ full size ----
def _full_inputs(s):
    x = workloads.make(s)
    cu = workloads.segments(s)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(DEV)
    o, lse, idx, kk = moba().moba_fwd(q, k, v, s.block_size, s.top_k, conv_w=w,
                                      conv_mode=s.conv_mode, cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    return x, cu, o, lse, idx


@pytest.mark.parametrize("name", ["H", "C3", "C4", "C5", "M256", "M512", "H5"])
def test_full_size_every_row(name):
    """Every workload that the oracle finishes in seconds, at its full size
    (H: 64K x 2 x 16 heads, d=64, B=128, top-8 -- the benchmarked launch; C3
    with key conv and the planted signal; C4 with B=64, top-16; C5 varlen
    with d=128 and key conv; M256 / M512: B=256 top-4 and B=512 top-2; H5:
    the kconv5 k + SiLU(conv) form): the whole GPU forward against the whole
    oracle forward, selection and output on every row."""
    s = workloads.spec(name)
    print(f"[full {s.name}] {s}", flush=True)
    x, cu, o, lse, idx = _full_inputs(s)
    ref = oracle.forward(x["q"], x["k"], x["v"], s.block_size, s.top_k, cu, conv_w=x["conv_w"],
                         conv_mode=0 if s.conv_mode == "plain" else 1, round_bf16=True)
    print(f"[full {s.name}] oracle done", flush=True)
    _verify_forward(o, lse, idx, ref, x["q"], ref["k_conv"], x["v"], s.block_size, s.top_k, cu,
                    s.dtype, f"{name} full")


def test_full_size_sampled_long_context():
    """L: one 512K-token sequence, 16 heads (4096 blocks per query at the
    end): the oracle's full routing would take minutes, so invariants run on
    every row on the GPU and selection and output on a seeded sample of rows
    computed one by one by the oracle's row-subset entry points."""
    s = workloads.spec("L")
    print(f"[full {s.name}] {s}", flush=True)
    x, cu, o, lse, idx = _full_inputs(s)
    H, K, B, d = s.heads, s.top_k, s.block_size, s.head_dim
    T = int(cu[-1])
    # invariants on every row (on the GPU)
    gi = idx.reshape(T, H, K)
    tl = torch.cat([torch.arange(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)]).to(DEV)
    own = (tl // B).to(torch.int32)[:, None]
    valid = gi >= 0
    assert torch.all((gi == own[..., None]).any(-1))
    full = valid.all(-1)
    assert torch.all(gi[full][..., 1:] > gi[full][..., :-1])
    assert torch.all(torch.where(valid, gi, torch.zeros_like(gi)) <= own[..., None])
    assert torch.all(valid.sum(-1) == torch.clamp(own + 1, max=K))
    g = np.random.default_rng(0)
    rows = np.unique(np.concatenate([
        g.integers(0, T * H, 1500), np.arange(0, 16), T * H - 1 - np.arange(0, 16)]))
    cent = oracle.centroids(x["k"], B, cu)
    ri, ga, gb, ex = oracle.route_rows(x["q"], cent, B, K, cu, rows)
    gidx = idx.cpu().numpy().reshape(-1, K)
    drows = _check_sel(gidx[rows], ri, ex, x["q"], cent, B, K, cu, rows=rows, what="L sampled")
    # O of the sampled rows: the oracle attends the GPU's selection (equal to
    # its own on every row that P3 did not flag)
    ro, rl = parity.outputs_on_gpu_selection(x["q"], x["k"], x["v"], gidx.reshape(T, H, K), B, K,
                                             cu, rows)
    go = _np(o).reshape(-1, d)[rows]
    gl = _np(lse).reshape(-1)[rows]
    _check_o(go, gl, ro, rl, "bf16", rows=True, what="L sampled")
    _assert_exact(drows, "L sampled")


def test_longest_sequence_sampled():
    """One sequence of 16384 blocks of 64 keys (the most a sequence may
    hold; 1M tokens, one head, top-8): block ids take 14 key bits, the index
    pass stages 16384 counters per workgroup, the backward takes the
    placement for long lists.  Invariants on every row; selection, output
    and the attention gradients (dq of sampled rows, dk / dv of sampled key
    blocks) against the oracle's row and key-block subsets."""
    B, K, d, H = 64, 8, 64, 1
    T = 16384 * B
    print(f"[longest sequence {T} tokens]", flush=True)
    g = torch.Generator().manual_seed(16384)
    q, k, v, do = (torch.randn((T, H, d), generator=g).to(torch.bfloat16) for _ in range(4))
    cu = [0, T]
    m = moba()
    gq, gk, gv, gdo = (t.to(DEV) for t in (q, k, v, do))
    o, lse, idx, _ = m.moba_fwd(gq, gk, gv, B, K, cu_seqlens=cu)
    dq, dk, dv = m.moba_attn_bwd(gq, gk, gv, idx, o, lse, gdo, B, K, cu_seqlens=cu)
    torch.cuda.synchronize()
    gi = idx.reshape(T, K)
    own = (torch.arange(T, device=DEV) // B).to(torch.int32)[:, None]
    assert torch.all((gi == own).any(-1))
    full = (gi >= 0).all(-1)
    assert torch.all(gi[full][:, 1:] > gi[full][:, :-1])
    assert torch.all(torch.where(gi >= 0, gi, torch.zeros_like(gi)) <= own)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.integers(0, T, 1000), T - 1 - np.arange(64)]))
    cent = oracle.centroids(k, B, cu)
    ri, ga, gb, ex = oracle.route_rows(q, cent, B, K, cu, rows)
    gidx = idx.cpu().numpy().reshape(-1, K)
    drows = _check_sel(gidx[rows], ri, ex, q, cent, B, K, cu, rows=rows, what="16384 blocks")
    ro, rl = parity.outputs_on_gpu_selection(q, k, v, gidx.reshape(T, H, K), B, K, cu, rows)
    _check_o(_np(o).reshape(-1, d)[rows], _np(lse).reshape(-1)[rows], ro, rl, "bf16", rows=True,
             what="16384 blocks")
    _assert_exact(drows, "16384 blocks")
    # gradients on the GPU's own selection: dq of the sampled rows, dk / dv
    # of sampled key blocks (block 0 holds the longest list)
    qsel = np.zeros((T, H), bool)
    qsel[rows, 0] = True
    kb = np.zeros((16384, H), bool)
    kb[[0, 1, 5000, 16382, 16383], 0] = True
    rq, rk, rv = oracle.attend_bwd(q, k, v, gidx.reshape(T, H, K), do, B, K, cu, qsel=qsel,
                                   kbsel=kb, nthreads=16)
    from test_bwd_gpu import _check as _check_grad
    _check_grad("16384 blocks", _np(dq).reshape(T, H, d)[rows], rq[rows], "dq")
    keys = np.concatenate([np.arange(j * B, (j + 1) * B) for j in np.nonzero(kb[:, 0])[0]])
    _check_grad("16384 blocks", _np(dk).reshape(T, H, d)[keys], rk[keys], "dk")
    _check_grad("16384 blocks", _np(dv).reshape(T, H, d)[keys], rv[keys], "dv")


def test_binding_rejects_wrong_buffers():
    """Wrong-sized or wrong-typed buffers raise MobaError before any launch."""
    m = moba()
    T, H, d, B, K = 512, 2, 64, 64, 3
    q = torch.zeros(T, H, d, dtype=torch.bfloat16, device=DEV)
    cu = [0, T]
    nb = m.moba_total_blocks(q, B, cu)
    cent = torch.zeros(nb, H, d, dtype=torch.float32, device=DEV)
    idx = torch.zeros(T, H, K, dtype=torch.int32, device=DEV)
    need = m.moba_attn_fwd_workspace_bytes(q, B, K, cu)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    bad = [
        lambda: m.moba_centroids(q, B, cu_seqlens=cu, out=cent[:-1]),
        lambda: m.moba_centroids(q, B, cu_seqlens=cu, out=cent.double()),
        lambda: m.moba_route_topk(q, cent[:, :1], B, K, cu_seqlens=cu),
        lambda: m.moba_route_topk(q, cent, B, K, cu_seqlens=cu, out=idx[:, :, :2]),
        lambda: m.moba_route_topk(q, cent, B, K, cu_seqlens=cu, workspace=ws[:8]),
        lambda: m.moba_attn_fwd(q, q, q, idx.long(), B, K, cu_seqlens=cu),
        lambda: m.moba_attn_fwd(q, q[:-1], q[:-1], idx, B, K, cu_seqlens=cu),
        lambda: m.moba_attn_fwd(q, q, q, idx, B, K, cu_seqlens=cu, out=q.float()),
        lambda: m.moba_attn_fwd(q, q, q, idx, B, K, cu_seqlens=cu, workspace=ws[: need - 1]),
        lambda: m.moba_attn_index(idx[1:], q, B, K, ws, cu_seqlens=cu),
        lambda: m.moba_attn_combine(q, q, q, idx, B, K, ws, q[:-1], cu_seqlens=cu),
        lambda: m.moba_key_conv(q, torch.zeros(H, d, 3, device=DEV), B, cu_seqlens=cu,
                                out=q),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(m.MobaError):
            f()
            pytest.fail(f"case {i} did not raise")
    torch.cuda.synchronize()
