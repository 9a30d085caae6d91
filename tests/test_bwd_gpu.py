"""GPU parity of the attention backward (moba_attn_bwd) against the oracle.

The HIP path's forward (o, lse) feeds its backward, as in training; the
oracle recomputes everything in fp64 from q, k, v, the selection and dO.
Both sides get the same seeded inputs (workloads) and the oracle's own
selection.

Bar for bf16 (from the arithmetic: each output is rounded once to bf16,
u = 2^-9, which alone gives a mean relative error near 0.7u; P and dS enter
the products as bf16 and D_t comes from the bf16 forward output, each a
further O(u) per term with random signs): for each of dq, dk, dv,
    max |err| <= 1e-2 * max |ref|  (about 5u)   and
    mean |err| <= 4e-3 * mean |ref| (about 2u).
At full size the oracle covers sampled rows (dq) and sampled key blocks
(dk, dv); every row is checked against the sum invariants
sum_u dv_u = sum_t dO_t and sum_u dk_u = 0 per (sequence, head).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_REL, MEAN_REL = 1e-2, 4e-3


def moba():
    import block_sparse_long_key_amd as m
    return m


def _np(t):
    return t.detach().float().cpu().numpy()


def _spec(base, seq=None, heads=None, seqlens=None, **kw):
    s = workloads.spec(base)
    if seqlens is not None:
        s = dataclasses.replace(s, batch=1, seq=sum(seqlens), seqlens=tuple(seqlens))
    elif seq is not None:
        s = s.scaled(seq)
    if heads is not None:
        s = dataclasses.replace(s, heads=heads)
    return dataclasses.replace(s, conv_width=0, plant=False, name=s.name + "-bwd", **kw)


CASES = {
    "H-2k": _spec("H", seq=2048, heads=4),
    "C4-4k": _spec("C4", seq=4096, heads=2),
    "C5-4k": _spec("C5", seq=4096, heads=2),
    "d128-B64-ragged": _spec("C5", seqlens=(1000, 777), heads=2, block_size=64, top_k=4),
    # fp32 at d = 128: 128-key blocks attended as 64-key sub-blocks
    "f32-d128-B128": _spec("C5", seqlens=(700, 330), heads=2, block_size=128, top_k=6, dtype="f32"),
    "ragged": _spec("H", seqlens=(1, 127, 129, 700, 0, 300), heads=2),
    "top1": _spec("H", seq=1000, heads=2, top_k=1),
    "top32-B64": _spec("C4", seq=4096, heads=1, top_k=32),
    # 1094 key blocks: more than 1024, so the index pass takes chunks of 128
    # query blocks instead of 32
    "long-B64": _spec("C4", seq=70000, heads=1, top_k=8),
    # 150 ragged sequences (some empty): more than one launch table holds,
    # so the call runs as groups of 64 with one workspace region each
    "many-seqs": _spec("H", seqlens=tuple((41 * i) % 300 for i in range(150)), heads=2,
                       block_size=64, top_k=4),
    # fp32 inputs (the plain recompute path)
    "f32-C1": _spec("C1"),
    "f32-B128": _spec("H", seq=1500, heads=2, dtype="f32"),
    "f32-varlen-d128": _spec("C5", seqlens=(300, 129, 0, 640), heads=2, block_size=64, top_k=4,
                             dtype="f32"),
}
# fp32: every product and sum in fp32 against the oracle's fp64
MAX_REL_F32, MEAN_REL_F32 = 1e-4, 1e-5


def _run(s):
    x = workloads.make(s)
    cu = workloads.segments(s)
    do = workloads.grad_output(s)
    B, K = s.block_size, s.top_k
    idx, *_ = oracle.route(x["q"], oracle.centroids(x["k"], B, cu), B, K, cu)
    m = moba()
    q, k, v, dog = (t.to(DEV) for t in (x["q"], x["k"], x["v"], do))
    idx_g = torch.from_numpy(idx).reshape(tuple(q.shape[:-1]) + (K,)).to(DEV)
    cus = x["cu_seqlens"]
    o, lse = m.moba_attn_fwd(q, k, v, idx_g, B, K, cu_seqlens=cus)
    dq, dk, dv = m.moba_attn_bwd(q, k, v, idx_g, o, lse, dog, B, K, cu_seqlens=cus)
    torch.cuda.synchronize()
    return x, cu, do, idx, (dq, dk, dv)


def _check(name, got, ref, what, dtype="bf16", zero_tol=None, max_bar=None):
    """Per-tensor relative bar (R25).  A reference that is exactly zero has no
    scale for it: when every query attends a single key, O = v and dS =
    P (dO.v - dO.O) vanishes, so dq and dk' are zero up to the rounding of
    the two fp32 dot products; then |got| must stay within zero_tol, the
    caller's bound on that rounding."""
    bar_max, bar_mean = (MAX_REL, MEAN_REL) if dtype == "bf16" else (MAX_REL_F32, MEAN_REL_F32)
    if max_bar is not None:
        bar_max = max_bar
    err = np.abs(got.astype(np.float64) - ref)
    if np.abs(ref).max() == 0.0:
        print(f"[{name}] {what}: zero reference, max|got| {err.max():.2e} (bound {zero_tol})", flush=True)
        assert zero_tol is not None and err.max() <= zero_tol, f"{name} {what}: max|got| {err.max():.3e}"
        return
    mx_rel = err.max() / max(np.abs(ref).max(), 1e-30)
    mean_rel = err.mean() / max(np.abs(ref).mean(), 1e-30)
    print(f"[{name}] {what}: max|err|/max|ref| {mx_rel:.2e}  mean|err|/mean|ref| {mean_rel:.2e}",
          flush=True)
    assert mx_rel <= bar_max, f"{name} {what}: max rel {mx_rel:.3e}"
    assert mean_rel <= bar_mean, f"{name} {what}: mean rel {mean_rel:.3e}"


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_matches_oracle(name):
    s = CASES[name]
    print(f"[bwd {name}] {s}", flush=True)
    x, cu, do, idx, got = _run(s)
    H, d = s.heads, s.head_dim
    ref = oracle.attend_bwd(x["q"], x["k"], x["v"], idx, do, s.block_size, s.top_k, cu)
    for g, r, w in zip(got, ref, ("dq", "dk", "dv")):
        _check(name, _np(g).reshape(-1, H, d), r, w, s.dtype)


def test_bwd_repeatable():
    """Two runs give bitwise-equal dq, dk, dv: each (query, slot) dq piece is
    computed alone and the pieces are added in slot order; the backward's
    index pass places each list's entries in an order that depends only on
    idx, so dK / dV sum the same rows in the same tiles every time."""
    for name in ("H-2k", "C4-4k", "long-B64", "f32-varlen-d128"):
        s = CASES[name]
        x, cu, do, idx, a = _run(s)
        _, _, _, _, b = _run(s)
        for u, w, n in zip(a, b, ("dq", "dk", "dv")):
            assert torch.equal(u, w), f"{name} {n} differs between runs"


def test_bwd_full_size_sampled():
    s = dataclasses.replace(workloads.spec("H"))
    print(f"[bwd full {s.name}] {s}", flush=True)
    x, cu, do, idx, got = _run(s)
    H, d, B = s.heads, s.head_dim, s.block_size
    dq, dk, dv = (_np(t).reshape(-1, H, d).astype(np.float64) for t in got)
    T = dq.shape[0]
    dof = do.float().numpy().reshape(-1, H, d).astype(np.float64)
    # invariants on every row
    for si in range(len(cu) - 1):
        a, b = cu[si], cu[si + 1]
        sv = dv[a:b].sum(0)
        assert np.all(np.abs(sv - dof[a:b].sum(0)) <= 2 ** -7 * np.abs(dv[a:b]).sum(0) + 1e-3)
        assert np.all(np.abs(dk[a:b].sum(0)) <= 2 ** -7 * np.abs(dk[a:b]).sum(0) + 1e-3)
    # sampled rows and key blocks against the oracle
    g = np.random.default_rng(11)
    qsel = np.zeros((T, H), bool)
    qsel.reshape(-1)[g.choice(T * H, 1024, replace=False)] = True
    nb = oracle.total_blocks(cu, B)
    kbsel = np.zeros((nb, H), bool)
    for h in range(H):
        kbsel[g.choice(nb), h] = True
        kbsel[0, h] = True if h == 0 else kbsel[0, h]     # the most-routed-to block
    ref = oracle.attend_bwd(x["q"], x["k"], x["v"], idx, do, B, s.top_k, cu,
                            qsel=qsel, kbsel=kbsel)
    _check("H", dq[qsel], ref[0][qsel], "dq (sampled rows)")
    boff = np.concatenate([[0], np.cumsum([-(-(cu[i + 1] - cu[i]) // B) for i in range(len(cu) - 1)])])
    tok_blk = np.empty(T, np.int64)
    for si in range(len(cu) - 1):
        tl = np.arange(cu[si + 1] - cu[si])
        tok_blk[cu[si]:cu[si + 1]] = boff[si] + tl // B
    km = kbsel[tok_blk]                      # [T, H]
    _check("H", dk[km], ref[1][km], "dk (sampled blocks)")
    _check("H", dv[km], ref[2][km], "dv (sampled blocks)")


# ------------------------------------------------ key-convolution backward
CONV_CASES = {
    # name: (spec, mode, width override)
    "C3-plain-W3": (_spec("C3", seq=4096, heads=4), "plain", 3),
    "C5-plain-W4-d128": (_spec("C5", seq=8192, heads=2), "plain", 4),
    "silu-W3-ragged": (_spec("H", seqlens=(1, 127, 129, 700, 0, 300), heads=2), "silu_residual", 3),
    "W1": (_spec("H", seq=1000, heads=2), "plain", 1),
    "W8-silu": (_spec("H", seq=1000, heads=2), "silu_residual", 8),
    "W2-silu": (_spec("H", seq=1000, heads=2), "silu_residual", 2),
    "W5-ragged": (_spec("H", seqlens=(1, 127, 129, 700), heads=2), "plain", 5),
    "W6-silu": (_spec("H", seq=1000, heads=2), "silu_residual", 6),
    "W7": (_spec("H", seq=1000, heads=2), "plain", 7),
    # rows of 2048 channels: plain convs of up to 4 taps run 8 channels per thread
    "wide-W2-d128": (_spec("C5", seqlens=(300, 129, 211), heads=16), "plain", 2),
    "wide-W4-d128": (_spec("C5", seqlens=(700,), heads=16), "plain", 4),
    "wide-W5-d128": (_spec("C5", seqlens=(500,), heads=16), "plain", 5),
    "wide-f32-W3": (dataclasses.replace(_spec("C5", seqlens=(400,), heads=16), dtype="f32", block_size=64), "plain", 3),
    "f32-W4": (_spec("C1"), "plain", 4),
    "C3-full-W3": (dataclasses.replace(workloads.spec("C3"), plant=False), "plain", 3),
    # 150 ragged sequences: dw sums every group's block partials in one pass
    "many-seqs-W4": (_spec("H", seqlens=tuple((41 * i) % 300 for i in range(150)), heads=2,
                           block_size=64, top_k=4), "plain", 4),
}


@pytest.mark.parametrize("name", list(CONV_CASES))
def test_key_conv_bwd_matches_oracle(name):
    s, mode, W = CONV_CASES[name]
    print(f"[conv bwd {name}] {s} mode={mode} W={W}", flush=True)
    x = workloads.make(s)
    cu = workloads.segments(s)
    g = workloads.grad_output(s)
    gen = torch.Generator().manual_seed(s.seed + 20011)
    w = torch.randn((s.heads, s.head_dim, W), generator=gen) * (1.0 / W) ** 0.5
    m = moba()
    dk, dw = m.moba_key_conv_bwd(x["k"].to(DEV), w.to(DEV), g.to(DEV), s.block_size, mode,
                                 cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    rk, rw = oracle.key_conv_bwd(x["k"], w.numpy(), g, cu, 0 if mode == "plain" else 1)
    H, d = s.heads, s.head_dim
    dk = _np(dk).reshape(-1, H, d).astype(np.float64)
    dw = dw.cpu().numpy().astype(np.float64)
    # dk: fp32 sums rounded once to the I/O dtype
    rel = 2.0 ** -8 if s.dtype == "bf16" else 1e-6
    ek = np.abs(dk - rk)
    assert np.all(ek <= rel * np.abs(rk) + 1e-6 * np.abs(rk).max()), \
        f"dk max err {ek.max():.3e}"
    # dw: fp32 per key block, fp64 across blocks
    ew = np.abs(dw - rw)
    print(f"[conv bwd {name}] dk max err {ek.max():.2e}  dw max err / max |dw| "
          f"{ew.max() / np.abs(rw).max():.2e}", flush=True)
    assert ew.max() <= 1e-5 * np.abs(rw).max()


# ------------------------------------------------------- attention sink ----
SINK_CASES = {
    "sink-B128": _spec("H", seq=8192, heads=2, sink=True),
    "sink-B64-varlen": _spec("C4", seqlens=(5000, 3000), heads=2, sink=True),
}


@pytest.mark.parametrize("name", list(SINK_CASES))
def test_attention_sink_long_lists(name):
    """Block 0 is selected by (nearly) every query, so its list holds ~all
    queries of the sequence: several forward work items of one list and one
    long backward list.  Selection, forward and backward against the
    oracle."""
    s = SINK_CASES[name]
    print(f"[sink {name}] {s}", flush=True)
    x = workloads.make(s)
    cu = workloads.segments(s)
    B, K, H, d = s.block_size, s.top_k, s.heads, s.head_dim
    ref = oracle.forward(x["q"], x["k"], x["v"], B, K, cu)
    sel0 = np.mean([(ref["idx"][cu[i] + B:cu[i + 1]] == 0).any(-1).mean()
                    for i in range(len(cu) - 1)])
    assert sel0 > 0.95, f"sink not formed ({sel0:.2f})"
    m = moba()
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    cus = x["cu_seqlens"]
    cent = m.moba_centroids(k, B, cus)
    idx = m.moba_route_topk(q, cent, B, K, cus)
    torch.cuda.synchronize()
    from test_parity_gpu import _assert_exact, _check_o, _check_sel
    _assert_exact(_check_sel(idx.cpu().numpy(), ref["idx"], ref["exempt"], x["q"], ref["cent"], B,
                             K, cu, what=name), name)
    idx_ref = torch.from_numpy(ref["idx"]).reshape(tuple(q.shape[:-1]) + (K,)).to(DEV)
    o, lse = m.moba_attn_fwd(q, k, v, idx_ref, B, K, cu_seqlens=cus)
    do = workloads.grad_output(s)
    dq, dk, dv = m.moba_attn_bwd(q, k, v, idx_ref, o, lse, do.to(DEV), B, K, cu_seqlens=cus)
    torch.cuda.synchronize()
    _check_o(o, lse, ref["o"], ref["lse"], s.dtype, what=name)
    rq, rk, rv = oracle.attend_bwd(x["q"], x["k"], x["v"], ref["idx"], do, B, K, cu)
    for g_, r_, w_ in zip((dq, dk, dv), (rq, rk, rv), ("dq", "dk", "dv")):
        _check(name, _np(g_).reshape(-1, H, d), r_, w_)


# ------------------------------------------------------- autograd wrapper --
@pytest.mark.parametrize("conv", [None, "plain"])
def test_autograd_wrapper_matches_the_oracle(conv):
    """moba_attention as a torch autograd op: o.backward(dO) gives the
    oracle's gradients for q, v, k (through the key conv when there is one)
    and the conv filter.  (The plain conv's k' is bit-exact, so the GPU's own
    selection equals the oracle's; the k + SiLU form's gradient is checked
    in the conv tests above.)"""
    s = _spec("H", seq=2048, heads=2)
    if conv is not None:
        s = dataclasses.replace(s, conv_width=3, conv_mode=conv)
    x = workloads.make(s)
    cu = workloads.segments(s)
    B, K, H, d = s.block_size, s.top_k, s.heads, s.head_dim
    do = workloads.grad_output(s)
    m = moba()
    q, k, v = (x[n].to(DEV).requires_grad_() for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(DEV).requires_grad_()
    o, lse = m.moba_attention(q, k, v, B, K, conv_w=w, conv_mode=s.conv_mode)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    mode = 0 if s.conv_mode == "plain" else 1
    ref = oracle.forward(x["q"], x["k"], x["v"], B, K, cu, conv_w=x["conv_w"], conv_mode=mode)
    gi = m.moba_route_topk(q.detach(), m.moba_centroids(
        m.moba_key_conv(k.detach(), w.detach(), B, s.conv_mode) if w is not None else k.detach(), B),
        B, K)
    assert np.array_equal(gi.cpu().numpy().reshape(ref["idx"].shape), ref["idx"])
    rq, rkk, rv = oracle.attend_bwd(x["q"], ref["k_conv"], x["v"], ref["idx"], do, B, K, cu)
    _check(f"autograd-{conv}", _np(q.grad).reshape(-1, H, d), rq, "dq")
    _check(f"autograd-{conv}", _np(v.grad).reshape(-1, H, d), rv, "dv")
    if w is None:
        _check(f"autograd-{conv}", _np(k.grad).reshape(-1, H, d), rkk, "dk")
        return
    # chain through the conv from the oracle's dk'.  The GPU rounds dk' to
    # bf16 before the conv backward and dk again after it: two roundings,
    # so twice the single-rounding bar
    rk, rw = oracle.key_conv_bwd(x["k"], x["conv_w"].numpy(), rkk.astype(np.float32), cu, mode)
    gk = _np(k.grad).reshape(-1, H, d).astype(np.float64)
    ek = np.abs(gk - rk)
    print(f"[autograd-{conv}] dk max {ek.max() / np.abs(rk).max():.2e} "
          f"mean {ek.mean() / np.abs(rk).mean():.2e}", flush=True)
    assert ek.max() <= 2 * MAX_REL * np.abs(rk).max()
    assert ek.mean() <= 2 * MEAN_REL * np.abs(rk).mean()
    ew = np.abs(w.grad.cpu().numpy() - rw)
    assert ew.max() <= 1e-2 * np.abs(rw).max(), ew.max()
