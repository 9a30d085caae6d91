"""GPU parity of the BLASST block skip on MoBA's selected blocks
(moba_attn_fwd_blasst) against the oracle's attend_blasst.

"BLASST: Dynamic BLocked Attention Sparsity via Softmax Thresholding",
section "Meccanismo di Pruning": a query's blocks are visited in order with
a running maximum; a block whose own maximum is below it by more than
ln(1/lambda) is skipped.  Here the blocks are the query's selected blocks in
ascending order, its own block last.

Bar: a row's skip decisions are integers decided from floating-point block
maxima, so a decision within rounding of the threshold may go either way:
the oracle flags each such decision (within 1e-4 * max(1, |M|)), and a
flagged row must match the oracle under one of the resolutions of its
flagged decisions; every other row must match the oracle's own decisions.
O: max |err| <= 2e-2, mean |err| <= 2e-3 (bf16), <= 1e-4 (fp32); LSE <= 1e-3
(bf16), 1e-5 (fp32) -- the forward's bar.  lambda = 0 keeps every block and
must equal moba_attn_fwd bitwise.  Both sides attend the oracle's own
selection (which the router reproduces exactly).

The forward's kept selection (kept_idx) is checked the same way: rows the
oracle does not flag keep exactly the oracle's blocks, flagged rows the
blocks of one resolution of their flagged decisions.  The BLASST backward
(moba_attn_bwd_blasst, the page's sparsity-aware training) is compared with
the oracle's backward on the GPU's own decisions (like against like), with
the plain backward's bar: max |err| <= 1e-2 max |ref|, mean |err| <=
4e-3 mean |ref| (bf16); 1e-4 / 1e-5 (fp32).
"""
import dataclasses
import itertools

import numpy as np
import pytest
import torch

import oracle
import test_bwd_gpu as tb
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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
    return dataclasses.replace(s, conv_width=0, plant=False, name=s.name + "-blasst", **kw)


CASES = {
    "Hs-lam0.5": (_spec("H", seq=8192, heads=4), 0.5),
    "Hs-lam0.9": (_spec("H", seq=8192, heads=4), 0.9),
    "Hs-lam1": (_spec("H", seq=4096, heads=2), 1.0),
    "C4s-lam0.7": (_spec("C4", seq=8192, heads=2), 0.7),
    "varlen-d128-B64": (_spec("C5", seqlens=(3000, 129, 0, 2000), heads=2, block_size=64,
                              top_k=6), 0.6),
    "sink-lam0.3": (_spec("H", seq=4096, heads=2, sink=True), 0.3),
    "f32-C1": (_spec("C1"), 0.8),
    "f32-d128-B64": (_spec("C5", seqlens=(700, 65, 500), heads=2, block_size=64, top_k=5,
                           dtype="f32"), 0.7),
    # 150 ragged sequences (some empty): the calls run as groups of 64
    "many-seqs": (_spec("H", seqlens=tuple((53 * i) % 400 for i in range(150)), heads=2,
                        block_size=64, top_k=4), 0.5),
}


def _bits(x):
    return [b for b in range(64) if (int(x) >> b) & 1]


def _keep_of(kept, idx):
    """Per-slot decisions of a kept selection: slot p of idx is kept iff its
    block is listed in the kept row."""
    return (idx[..., :, None] == kept[..., None, :]).any(-1) & (idx >= 0)


def _check_kept_format(kept, idx):
    """Rows ascending, -1 padded, a subset of idx's blocks, the first listed
    block kept (BLASST never skips the first block it visits)."""
    K = idx.shape[-1]
    kr, ir = kept.reshape(-1, K), idx.reshape(-1, K)
    n = (kr >= 0).sum(1)
    pos = np.arange(K)[None, :]
    assert np.all((kr >= 0) == (pos < n[:, None])), "kept rows are not -1 padded"
    v = np.where(kr >= 0, kr, np.iinfo(np.int32).max)
    assert np.all(np.diff(v, axis=1)[(pos[:, 1:] < n[:, None])] > 0), "kept rows not ascending"
    assert np.all(_keep_of(kr, ir).sum(1) == n), "kept rows name blocks outside idx"
    first = ir[:, 0] >= 0
    assert np.all(kr[first, 0] == ir[first, 0]), "the first visited block was skipped"


def check_blasst(x, cu, B, K, lam, dtype, name, min_changed=0.0, bwd=False):
    """moba_attn_fwd_blasst on the oracle's selection against
    oracle.attend_blasst (x: the CPU inputs q, k, v and cu_seqlens as
    workloads.make gives them; cu: the token segments); its kept selection
    against the oracle's decisions; with bwd, moba_attn_bwd_blasst against
    oracle.attend_bwd on the GPU's decisions."""
    H, d = x["q"].shape[-2], x["q"].shape[-1]
    idx, *_ = oracle.route(x["q"], oracle.centroids(x["k"], B, cu), B, K, cu)
    ro, rl, near, rkeep = oracle.attend_blasst(x["q"], x["k"], x["v"], idx, B, K, cu, lam,
                                               return_keep=True)
    po, pl = oracle.attend(x["q"], x["k"], x["v"], idx, B, K, cu)
    changed = np.any(np.abs(ro - po) > 0, axis=-1).mean()
    print(f"[blasst {name}] rows with a skipped block {changed:.3f}; flagged rows "
          f"{int((near != 0).sum())}", flush=True)
    assert changed >= min_changed, "the rule skipped (almost) nothing: the case tests nothing"
    m = moba()
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    gi = torch.from_numpy(idx).reshape(tuple(q.shape[:-1]) + (K,)).to(DEV)
    o, lse, kept = m.moba_attn_fwd_blasst(q, k, v, gi, B, K, lam, cu_seqlens=x["cu_seqlens"],
                                          return_kept=True)
    torch.cuda.synchronize()
    go = _np(o).reshape(-1, H, d).astype(np.float64)
    gl = _np(lse).reshape(-1, H).astype(np.float64)
    gk = kept.cpu().numpy().reshape(idx.shape)
    _check_kept_format(gk, idx)
    gkeep = _keep_of(gk, idx)
    ref_o, ref_l = ro.copy(), rl.copy()
    plain = near == 0
    bad = np.argwhere(plain & np.any(gkeep != rkeep, axis=-1))
    assert len(bad) == 0, f"{name}: {len(bad)} unflagged rows keep other blocks, first {bad[:3]}"
    # flagged rows: the resolution of their flagged decisions closest to the
    # GPU.  A row's resolutions take every non-empty subset of its flagged
    # decisions the other way; flips act per row, so the c-th subset of
    # every flagged row goes into one oracle call.
    rows = [tuple(r) for r in np.argwhere(near != 0)]
    subsets = {}
    for t, h in rows:
        nb = _bits(near[t, h])
        assert len(nb) <= 4, f"row {t},{h}: {len(nb)} flagged decisions"
        subsets[(t, h)] = [sum(1 << b for b in sub) for n in range(1, len(nb) + 1)
                           for sub in itertools.combinations(nb, n)]
    best = {r: None for r in rows}
    keeps = {r: [rkeep[r]] for r in rows}
    for c in range(max((len(v) for v in subsets.values()), default=0)):
        flip = np.zeros(near.shape, np.uint64)
        for r, sub in subsets.items():
            if c < len(sub):
                flip[r] = sub[c]
        ao, al, _, ak = oracle.attend_blasst(x["q"], x["k"], x["v"], idx, B, K, cu, lam,
                                             flip=flip, return_keep=True)
        for r, sub in subsets.items():
            if c >= len(sub):
                continue
            keeps[r].append(ak[r])
            err = np.abs(go[r] - ao[r]).max()
            if best[r] is None or err < best[r][0]:
                best[r] = (err, ao[r], al[r])
    for r in rows:
        if np.abs(go[r] - ro[r]).max() > best[r][0]:
            ref_o[r], ref_l[r] = best[r][1], best[r][2]
        assert any(np.array_equal(gkeep[r], kk) for kk in keeps[r]), \
            f"{name}: flagged row {r} keeps blocks no resolution keeps"
    mx, mean, ltol = (2e-2, 2e-3, 1e-3) if dtype == "bf16" else (1e-4, 1e-4, 1e-5)
    err = np.abs(go - ref_o)
    assert err.max() <= mx, f"{name}: max |O err| {err.max():.3e}"
    assert err.mean() <= mean, f"{name}: mean |O err| {err.mean():.3e}"
    assert np.abs(gl - ref_l).max() <= ltol, f"{name}: max |LSE err| {np.abs(gl - ref_l).max():.3e}"
    if not bwd:
        return
    # the backward on the GPU's decisions
    do = x["do"]
    dog = do.to(DEV)
    dq, dk, dv = m.moba_attn_bwd_blasst(q, k, v, kept, o, lse, dog, B, K,
                                        cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    own_dropped = int(np.sum(~gkeep & (idx == (_local_block(cu, B, idx.shape[0])[:, None, None]))))
    print(f"[blasst-bwd {name}] rows whose own block was skipped: {own_dropped}", flush=True)
    ref = oracle.attend_bwd(x["q"], x["k"], x["v"], idx, do, B, K, cu, keep=gkeep)
    # the plain backward's per-tensor bar; an exactly-zero reference (every
    # query left with one key) gets the rounding bound of the two fp32 dot
    # products that form dS, as in the sweep
    mag = d * float(do.float().abs().max()) * float(x["v"].float().abs().max())
    ztol = 8 * d * 2.0 ** -24 * mag * d ** -0.5 * max(float(x["k"].float().abs().max()),
                                                      float(x["q"].float().abs().max()))
    for g, r, w in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        tb._check(f"blasst-bwd {name}", _np(g).reshape(-1, H, d), r, w, dtype, zero_tol=ztol)


def _local_block(cu, B, T):
    """Each token's own block (local to its sequence)."""
    out = np.zeros(T, np.int64)
    for a, b in zip(cu[:-1], cu[1:]):
        out[a:b] = np.arange(b - a) // B
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_blasst_matches_oracle(name):
    s, lam = CASES[name]
    print(f"[blasst {name}] {s} lambda={lam}", flush=True)
    x = workloads.make(s)
    x["do"] = workloads.grad_output(s)
    check_blasst(x, workloads.segments(s), s.block_size, s.top_k, lam, s.dtype, name,
                 min_changed=0.01, bwd=True)


def test_blasst_lambda_zero_is_the_plain_forward():
    s = _spec("H", seq=4096, heads=2)
    x = workloads.make(s)
    m = moba()
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o, lse, idx, _ = m.moba_fwd(q, k, v, s.block_size, s.top_k)
    o0, lse0, idx0, _ = m.moba_fwd(q, k, v, s.block_size, s.top_k, blasst_lambda=0.0)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(o, o0) and torch.equal(lse, lse0)


def test_blasst_lambda_zero_backward_is_the_plain_backward():
    """lambda = 0: the kept selection is idx itself and the BLASST backward
    on it equals moba_attn_bwd bitwise (every row lists its own block)."""
    s = _spec("H", seq=4096, heads=2)
    x = workloads.make(s)
    m = moba()
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    do = workloads.grad_output(s).to(DEV)
    o, lse, idx, _ = m.moba_fwd(q, k, v, s.block_size, s.top_k)
    o0, lse0, kept = m.moba_attn_fwd_blasst(q, k, v, idx, s.block_size, s.top_k, 0.0,
                                            return_kept=True)
    g = m.moba_attn_bwd(q, k, v, idx, o, lse, do, s.block_size, s.top_k)
    gb = m.moba_attn_bwd_blasst(q, k, v, kept, o0, lse0, do, s.block_size, s.top_k)
    torch.cuda.synchronize()
    assert torch.equal(kept, idx)
    assert all(torch.equal(a, b) for a, b in zip(g, gb))


def test_blasst_autograd_wrapper():
    """moba_attention(blasst_lambda=...) runs the BLASST forward and, on
    backward, moba_attn_bwd_blasst on the forward's kept selection."""
    s = _spec("H", seq=2048, heads=2)
    x = workloads.make(s)
    m = moba()
    q, k, v = (x[n].to(DEV).requires_grad_() for n in ("q", "k", "v"))
    do = workloads.grad_output(s).to(DEV)
    o, lse = m.moba_attention(q, k, v, s.block_size, s.top_k, blasst_lambda=0.5)
    o.backward(do)
    with torch.no_grad():
        o2, lse2, kept, _ = m.moba_fwd(q, k, v, s.block_size, s.top_k, blasst_lambda=0.5)
        g = m.moba_attn_bwd_blasst(q, k, v, kept, o2, lse2, do, s.block_size, s.top_k)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for a, b in zip((q.grad, k.grad, v.grad), g):
        assert torch.equal(a, b)


def test_blasst_rejects_bad_lambda_and_large_blocks():
    m = moba()
    s = _spec("M256", seq=2048, heads=2)
    x = workloads.make(s)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    idx = torch.zeros(q.shape[:-1] + (s.top_k,), dtype=torch.int32, device=DEV)
    with pytest.raises(m.MobaError):
        m.moba_attn_fwd_blasst(q, k, v, idx, 256, s.top_k, 0.5)
    with pytest.raises(m.MobaError):
        m.moba_attn_fwd_blasst(q, k, v, idx, 128, s.top_k, 1.5)
    torch.cuda.synchronize()
