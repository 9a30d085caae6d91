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
"""
import dataclasses
import itertools

import numpy as np
import pytest
import torch

import oracle
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
}


def _bits(x):
    return [b for b in range(64) if (int(x) >> b) & 1]


def check_blasst(x, cu, B, K, lam, dtype, name, min_changed=0.0):
    """moba_attn_fwd_blasst on the oracle's selection against
    oracle.attend_blasst (x: the CPU inputs q, k, v and cu_seqlens as
    workloads.make gives them; cu: the token segments)."""
    H, d = x["q"].shape[-2], x["q"].shape[-1]
    idx, *_ = oracle.route(x["q"], oracle.centroids(x["k"], B, cu), B, K, cu)
    ro, rl, near = oracle.attend_blasst(x["q"], x["k"], x["v"], idx, B, K, cu, lam)
    po, pl = oracle.attend(x["q"], x["k"], x["v"], idx, B, K, cu)
    changed = np.any(np.abs(ro - po) > 0, axis=-1).mean()
    print(f"[blasst {name}] rows with a skipped block {changed:.3f}; flagged rows "
          f"{int((near != 0).sum())}", flush=True)
    assert changed >= min_changed, "the rule skipped (almost) nothing: the case tests nothing"
    m = moba()
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    gi = torch.from_numpy(idx).reshape(tuple(q.shape[:-1]) + (K,)).to(DEV)
    o, lse = m.moba_attn_fwd_blasst(q, k, v, gi, B, K, lam, cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    go = _np(o).reshape(-1, H, d).astype(np.float64)
    gl = _np(lse).reshape(-1, H).astype(np.float64)
    ref_o, ref_l = ro.copy(), rl.copy()
    # flagged rows: the resolution of their flagged decisions closest to the GPU
    rows = np.argwhere(near != 0)
    for t, h in rows:
        nb = _bits(near[t, h])
        assert len(nb) <= 4, f"row {t},{h}: {len(nb)} flagged decisions"
        best = None
        for n in range(1, len(nb) + 1):
            for sub in itertools.combinations(nb, n):
                flip = np.zeros(near.shape, np.uint64)
                flip[t, h] = sum(1 << b for b in sub)
                ao, al, _ = oracle.attend_blasst(x["q"], x["k"], x["v"], idx, B, K, cu, lam,
                                                 flip=flip)
                err = np.abs(go[t, h] - ao[t, h]).max()
                if best is None or err < best[0]:
                    best = (err, ao[t, h], al[t, h])
        if np.abs(go[t, h] - ro[t, h]).max() > best[0]:
            ref_o[t, h], ref_l[t, h] = best[1], best[2]
    mx, mean, ltol = (2e-2, 2e-3, 1e-3) if dtype == "bf16" else (1e-4, 1e-4, 1e-5)
    err = np.abs(go - ref_o)
    assert err.max() <= mx, f"{name}: max |O err| {err.max():.3e}"
    assert err.mean() <= mean, f"{name}: mean |O err| {err.mean():.3e}"
    assert np.abs(gl - ref_l).max() <= ltol, f"{name}: max |LSE err| {np.abs(gl - ref_l).max():.3e}"


@pytest.mark.parametrize("name", list(CASES))
def test_blasst_matches_oracle(name):
    s, lam = CASES[name]
    print(f"[blasst {name}] {s} lambda={lam}", flush=True)
    x = workloads.make(s)
    check_blasst(x, workloads.segments(s), s.block_size, s.top_k, lam, s.dtype, name,
                 min_changed=0.01)


def test_blasst_lambda_zero_is_the_plain_forward():
    s = _spec("H", seq=4096, heads=2)
    x = workloads.make(s)
    m = moba()
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    o, lse, idx, _ = m.moba_fwd(q, k, v, s.block_size, s.top_k)
    o0, lse0, idx0, _ = m.moba_fwd(q, k, v, s.block_size, s.top_k, blasst_lambda=0.0)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(o, o0) and torch.equal(lse, lse0)


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
