"""Seeded random sweep of the support matrix on the GPU: every case draws a
dtype, head dim, block size, top-k, head count, a ragged varlen batch
(empty and one-token sequences included), an optional key convolution
(width 1..8, plain or k + SiLU) and a softmax scale, runs the whole forward
through the C ABI and checks it against the oracle to the same bar as the
fixed cases: k' bit-exact, the selection on every row (P3: exact, or a valid
tolerant top-(k-1) at an oracle near-tie), O and LSE on every row against
the oracle's attention on the GPU's selection.  Every third case also runs
the attention backward (dq, dk', dv against the oracle's fp64 gradients for
the same selection).  Cases follow the pages' task definition ("Optimizing
Mixture of Block Attention", summary page, "Definizione del Compito") and
key convolution ("Progettazione della Convoluzione delle Chiavi
(Appendice B)")."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
import test_blasst_gpu as tbl  # noqa: E402
import test_bwd_gpu as tb  # noqa: E402
import test_parity_gpu as tp  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NCASES = int(os.environ.get("MOBA_SWEEP_CASES", "192"))   # more cases on request
FIRST = int(os.environ.get("MOBA_SWEEP_FIRST", "0"))      # index of the first case
NBLASST = int(os.environ.get("MOBA_SWEEP_BLASST_CASES", "48"))


def _draw(i):
    """Case i of the sweep: a shape inside the support matrix."""
    g = np.random.default_rng(7100 + i)
    dtype = "bf16" if g.random() < 0.7 else "f32"
    d = int(g.choice([64, 128]))
    Bs = [64, 128, 256] + ([512] if dtype == "bf16" else [])
    B = int(g.choice(Bs))
    ab = min(B, 64 if (dtype == "f32" and d == 128) else 128)
    kmax = min(8 if B > 128 else 32, 32 // (B // ab))
    K = int(g.integers(1, kmax + 1))
    H = int(g.integers(1, 4))
    nseq = int(g.integers(1, 5))
    lens = [int(x) for x in g.integers(0, 1600, size=nseq)]
    if g.random() < 0.3:
        lens[int(g.integers(0, nseq))] = int(g.choice([0, 1, B - 1, B + 1]))
    if sum(lens) == 0:
        lens[0] = B + 3
    W = int(g.integers(1, 9)) if g.random() < 0.4 else 0
    mode = "silu_residual" if (W and g.random() < 0.4) else "plain"
    scale = float(g.uniform(0.05, 0.3)) if g.random() < 0.3 else None
    return dict(dtype=dtype, d=d, B=B, K=K, H=H, lens=lens, W=W, mode=mode, scale=scale)


@pytest.mark.parametrize("i", range(FIRST, FIRST + NCASES))
def test_random_shape_matches_oracle(i):
    c = _draw(i)
    print(f"[sweep {i}] {c}", flush=True)
    dtype, d, B, K, H, lens = c["dtype"], c["d"], c["B"], c["K"], c["H"], c["lens"]
    T = sum(lens)
    g = torch.Generator().manual_seed(9300 + i)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((T, H, d), generator=g).to(dt)
    k = torch.randn((T, H, d), generator=g).to(dt)
    v = torch.randn((T, H, d), generator=g).to(dt)
    w = torch.randn((H, d, c["W"]), generator=g) / max(c["W"], 1) ** 0.5 if c["W"] else None
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    mode = 0 if c["mode"] == "plain" else 1
    ref = oracle.forward(q, k, v, B, K, cu, conv_w=w, conv_mode=mode,
                         round_bf16=(dtype == "bf16"), scale=c["scale"] or 0.0)
    m = tp.moba()
    gq, gk, gv = (t.to(DEV) for t in (q, k, v))
    o, lse, idx, kk = m.moba_fwd(gq, gk, gv, B, K, conv_w=None if w is None else w.to(DEV),
                                 conv_mode=c["mode"], cu_seqlens=cu, scale=c["scale"])
    torch.cuda.synchronize()
    if w is not None:
        got = tp._np(kk).reshape(ref["k_conv"].shape)
        assert np.array_equal(got, ref["k_conv"]), f"k' differs in {int((got != ref['k_conv']).sum())} elements"
    # the drawn softmax scales reach 3.4x 1/sqrt(d): outputs near single v
    # rows, |O| up to ~4, so the O bar counts the error beyond O's own bf16
    # rounding, and the backward's max bar is 1.5e-2 (~8u) where the scale is
    # sharper than 1/sqrt(d) (fewer keys average out the bf16 roundings of
    # P and dS); the mean bars are unchanged
    sharp = c["scale"] is not None and c["scale"] > d ** -0.5
    tp._verify_forward(o, lse, idx, ref, q, ref["k_conv"], v, B, K, cu, dtype, f"sweep {i}",
                       scale=c["scale"] or 0.0, out_round=(dtype == "bf16"))
    if w is not None:
        # key conv backward for a drawn dL/dk' (the fixed conv cases' bar:
        # dk one rounding to the I/O dtype, dw within 1e-5 of max |dw|)
        gkc = torch.randn((T, H, d), generator=g).to(dt)
        dkx, dwx = m.moba_key_conv_bwd(gk, w.to(DEV), gkc.to(DEV), B, c["mode"], cu_seqlens=cu)
        torch.cuda.synchronize()
        rkx, rwx = oracle.key_conv_bwd(k, w.numpy(), gkc, cu, mode)
        ekx = np.abs(tp._np(dkx).reshape(-1, H, d).astype(np.float64) - rkx)
        rel = 2.0 ** -8 if dtype == "bf16" else 1e-6
        assert np.all(ekx <= rel * np.abs(rkx) + 1e-6 * np.abs(rkx).max()), f"sweep {i} conv dk max err {ekx.max():.3e}"
        ewx = np.abs(dwx.cpu().numpy().astype(np.float64) - rwx)
        assert ewx.max() <= 1e-5 * max(np.abs(rwx).max(), 1e-30), f"sweep {i} conv dw max err {ewx.max():.3e}"
    if i % 3:
        return
    # backward for the GPU's selection (equal to the oracle's: exactness was
    # asserted above), on the convolved keys the forward attended
    do = torch.randn((T, H, d), generator=g).to(dt)
    kc = torch.from_numpy(ref["k_conv"]).to(dt)
    dq, dk, dv = m.moba_attn_bwd(gq, kc.to(DEV), gv, idx, o, lse, do.to(DEV), B, K,
                                 cu_seqlens=cu, scale=c["scale"])
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attend_bwd(q, kc, v, ref["idx"], do, B, K, cu, scale=c["scale"] or 0.0)
    # bound for an exactly-zero reference (every query attends one key): dS
    # is the difference of two fp32 dot products over d channels, each
    # within about d 2^-24 sum |dO_c v_c|; dq / dk' scale it by the softmax
    # scale and |k| / |q| (8x margin)
    sc = c["scale"] or d ** -0.5
    mag = d * float(do.float().abs().max()) * float(v.float().abs().max())
    ztol = 8 * d * 2.0 ** -24 * mag * sc * max(float(kc.float().abs().max()), float(q.float().abs().max()))
    for got, r, what in ((dq, rq, "dq"), (dk, rk, "dk'"), (dv, rv, "dv")):
        tb._check(f"sweep {i}", tp._np(got).reshape(-1, H, d), r, what, dtype, zero_tol=ztol,
                  max_bar=1.5e-2 if (sharp and dtype == "bf16") else None)


@pytest.mark.parametrize("i", range(FIRST, FIRST + NBLASST))
def test_random_blasst_matches_oracle(i):
    """The BLASST skip ("BLASST", summary page, "Meccanismo di Pruning") on a
    drawn shape: blocks the attention kernels take whole (B <= 128; 64 for
    fp32 at d = 128), a drawn lambda, the default scale; the bar and the
    treatment of near-threshold decisions are those of test_blasst_gpu."""
    c = _draw(i)
    dtype, d, K, H, lens = c["dtype"], c["d"], c["K"], c["H"], c["lens"]
    B = min(c["B"], 64 if (dtype == "f32" and d == 128) else 128)
    lam = float(np.random.default_rng(9900 + i).uniform(0.05, 0.95))
    print(f"[sweep-blasst {i}] {dict(c, B=B)} lambda={lam:.3f}", flush=True)
    T = sum(lens)
    g = torch.Generator().manual_seed(9300 + i)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = {n: torch.randn((T, H, d), generator=g).to(dt) for n in ("q", "k", "v")}
    x["do"] = torch.randn((T, H, d), generator=g).to(dt)
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    x["cu_seqlens"] = cu
    # every third case also runs the BLASST backward on the GPU's decisions
    tbl.check_blasst(x, cu, B, K, lam, dtype, f"sweep-blasst {i}", bwd=(i % 3 == 0))
