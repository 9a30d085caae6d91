"""GPU parity of the larger-block variants (summary page, "Configurazione
MoBA": MoBA-256 with B=256 k=4 and MoBA-512 with B=512 k=2, both at 7/8
sparsity) against the oracle, which works on the blocks as given.

The library routes on the large blocks and attends each selected block as
its 128-key sub-blocks (the own block split into the sub-blocks before the
query's own sub-block, plus that sub-block token-causally).  The oracle
knows nothing of sub-blocks, so agreement checks that re-expression as well
as the kernels.  Bars are those of the B=128 tests: identical selections
(a differing near-tie row would also have to be valid), O / LSE within the
forward bar, dq / dk / dv within the backward bar.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_bwd_gpu import _check as _check_grad
from test_parity_gpu import _check_o, _verify_forward

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def moba():
    import block_sparse_long_key_amd as m
    return m


def _spec(base, seq=None, heads=None, seqlens=None, **kw):
    s = workloads.spec(base)
    if seqlens is not None:
        s = dataclasses.replace(s, batch=1, seq=sum(seqlens), seqlens=tuple(seqlens))
    elif seq is not None:
        s = s.scaled(seq)
    if heads is not None:
        s = dataclasses.replace(s, heads=heads)
    return dataclasses.replace(s, name=s.name + "-lb", **kw)


CASES = {
    "M256-8k": _spec("M256", seq=8192, heads=4),
    "M512-8k": _spec("M512", seq=8192, heads=4),
    "M256-ragged": _spec("M256", seqlens=(1, 300, 513, 1000, 0, 255), heads=2),
    "M512-ragged": _spec("M512", seqlens=(700, 1500), heads=2),
    "B256-top1": _spec("M256", seq=2048, heads=2, top_k=1),
    "B512-top8-d128": _spec("M512", seq=4096, heads=2, top_k=8, head_dim=128),
    "B256-f32": _spec("M256", seq=2048, heads=2, top_k=3, dtype="f32"),
    "B256-conv": _spec("M256", seq=4096, heads=2, conv_width=3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_large_block_forward_and_backward(name):
    s = CASES[name]
    print(f"[large {name}] {s}", flush=True)
    x = workloads.make(s)
    cu = workloads.segments(s)
    B, K = s.block_size, s.top_k
    ref = oracle.forward(x["q"], x["k"], x["v"], B, K, cu, conv_w=x["conv_w"],
                         round_bf16=(s.dtype == "bf16"))
    m = moba()
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(DEV)
    cus = x["cu_seqlens"]
    # whole forward on the GPU: selection (every row equal to the oracle's)
    # and output against the oracle on the same selection
    o, lse, idx, kk = m.moba_fwd(q, k, v, B, K, conv_w=w, cu_seqlens=cus)
    torch.cuda.synchronize()
    H, d = s.heads, s.head_dim
    _verify_forward(o, lse, idx, ref, x["q"], ref["k_conv"], x["v"], B, K, cu, s.dtype, name)
    # attention on the oracle's selection (so near-tie rows cannot matter)
    idx_ref = torch.from_numpy(ref["idx"]).reshape(tuple(q.shape[:-1]) + (K,)).to(DEV)
    o2, lse2 = m.moba_attn_fwd(q, kk, v, idx_ref, B, K, cu_seqlens=cus)
    torch.cuda.synchronize()
    _check_o(o2, lse2, ref["o"], ref["lse"], s.dtype, what=name)
    # backward on the oracle's selection
    do = workloads.grad_output(s)
    dq, dk, dv = m.moba_attn_bwd(q, kk, v, idx_ref, o2, lse2, do.to(DEV), B, K, cu_seqlens=cus)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attend_bwd(x["q"], ref["k_conv"], x["v"], ref["idx"], do, B, K, cu)
    for g, r, wname in zip((dq, dk, dv), (rq, rk, rv), ("dq", "dk", "dv")):
        _check_grad(name, g.detach().float().cpu().numpy().reshape(-1, H, d), r, wname, s.dtype)
