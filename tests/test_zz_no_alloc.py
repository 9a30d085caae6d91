"""moba_route_topk_noalloc -- the routing call for callers that cannot
allocate -- against moba_route_topk on the same inputs: the selections are
integers and must be identical, on two calls in a row (the second on a
smaller problem, so the fixed scratch still holds the first call's larger
contents) and on head_dim 128."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(name, seq):
    s = workloads.spec(name).scaled(seq, "-noalloc")
    x = workloads.make(s)
    q = x["q"].to(DEV)
    k = x["k"].to(DEV)
    return s, q, k, x["cu_seqlens"]


def test_route_noalloc_equals_route_topk():
    import block_sparse_long_key_amd as moba
    for name, seq in (("H", 16384), ("C4", 4096), ("C5", 8192)):
        s, q, k, cu = _case(name, seq)
        print(f"[noalloc {name} {seq}]", flush=True)
        B, K = s.block_size, s.top_k
        cent = moba.moba_centroids(k, B, cu)
        ref = moba.moba_route_topk(q, cent, B, K, cu)
        out = torch.full_like(ref, -7)
        got = moba.moba_route_topk_noalloc(q, cent, B, K, cu, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref), f"{name}: {(got != ref).any(-1).sum().item()} rows differ"
