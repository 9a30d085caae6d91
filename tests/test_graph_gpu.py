"""The library's calls only enqueue kernels (no allocation, memset or
synchronisation), so a whole forward and backward can be captured in a HIP
graph and replayed.  Each replay, with eager work and synchronisations in
between, must equal the eager result bitwise (both passes are
deterministic)."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_forward_and_backward_replay_from_a_graph():
    import block_sparse_long_key_amd as moba
    s = workloads.spec("H").scaled(4096, "-graph")
    x = workloads.make(s)
    B, K = s.block_size, s.top_k
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    do = workloads.grad_output(s).to(DEV)
    nb = moba.moba_total_blocks(q, B)
    cent = torch.empty((nb, s.heads, s.head_dim), dtype=torch.float32, device=DEV)
    idx = torch.empty(q.shape[:-1] + (K,), dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    wsf = torch.empty(moba.moba_attn_fwd_workspace_bytes(q, B, K), dtype=torch.uint8, device=DEV)
    wsb = torch.empty(moba.moba_attn_bwd_workspace_bytes(q, B, K), dtype=torch.uint8, device=DEV)
    state = {}

    def step():
        moba.moba_centroids(k, B, out=cent)
        moba.moba_route_topk(q, cent, B, K, out=idx, workspace=wsf)
        _, lse = moba.moba_attn_fwd(q, k, v, idx, B, K, workspace=wsf, out=o)
        state["lse"] = lse
        moba.moba_attn_bwd(q, k, v, idx, o, lse, do, B, K, workspace=wsb, out=grads)

    # eager reference (also warms up the library on this stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, o, state["lse"], *grads)]

    g = torch.cuda.CUDAGraph()
    for t in (idx, o, *grads):
        t.zero_()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (idx, o, *grads):
            t.fill_(7)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [idx, o, state["lse"], *grads]
        for a, b, name in zip(got, ref, ("idx", "o", "lse", "dq", "dk", "dv")):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"


def test_concurrent_streams_match_sequential():
    """Calls keep no state between them: two problems run at the same time on
    two streams, each with its own workspace, give the sequential results
    bitwise (forward and backward)."""
    import block_sparse_long_key_amd as moba
    probs = []
    for name, n in (("H", 4096), ("C5", 6144)):      # C5: 4 sequences, d = 128
        s = workloads.spec(name).scaled(n, "-streams")
        x = workloads.make(s)
        q, k, v = (x[t].to(DEV) for t in ("q", "k", "v"))
        cu = None
        if s.seqlens is not None:
            cu = [0]
            for ln in s.seqlens:
                cu.append(cu[-1] + ln)
        do = workloads.grad_output(s).to(DEV)
        B, K = s.block_size, s.top_k
        wsf = torch.empty(max(moba.moba_attn_fwd_workspace_bytes(q, B, K, cu),
                              moba.moba_route_topk_workspace_bytes(q, B, K, cu), 256),
                          dtype=torch.uint8, device=DEV)
        wsb = torch.empty(moba.moba_attn_bwd_workspace_bytes(q, B, K, cu), dtype=torch.uint8, device=DEV)
        probs.append(dict(q=q, k=k, v=v, do=do, B=B, K=K, cu=cu, wsf=wsf, wsb=wsb))

    def run(p):
        cent = moba.moba_centroids(p["k"], p["B"], cu_seqlens=p["cu"])
        idx = moba.moba_route_topk(p["q"], cent, p["B"], p["K"], cu_seqlens=p["cu"], workspace=p["wsf"])
        o, lse = moba.moba_attn_fwd(p["q"], p["k"], p["v"], idx, p["B"], p["K"], cu_seqlens=p["cu"],
                                    workspace=p["wsf"])
        g = moba.moba_attn_bwd(p["q"], p["k"], p["v"], idx, o, lse, p["do"], p["B"], p["K"],
                               cu_seqlens=p["cu"], workspace=p["wsb"])
        return (idx, o, lse, *g)

    ref = [run(p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in probs]
    for rep in range(3):
        outs = [None] * len(probs)
        for i, (p, st) in enumerate(zip(probs, streams)):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs[i] = run(p)
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        for i in range(len(probs)):
            for a, b, name in zip(outs[i], ref[i], ("idx", "o", "lse", "dq", "dk", "dv")):
                assert torch.equal(a, b), f"problem {i} replay {rep}: {name} differs"


def test_explicit_stream_owns_its_buffers():
    """A call given ``stream=`` (not inside ``torch.cuda.stream``) allocates
    its outputs and workspace on that stream: right after it returns, the
    current stream allocates and overwrites the same amount of memory while
    the call's kernels may still run, and the results must not change."""
    import block_sparse_long_key_amd as moba
    s = workloads.spec("H").scaled(8192, "-explicit-stream")
    x = workloads.make(s)
    B, K = s.block_size, s.top_k
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    ref = moba.moba_fwd(q, k, v, B, K)
    torch.cuda.synchronize()
    need = moba.moba_attn_fwd_workspace_bytes(q, B, K) + 2 * q.numel() * 2
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        got = moba.moba_fwd(q, k, v, B, K, stream=side)
        junk = torch.empty(need, dtype=torch.uint8, device=DEV)
        junk.fill_(0xA5)                     # on the current stream, racing the side stream
        del junk
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("o", "lse", "idx", "k")):
            assert torch.equal(a, b), f"rep {rep}: {name} differs with stream="
