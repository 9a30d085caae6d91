"""Non-finite inputs (GPU).  The pages define the method on real-valued
inputs ("Optimizing Mixture of Block Attention", summary page, "Definizione
del Compito"); the C ABI promises, beyond that, that a NaN or infinity in a
query row leaves every other row exactly as without it, and that no call
writes outside the buffers it is given whatever the values.

Rows of q are set to NaN, +inf, -inf, a single NaN element and a huge
finite value whose scores overflow; the forward's idx, O and LSE of every
other row must equal a clean run's bitwise (each row's selection, scores,
softmax and merge depend only on that row).  Keys with a NaN block and the
backward on the dirty forward must stay inside their guarded buffers."""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import test_canary_gpu as tc  # noqa: E402

import block_sparse_long_key_amd as moba  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # (dtype, d, B, K, heads, sequence lengths)
    ("bf16", 64, 128, 8, 2, [2048, 1500]),
    ("bf16", 128, 128, 8, 2, [1300, 700]),
    ("bf16", 64, 64, 16, 2, [2100]),
    ("bf16", 64, 256, 4, 2, [1800, 300]),
    ("f32", 64, 64, 6, 2, [900, 333]),
]


def _forward(q, k, v, B, K, cu, dt):
    """The staged forward into guarded outputs; returns (bufs, idx, o, lse)."""
    T, H, d = q.shape
    nb = moba.moba_total_blocks(q, B, cu)
    b = {"cent": tc.Guarded((nb, H, d), torch.float32),
         "idx": tc.Guarded((T, H, K), torch.int32),
         "rws": tc._ws(moba.moba_route_topk_workspace_bytes(q, B, K, cu)),
         "ws": tc._ws(moba.moba_attn_fwd_workspace_bytes(q, B, K, cu)),
         "o": tc.Guarded((T, H, d), dt), "lse": tc.Guarded((T, H), torch.float32)}
    moba.moba_centroids(k, B, cu, out=b["cent"].t)
    moba.moba_route_topk(q, b["cent"].t, B, K, cu, out=b["idx"].t, workspace=b["rws"].t)
    moba.moba_attn_index(b["idx"].t, q, B, K, b["ws"].t, cu)
    moba.moba_attn_routed(q, k, v, B, K, b["ws"].t, None, cu)
    moba.moba_attn_combine(q, k, v, b["idx"].t, B, K, b["ws"].t, b["o"].t, b["lse"].t, None, cu)
    tc._check(b)
    return b, b["idx"].t, b["o"].t, b["lse"].t


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-B{c[2]}-k{c[3]}" for c in CASES])
def test_nonfinite_query_rows_leave_other_rows_unchanged(case):
    dtype, d, B, K, H, lens = case
    print(f"[nonfinite] {case}", flush=True)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    T = sum(lens)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    g = torch.Generator().manual_seed(2468 + d + B + K)
    q, k, v, dout = (torch.randn((T, H, d), generator=g).to(dt).to(DEV) for _ in range(4))
    _, idx0, o0, lse0 = _forward(q, k, v, B, K, cu, dt)

    # dirty query rows: whole-row NaN / +inf / -inf, one NaN element, and a
    # huge finite row whose scores overflow to infinity
    q1 = q.clone()
    rows = torch.randperm(T * H, generator=g)[:40].tolist()
    dirty = torch.zeros((T, H), dtype=torch.bool)
    big = 3.0e38                        # scores overflow to +-inf
    for n, rh in enumerate(rows):
        t, h = divmod(rh, H)
        kind = n % 5
        if kind == 0:
            q1[t, h] = float("nan")
        elif kind == 1:
            q1[t, h] = float("inf")
        elif kind == 2:
            q1[t, h] = float("-inf")
        elif kind == 3:
            q1[t, h, n % d] = float("nan")
        else:
            q1[t, h] = big
        dirty[t, h] = True
    b1, idx1, o1, lse1 = _forward(q1, k, v, B, K, cu, dt)
    clean = (~dirty).to(DEV)
    assert torch.equal(idx1[clean], idx0[clean]), "a clean row's selection changed"
    assert torch.equal(o1[clean].view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                       o0[clean].view(torch.int16 if dt == torch.bfloat16 else torch.int32)), \
        "a clean row's output changed"
    assert torch.equal(lse1[clean].view(torch.int32), lse0[clean].view(torch.int32)), \
        "a clean row's LSE changed"

    # backward on the dirty forward: inside its buffers
    bw = {"ws": tc._ws(moba.moba_attn_bwd_workspace_bytes(q1, B, K, cu)),
          "dq": tc.Guarded((T, H, d), dt), "dk": tc.Guarded((T, H, d), dt),
          "dv": tc.Guarded((T, H, d), dt)}
    moba.moba_attn_bwd(q1, k, v, idx1, o1, lse1, dout, B, K, cu_seqlens=cu, workspace=bw["ws"].t,
                       out=(bw["dq"].t, bw["dk"].t, bw["dv"].t))
    tc._check(bw)

    # a NaN key block (its centroid is NaN for every later query)
    k1 = k.clone()
    k1[B:B + 3, 0] = float("nan")
    _forward(q, k1, v, B, K, cu, dt)
    torch.cuda.synchronize()
