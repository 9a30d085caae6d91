"""Canary-guarded buffers around every entry point of the C ABI (GPU).

Each output and each workspace is a view into a larger device buffer whose
4 KiB on either side hold a guard byte pattern; outputs are pre-filled with
a canary value the kernels never produce (a NaN bit pattern for floating
point, 0x5A5A5A5A for block ids).  After every call the guards must be
intact (no write outside the buffer the caller passed or past the workspace
size the library asked for), every output element the header promises to
write must have been overwritten, and the inputs must be unchanged.  Shapes
are ragged varlen batches (block-partial sequences, an empty one), top-k not
a multiple of 4, 64- to 256-key blocks, both head dims and both dtypes."""
import math

import pytest
import torch

import block_sparse_long_key_amd as moba

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
G = 4096                                  # guard bytes on each side
GUARD = 0xA5
CANARY = {torch.float32: (torch.int32, 0x7FC0DEAD), torch.bfloat16: (torch.int16, 0x7FDE),
          torch.int32: (torch.int32, 0x5A5A5A5A)}


class Guarded:
    """A device buffer of `shape` / `dtype` with guard regions around it."""

    def __init__(self, shape, dtype, canary=True):
        self.n = math.prod(shape) * torch.tensor([], dtype=dtype).element_size()
        self.big = torch.full((G + self.n + G,), GUARD, dtype=torch.uint8, device=DEV)
        self.t = self.big[G:G + self.n].view(dtype).view(shape)
        self.dtype = dtype
        if canary:
            it, bits = CANARY[dtype]
            self.t.view(it).fill_(bits)

    def guards_intact(self):
        g = torch.cat([self.big[:G], self.big[G + self.n:]])
        return bool((g == GUARD).all())

    def canaries_left(self):
        it, bits = CANARY[self.dtype]
        return int((self.t.view(it) == bits).sum())


def _ws(nbytes):
    return Guarded((max(int(nbytes), 256),), torch.uint8, canary=False)


def _check(bufs, full=()):
    torch.cuda.synchronize()
    for name, b in bufs.items():
        assert b.guards_intact(), f"{name}: a guard byte changed (write outside the buffer)"
    for name in full:
        left = bufs[name].canaries_left()
        assert left == 0, f"{name}: {left} elements were not written"


CASES = [
    # (dtype, d, B, K, heads, sequence lengths, conv width)
    ("bf16", 64, 128, 5, 3, [700, 0, 129, 1], 3),
    ("bf16", 128, 128, 8, 2, [513, 384], 4),
    ("bf16", 64, 64, 16, 2, [1500, 65], 0),
    ("bf16", 64, 256, 4, 2, [1100, 300], 0),
    ("f32", 64, 64, 6, 2, [450, 77], 2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-B{c[2]}-k{c[3]}" for c in CASES])
def test_entry_points_write_inside_their_buffers(case):
    dtype, d, B, K, H, lens, W = case
    print(f"[canary] {case}", flush=True)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    T = sum(lens)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    g = torch.Generator().manual_seed(4321 + d + B + K)
    q, k, v, dout = (torch.randn((T, H, d), generator=g).to(dt).to(DEV) for _ in range(4))
    inputs = {"q": q, "k": k, "v": v, "dout": dout}
    saved = {n: t.clone() for n, t in inputs.items()}
    nb = moba.moba_total_blocks(q, B, cu)

    # key conv (+ centroids), or centroids alone
    bufs = {"cent": Guarded((nb, H, d), torch.float32)}
    if W:
        w = (torch.randn((H, d, W), generator=g) / W).to(DEV)
        bufs["kc"] = Guarded((T, H, d), dt)
        moba.moba_key_conv(k, w, B, "silu_residual" if W == 3 else "plain", cu,
                           with_centroids=True, out=bufs["kc"].t, cent=bufs["cent"].t)
        _check(bufs, full=("kc", "cent"))
        kk = bufs["kc"].t
    else:
        moba.moba_centroids(k, B, cu, out=bufs["cent"].t)
        _check(bufs, full=("cent",))
        kk = k
    cent = bufs["cent"].t

    # router (caller's workspace), and the no-allocation router
    b = {"idx": Guarded((T, H, K), torch.int32),
         "ws": _ws(moba.moba_route_topk_workspace_bytes(q, B, K, cu))}
    moba.moba_route_topk(q, cent, B, K, cu, out=b["idx"].t, workspace=b["ws"].t)
    _check(b, full=("idx",))
    idx = b["idx"].t
    if dtype == "bf16":
        b2 = {"idx2": Guarded((T, H, K), torch.int32)}
        moba.moba_route_topk_noalloc(q, cent, B, K, cu, out=b2["idx2"].t)
        _check(b2, full=("idx2",))
        assert torch.equal(b2["idx2"].t, idx)

    # attention in stages: index, routed, combine (o and lse given)
    nws = moba.moba_attn_fwd_workspace_bytes(q, B, K, cu)
    a = {"ws": _ws(nws), "o": Guarded((T, H, d), dt), "lse": Guarded((T, H), torch.float32)}
    idx_saved = idx.clone()
    moba.moba_attn_index(idx, q, B, K, a["ws"].t, cu)
    moba.moba_attn_routed(q, kk, v, B, K, a["ws"].t, None, cu)
    moba.moba_attn_combine(q, kk, v, idx, B, K, a["ws"].t, a["o"].t, a["lse"].t, None, cu)
    _check(a, full=("o", "lse"))
    o, lse = a["o"].t, a["lse"].t

    # one-call forward and the BLASST forward (with its kept selection) into
    # guarded outputs
    blasst = None
    for lam in ((None, 0.5) if B <= 128 else (None,)):   # BLASST takes whole blocks only
        f = {"ws": _ws(nws), "o": Guarded((T, H, d), dt)}
        if lam is None:
            o2, _ = moba.moba_attn_fwd(q, kk, v, idx, B, K, cu_seqlens=cu, workspace=f["ws"].t,
                                       return_lse=False, out=f["o"].t)
            _check(f, full=("o",))
            assert torch.equal(o2, o)
        else:
            f["kept"] = Guarded((T, H, K), torch.int32)
            o3, lse3, kept3 = moba.moba_attn_fwd(q, kk, v, idx, B, K, cu_seqlens=cu,
                                                 workspace=f["ws"].t, out=f["o"].t,
                                                 blasst_lambda=lam, return_kept=True,
                                                 kept_out=f["kept"].t)
            _check(f, full=("o", "kept"))
            blasst = (o3, lse3, kept3)

    # attention backward into guarded dq, dk, dv
    bw = {"ws": _ws(moba.moba_attn_bwd_workspace_bytes(q, B, K, cu)),
          "dq": Guarded((T, H, d), dt), "dk": Guarded((T, H, d), dt), "dv": Guarded((T, H, d), dt)}
    moba.moba_attn_bwd(q, kk, v, idx, o, lse, dout, B, K, cu_seqlens=cu, workspace=bw["ws"].t,
                       out=(bw["dq"].t, bw["dk"].t, bw["dv"].t))
    _check(bw, full=("dq", "dk", "dv"))
    if blasst is not None:
        kept = blasst[2]
        kept_saved = kept.clone()
        bb = {"ws": _ws(moba.moba_attn_bwd_workspace_bytes(q, B, K, cu)),
              "dq": Guarded((T, H, d), dt), "dk": Guarded((T, H, d), dt),
              "dv": Guarded((T, H, d), dt)}
        moba.moba_attn_bwd_blasst(q, kk, v, kept, blasst[0], blasst[1], dout, B, K, cu_seqlens=cu,
                                  workspace=bb["ws"].t, out=(bb["dq"].t, bb["dk"].t, bb["dv"].t))
        _check(bb, full=("dq", "dk", "dv"))
        assert torch.equal(kept, kept_saved), "kept_idx was modified by the backward"

    # key conv backward: its workspace stays inside the asked size
    if W:
        cw = {"ws": _ws(moba.moba_key_conv_bwd_workspace_bytes(k, B, W, cu))}
        moba.moba_key_conv_bwd(k, w, bw["dk"].t, B, "silu_residual" if W == 3 else "plain", cu,
                               workspace=cw["ws"].t)
        _check(cw)

    torch.cuda.synchronize()
    for n, t in inputs.items():
        assert torch.equal(t, saved[n]), f"input {n} was modified"
    assert torch.equal(idx, idx_saved), "idx was modified by the attention calls"
