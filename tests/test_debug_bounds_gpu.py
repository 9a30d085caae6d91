"""The bounds-checking build of the library (libmoba_amd_debug.so, compiled
with MOBA_DEBUG_BOUNDS): every index the kernels take from data -- list
entries, list positions, work items -- is checked against the region it
addresses.  On each shape below the whole path (conv or pooling, routing,
index pass, routed attention, merge, the BLASST forward and both backwards,
the conv backward) runs through the debug build; no check may fail
(moba_debug_violations reports 0) and every output must equal the release
build's bitwise (the checks change nothing on valid input).  Shapes: ragged
varlen with empty and one-token sequences, 150 sequences (groups of 64),
64- to 256-key blocks, both head dims and both dtypes, top-k up to 16."""
import contextlib
import ctypes
import dataclasses

import pytest
import torch

import block_sparse_long_key_amd as m
import workloads
from block_sparse_long_key_amd import build as mbuild

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _spec(base, seq=None, heads=None, seqlens=None, **kw):
    s = workloads.spec(base)
    if seqlens is not None:
        s = dataclasses.replace(s, batch=1, seq=sum(seqlens), seqlens=tuple(seqlens))
    elif seq is not None:
        s = s.scaled(seq)
    if heads is not None:
        s = dataclasses.replace(s, heads=heads)
    return dataclasses.replace(s, plant=False, name=s.name + "-dbg", **kw)


CASES = {
    "H-8k": (_spec("H", seq=8192, heads=2), 0.5),
    "ragged-conv-d128-B64": (_spec("C5", seqlens=(1000, 0, 1, 777, 129), heads=2, block_size=64,
                                   top_k=6), 0.6),
    "B64-k16": (_spec("C4", seq=8192, heads=2), 0.7),
    "B256-k4": (_spec("M256", seq=4096, heads=2), None),
    "many-seqs": (_spec("H", seqlens=tuple((53 * i) % 400 for i in range(150)), heads=2,
                        block_size=64, top_k=4), 0.5),
    "f32-d64-B64": (_spec("C1", seq=3000, heads=2), 0.8),
}


@contextlib.contextmanager
def _library(path):
    saved = (m._lib, m._LIB_PATH)
    m._lib, m._LIB_PATH = None, path
    try:
        lib = m._load()
        lib.moba_debug_violations.argtypes = [ctypes.c_void_p]
        lib.moba_debug_violations.restype = ctypes.c_int32
        yield lib
    finally:
        m._lib, m._LIB_PATH = saved


def _violations(lib):
    torch.cuda.synchronize()
    f = ctypes.c_uint32(0xDEAD)
    assert lib.moba_debug_violations(ctypes.byref(f)) == 0
    return f.value


def _run(s, lam):
    """The whole path on workload s; returns every output."""
    x = workloads.make(s)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(DEV)
    do = workloads.grad_output(s).to(DEV)
    cu = x["cu_seqlens"]
    B, K = s.block_size, s.top_k
    o, lse, idx, kk = m.moba_fwd(q, k, v, B, K, conv_w=w, conv_mode=s.conv_mode, cu_seqlens=cu)
    g = m.moba_attn_bwd(q, kk, v, idx, o, lse, do, B, K, cu_seqlens=cu)
    out = [o, lse, idx, kk, *g]
    if w is not None:
        out += list(m.moba_key_conv_bwd(k, w, g[1], B, s.conv_mode, cu_seqlens=cu))
    if lam is not None:
        ob, lb, kept = m.moba_attn_fwd(q, kk, v, idx, B, K, cu_seqlens=cu, blasst_lambda=lam,
                                       return_kept=True)
        out += [ob, lb, kept, *m.moba_attn_bwd_blasst(q, kk, v, kept, ob, lb, do, B, K, cu_seqlens=cu)]
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_debug_build_finds_no_violation_and_changes_nothing(name):
    s, lam = CASES[name]
    print(f"[debug-bounds {name}] {s} lambda={lam}", flush=True)
    ref = _run(s, lam)
    with _library(mbuild.DEBUG_LIB) as lib:
        assert _violations(lib) == 0            # nothing recorded before the run
        got = _run(s, lam)
        v = _violations(lib)
    assert v == 0, f"{name}: bounds checks failed, flags {v:#x}"
    assert len(got) == len(ref)
    for n, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), f"{name}: output {n} differs between the debug and release builds"

