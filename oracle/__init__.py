"""CPU oracle of the MoBA forward pass and of its attention backward
(test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never does: it shares no code with this oracle.

The arithmetic lives in ``moba_oracle.c`` (plain C, fp64 accumulation, see
its header for the citation of each step).  This file only marshals numpy
arrays through ctypes.

Arrays are numpy float32 ``[tokens, heads, d]`` holding the exact values of
the I/O dtype; ``cu`` is the list of sequence starts over the token axis
(``[0, L0, L0+L1, ...]``); a uniform batch is ``[0, N, 2N, ...]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moba_oracle.c")
_LIB = os.path.join(_HERE, "libmoba_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
            "-fno-fast-math", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp,
            "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.moba_oracle_key_conv.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _I]
        lib.moba_oracle_centroids.argtypes = [_P, _I, _I, _I, _P, _I, _P, _I]
        lib.moba_oracle_route.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _I]
        lib.moba_oracle_attend.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _D, _P, _P, _I]
        lib.moba_oracle_total_blocks.argtypes = [_P, _I, _I]
        lib.moba_oracle_route_rows.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P, _P, _P]
        lib.moba_oracle_attend_rows.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _D, _P, _I, _P, _P]
        lib.moba_oracle_route_scores.argtypes = [_P, _P, _I, _I, _I, _P, _I, _P, _I, _I, _P]
        lib.moba_oracle_attend_blasst.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _D, _D,
                                                  _P, _P, _D, _P, _P, _P, _P, _I]
        lib.moba_oracle_attend_blasst.restype = _I
        lib.moba_oracle_route_scores.restype = _I
        lib.moba_oracle_attend_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _D,
                                               _P, _P, _P, _P, _P, _I]
        lib.moba_oracle_attend_bwd.restype = _I
        lib.moba_oracle_key_conv_bwd.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _I]
        lib.moba_oracle_key_conv_bwd.restype = _I
        lib.moba_oracle_route_rows.restype = _I
        lib.moba_oracle_attend_rows.restype = _I
        for f in (lib.moba_oracle_key_conv, lib.moba_oracle_centroids,
                  lib.moba_oracle_route, lib.moba_oracle_attend,
                  lib.moba_oracle_total_blocks):
            f.restype = _I
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").float().numpy()
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim == 4:  # [batch, seq, H, d] -> [tokens, H, d]
        a = a.reshape(-1, a.shape[2], a.shape[3])
    return a


def _cu(cu: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def total_blocks(cu: Sequence[int], B: int) -> int:
    c = _cu(cu)
    return int(_load().moba_oracle_total_blocks(_ptr(c), len(c) - 1, B))


def key_conv(k, w, cu, mode: int = 0, round_bf16: bool = True,
             nthreads: Optional[int] = None) -> np.ndarray:
    """k' = depthwise causal conv of k (mode 0 plain, 1 = k + SiLU(conv))."""
    k = _f32(k)
    w = _f32(w) if not isinstance(w, np.ndarray) or w.dtype != np.float32 else np.ascontiguousarray(w)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, H, d = k.shape
    W = w.shape[-1]
    assert w.shape == (H, d, W)
    c = _cu(cu)
    out = np.empty_like(k)
    rc = _load().moba_oracle_key_conv(_ptr(k), _ptr(w), H, d, W, mode,
                                      1 if round_bf16 else 0, _ptr(c),
                                      len(c) - 1, _ptr(out),
                                      nthreads or default_threads())
    assert rc == 0
    return out


def centroids(k, B: int, cu, nthreads: Optional[int] = None) -> np.ndarray:
    """Block means (fp64 sums, rounded once to fp32): [total_blocks, H, d]."""
    k = _f32(k)
    T, H, d = k.shape
    c = _cu(cu)
    nb = total_blocks(cu, B)
    cent = np.empty((nb, H, d), dtype=np.float32)
    rc = _load().moba_oracle_centroids(_ptr(k), H, d, B, _ptr(c), len(c) - 1,
                                       _ptr(cent), nthreads or default_threads())
    assert rc == 0
    return cent


def route(q, cent, B: int, K: int, cu, nthreads: Optional[int] = None):
    """Causal top-k block selection.

    Returns (idx int32 [T,H,K], gap_a f64 [T,H], gap_b f64 [T,H],
    exempt bool [T,H]).
    """
    q = _f32(q)
    cent = np.ascontiguousarray(cent, dtype=np.float32)
    T, H, d = q.shape
    c = _cu(cu)
    idx = np.empty((T, H, K), dtype=np.int32)
    ga = np.empty((T, H), dtype=np.float64)
    gb = np.empty((T, H), dtype=np.float64)
    ex = np.empty((T, H), dtype=np.uint8)
    rc = _load().moba_oracle_route(_ptr(q), _ptr(cent), H, d, B, K, _ptr(c),
                                   len(c) - 1, _ptr(idx), _ptr(ga), _ptr(gb),
                                   _ptr(ex), nthreads or default_threads())
    assert rc == 0
    return idx, ga, gb, ex.astype(bool)


def attend(q, k, v, idx, B: int, K: int, cu, scale: float = 0.0,
           nthreads: Optional[int] = None):
    """Attention over the blocks listed in idx (+ the causal own block).

    Returns (o f64 [T,H,d], lse f64 [T,H]).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(q.shape[0], q.shape[1], K)
    T, H, d = q.shape
    c = _cu(cu)
    o = np.empty((T, H, d), dtype=np.float64)
    lse = np.empty((T, H), dtype=np.float64)
    rc = _load().moba_oracle_attend(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), H, d,
                                    B, K, _ptr(c), len(c) - 1, float(scale),
                                    _ptr(o), _ptr(lse),
                                    nthreads or default_threads())
    assert rc == 0
    return o, lse


def forward(q, k, v, B: int, K: int, cu, conv_w=None, conv_mode: int = 0,
            round_bf16: bool = True, scale: float = 0.0,
            nthreads: Optional[int] = None) -> dict:
    """The whole pass: [key conv] -> centroids -> route -> attend."""
    kk = _f32(k)
    if conv_w is not None:
        kk = key_conv(kk, conv_w, cu, conv_mode, round_bf16, nthreads)
    cent = centroids(kk, B, cu, nthreads)
    idx, ga, gb, ex = route(q, cent, B, K, cu, nthreads)
    o, lse = attend(q, kk, v, idx, B, K, cu, scale, nthreads)
    return {"k_conv": kk, "cent": cent, "idx": idx, "gap_a": ga, "gap_b": gb,
            "exempt": ex, "o": o, "lse": lse}


def attend_blasst(q, k, v, idx, B: int, K: int, cu, lam: float, scale: float = 0.0,
                  keep=None, flip=None, tau: float = 1e-4, nthreads: Optional[int] = None,
                  return_keep: bool = False):
    """Step 5 with the BLASST block skip (blocks visited in ascending order,
    own block last; a block whose maximum score is below the running maximum
    of the attended scores + ln(lam) is skipped).  lam = 0 keeps every block.

    keep (bool [T, H, K], optional) replaces the rule by an explicit choice
    per idx slot.  flip (uint64 [T, H], optional) takes the near decisions
    whose bit is set the other way.  Returns (o f64 [T,H,d], lse f64 [T,H],
    near uint64 [T,H]): bit b of near marks a decision on the b-th visited
    block within tau * max(1, |M|) of the threshold.  With return_keep, a
    fourth result holds the decisions taken (bool [T, H, K]: True where the
    slot's block was attended, own block included).
    """
    import math
    q, k, v = _f32(q), _f32(k), _f32(v)
    T, H, d = q.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(T, H, K)
    c = _cu(cu)
    o = np.empty((T, H, d), dtype=np.float64)
    lse = np.empty((T, H), dtype=np.float64)
    near = np.zeros((T, H), dtype=np.uint64)
    kp = None
    if keep is not None:
        kp = np.ascontiguousarray(np.asarray(keep, dtype=np.uint8).reshape(T, H, K))
    fl = None
    if flip is not None:
        fl = np.ascontiguousarray(np.asarray(flip, dtype=np.uint64).reshape(T, H))
    ll = math.log(lam) if lam > 0 else -math.inf
    ko = np.zeros((T, H, K), dtype=np.uint8) if return_keep else None
    rc = _load().moba_oracle_attend_blasst(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), H, d, B, K,
                                           _ptr(c), len(c) - 1, float(scale), float(ll),
                                           None if kp is None else _ptr(kp),
                                           None if fl is None else _ptr(fl), float(tau),
                                           _ptr(o), _ptr(lse), _ptr(near),
                                           None if ko is None else _ptr(ko),
                                           nthreads or default_threads())
    assert rc == 0
    if return_keep:
        return o, lse, near, ko.astype(bool)
    return o, lse, near


def route_rows(q, cent, B: int, K: int, cu, rows):
    """Routing for the listed rows only (row = token * H + head).

    Returns (idx [nrows, K], gap_a, gap_b, exempt) for those rows.
    """
    q = _f32(q)
    cent = np.ascontiguousarray(cent, dtype=np.float32)
    T, H, d = q.shape
    c = _cu(cu)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    idx = np.full((T * H, K), -7, dtype=np.int32)
    ga = np.zeros(T * H)
    gb = np.zeros(T * H)
    ex = np.zeros(T * H, dtype=np.uint8)
    rc = _load().moba_oracle_route_rows(_ptr(q), _ptr(cent), H, d, B, K, _ptr(c),
                                        len(c) - 1, _ptr(rows), len(rows), _ptr(idx),
                                        _ptr(ga), _ptr(gb), _ptr(ex))
    assert rc == 0
    return idx[rows], ga[rows], gb[rows], ex[rows].astype(bool)


def route_scores(q, cent, B: int, cu, rows) -> np.ndarray:
    """fp64 router scores of the listed rows against every past block.

    Returns f64 [nrows, nmax] (nmax = the longest sequence's block count);
    entry j of a row is NaN for j >= its own block.
    """
    q = _f32(q)
    cent = np.ascontiguousarray(cent, dtype=np.float32)
    T, H, d = q.shape
    c = _cu(cu)
    nmax = max(1, max((int(c[s + 1] - c[s]) + B - 1) // B for s in range(len(c) - 1)))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((len(rows), nmax), dtype=np.float64)
    rc = _load().moba_oracle_route_scores(_ptr(q), _ptr(cent), H, d, B, _ptr(c), len(c) - 1,
                                          _ptr(rows), len(rows), nmax, _ptr(out))
    assert rc == 0
    return out


def attend_rows(q, k, v, idx, B: int, K: int, cu, rows, scale: float = 0.0):
    """Attention for the listed rows only; idx is the full [T, H, K] array.

    Returns (o [nrows, d], lse [nrows]).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    T, H, d = q.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(T, H, K)
    c = _cu(cu)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    o = np.zeros((T * H, d), dtype=np.float64)
    lse = np.zeros(T * H, dtype=np.float64)
    rc = _load().moba_oracle_attend_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), H, d, B, K,
                                         _ptr(c), len(c) - 1, float(scale), _ptr(rows),
                                         len(rows), _ptr(o), _ptr(lse))
    assert rc == 0
    return o[rows], lse[rows]


def attend_bwd(q, k, v, idx, dout, B: int, K: int, cu, scale: float = 0.0,
               qsel=None, kbsel=None, nthreads: Optional[int] = None, keep=None):
    """Gradients of the attention output for the fixed selection idx.

    dout is dL/dO ([T, H, d]).  Returns (dq, dk, dv), f64 [T, H, d].
    qsel (bool [T, H]) limits the rows whose dq is computed, kbsel (bool
    [total_blocks, H]) the key blocks whose dk / dv are computed; entries
    outside them are NaN.  keep (bool [T, H, K], optional): the BLASST
    decisions per idx slot (as attend_blasst's keep); only the kept blocks'
    keys, the own block's included, are in a row's key set.
    """
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    T, H, d = q.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(T, H, K)
    kp = None
    if keep is not None:
        kp = np.ascontiguousarray(np.asarray(keep, dtype=np.uint8).reshape(T, H, K))
    c = _cu(cu)
    dq = np.full((T, H, d), np.nan)
    dk = np.full((T, H, d), np.nan)
    dv = np.full((T, H, d), np.nan)
    qs = None if qsel is None else np.ascontiguousarray(np.asarray(qsel, dtype=np.uint8).reshape(T, H))
    ks = None if kbsel is None else np.ascontiguousarray(np.asarray(kbsel, dtype=np.uint8))
    if ks is not None:
        assert ks.shape == (total_blocks(cu, B), H)
    rc = _load().moba_oracle_attend_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                        None if kp is None else _ptr(kp), _ptr(dout),
                                        H, d, B, K, _ptr(c), len(c) - 1, float(scale),
                                        None if qs is None else _ptr(qs),
                                        None if ks is None else _ptr(ks),
                                        _ptr(dq), _ptr(dk), _ptr(dv),
                                        nthreads or default_threads())
    assert rc == 0
    return dq, dk, dv


def key_conv_bwd(k, w, g, cu, mode: int = 0, nthreads: Optional[int] = None):
    """Gradients of the key convolution given g = dL/dk'.

    Returns (dk f64 [T, H, d], dw f64 [H, d, W]).
    """
    k, g = _f32(k), _f32(g)
    w = np.ascontiguousarray(_f32(w) if not isinstance(w, np.ndarray) else w, dtype=np.float32)
    T, H, d = k.shape
    W = w.shape[-1]
    assert w.shape == (H, d, W) and g.shape == k.shape
    c = _cu(cu)
    dk = np.empty((T, H, d), dtype=np.float64)
    dw = np.empty((H, d, W), dtype=np.float64)
    rc = _load().moba_oracle_key_conv_bwd(_ptr(k), _ptr(w), _ptr(g), H, d, W, mode, _ptr(c),
                                          len(c) - 1, _ptr(dk), _ptr(dw),
                                          nthreads or default_threads())
    assert rc == 0
    return dk, dw
