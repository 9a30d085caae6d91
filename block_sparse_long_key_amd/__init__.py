"""MI355X (gfx950) Mixture of Block Attention forward and attention
backward -- Python binding.

A thin ctypes layer over ``libmoba_amd.so`` (C ABI in ``include/moba.h``).
It only marshals arguments: it checks tensor devices, dtypes and layouts,
allocates outputs and workspaces with torch (device memory only) and passes
``data_ptr()`` values and torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels.  If the library is missing
the calls raise -- there is no CPU fallback.

Names follow the C ABI: ``moba_key_conv``, ``moba_centroids``,
``moba_route_topk``, ``moba_attn_fwd`` (plus its three stages
``moba_attn_index``, ``moba_attn_routed``, ``moba_attn_combine``), the
convenience ``moba_fwd`` that chains them (``fwd``: the same, returning
(o, lse, idx)), ``moba_attn_bwd`` and
``moba_key_conv_bwd``, and ``moba_attention``: the whole layer as a
differentiable op (torch autograd glue around the same calls).

Tensors are ``[batch, seq, heads, head_dim]`` (uniform batch) or
``[total_tokens, heads, head_dim]`` with ``cu_seqlens`` (a python list or CPU
int tensor of num_seqs + 1 offsets).
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "moba_key_conv", "moba_centroids", "moba_route_topk", "moba_route_topk_noalloc",
    "moba_attn_fwd", "moba_attn_fwd_blasst",
    "moba_attn_index", "moba_attn_routed", "moba_attn_combine", "moba_fwd", "fwd",
    "moba_attn_fwd_workspace_bytes", "moba_route_topk_workspace_bytes", "moba_total_blocks",
    "library_path",
    "moba_attn_bwd", "moba_attn_bwd_blasst", "moba_attn_bwd_workspace_bytes", "moba_key_conv_bwd",
    "moba_key_conv_bwd_workspace_bytes", "moba_attention",
    "MobaError",
]

_ABI_VERSION = 3                 # MOBA_ABI_VERSION of include/moba.h
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoba_amd.so")
_lib = None

MOBA_F32, MOBA_BF16 = 0, 1
_CONV_MODES = {"plain": 0, "silu_residual": 1}


class MobaError(RuntimeError):
    pass


class _Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seq", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("num_seqs", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
    ]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MobaError(
            f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
            "python block_sparse_long_key_amd/build.py")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    SH = ctypes.POINTER(_Shape)
    sig = {
        "moba_key_conv": [SH, P, P, I32, I32, P, P, P],
        "moba_centroids": [SH, P, P, P],
        "moba_route_topk": [SH, P, P, P, P, SZ, P],
        "moba_route_topk_noalloc": [SH, P, P, P, P],
        "moba_attn_fwd": [SH, P, P, P, P, F32, P, P, P, SZ, P],
        "moba_attn_fwd_blasst": [SH, P, P, P, P, F32, F32, P, P, P, P, SZ, P],
        "moba_attn_index": [SH, P, P, SZ, P],
        "moba_attn_routed": [SH, P, P, P, F32, P, SZ, P],
        "moba_attn_combine": [SH, P, P, P, P, F32, P, P, P, SZ, P],
        "moba_attn_bwd": [SH, P, P, P, P, F32, P, P, P, P, P, P, P, SZ, P],
        "moba_attn_bwd_blasst": [SH, P, P, P, P, F32, P, P, P, P, P, P, P, SZ, P],
        "moba_key_conv_bwd": [SH, P, P, I32, I32, P, P, P, P, SZ, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.moba_attn_fwd_workspace_bytes.argtypes = [SH]
    lib.moba_attn_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.moba_route_topk_workspace_bytes.argtypes = [SH]
    lib.moba_route_topk_workspace_bytes.restype = ctypes.c_size_t
    lib.moba_key_conv_bwd_workspace_bytes.argtypes = [SH, I32]
    lib.moba_key_conv_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.moba_attn_bwd_workspace_bytes.argtypes = [SH]
    lib.moba_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.moba_total_blocks.argtypes = [SH]
    lib.moba_total_blocks.restype = ctypes.c_int64
    lib.moba_status_string.argtypes = [ctypes.c_int]
    lib.moba_status_string.restype = ctypes.c_char_p
    lib.moba_abi_version.restype = ctypes.c_int32
    if lib.moba_abi_version() != _ABI_VERSION:
        raise MobaError(f"{_LIB_PATH} has C ABI version {lib.moba_abi_version()}, this binding "
                        f"expects {_ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = _load().moba_status_string(rc).decode()
        raise MobaError(f"{what} failed: {msg} (status {rc})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOBA_BF16
    if t.dtype == torch.float32:
        return MOBA_F32
    raise MobaError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _make_shape(x: torch.Tensor, block_size: int, top_k: int,
                cu_seqlens: Optional[Sequence[int]]):
    if x.dim() == 4:
        if cu_seqlens is not None:
            raise MobaError("cu_seqlens needs [total_tokens, heads, head_dim] tensors")
        b, n, h, d = x.shape
        sh = _Shape(b, n, h, d, None, 0, block_size, top_k, _dtype_code(x))
        return sh, None
    if x.dim() == 3:
        t, h, d = x.shape
        if cu_seqlens is None:
            cu = [0, t]
        else:
            cu = [int(c) for c in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        arr = (ctypes.c_int32 * len(cu))(*cu)
        sh = _Shape(1, t, h, d, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)),
                    len(cu) - 1, block_size, top_k, _dtype_code(x))
        return sh, arr
    raise MobaError("expected [batch, seq, heads, head_dim] or [tokens, heads, head_dim]")


def _dev(*ts: torch.Tensor):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise MobaError("tensors must be on the GPU")
        # the kernels run on the current device: a tensor elsewhere would be
        # read through a foreign pointer
        if t.device.index != torch.cuda.current_device():
            raise MobaError(f"tensors must be on the current device (cuda:{torch.cuda.current_device()}), "
                            f"got {t.device}")
        if not t.is_contiguous():
            raise MobaError("tensors must be contiguous")


def _stream(stream=None) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Runs a call whose ``stream`` (keyword) is given with that stream as
    torch's current one, so the outputs and workspaces the call allocates
    belong to the stream its kernels run on: torch's caching allocator then
    hands a dropped workspace only to later work on that same stream, never
    to another stream while the kernels may still read it.  Outputs are
    ready on ``stream``; another stream must wait for it before using them."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return call


def _p(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _rows(x: torch.Tensor) -> Tuple[int, ...]:
    return tuple(x.shape[:-1])


# The C ABI takes plain pointers, so every buffer size is checked here: a
# wrong-sized tensor raises instead of reaching a kernel.
def _expect(t: Optional[torch.Tensor], shape, dtype, name: str):
    if t is None:
        return
    _dev(t)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise MobaError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _like(t: Optional[torch.Tensor], ref: torch.Tensor, name: str):
    _expect(t, ref.shape, ref.dtype, name)


def _ws(t: torch.Tensor, need: int):
    _dev(t)
    if t.dtype != torch.uint8 or t.dim() != 1:
        raise MobaError("workspace must be a 1-D uint8 tensor")
    if t.numel() < need:
        raise MobaError(f"workspace has {t.numel()} bytes, {need} needed")


def _qkv(q, k, v):
    _dev(q, k, v)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise MobaError("q, k, v must share shape and dtype")


def _idx(idx, q, top_k):
    _expect(idx, _rows(q) + (top_k,), torch.int32, "idx")


def _cent_shape(k, block_size, cu_seqlens):
    return (moba_total_blocks(k, block_size, cu_seqlens), k.shape[-2], k.shape[-1])


def moba_total_blocks(x: torch.Tensor, block_size: int, cu_seqlens=None) -> int:
    sh, keep = _make_shape(x, block_size, 1, cu_seqlens)
    n = _load().moba_total_blocks(ctypes.byref(sh))
    if n < 0:
        raise MobaError("invalid shape")
    return int(n)


def moba_attn_fwd_workspace_bytes(q: torch.Tensor, block_size: int, top_k: int,
                                  cu_seqlens=None) -> int:
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    return int(_load().moba_attn_fwd_workspace_bytes(ctypes.byref(sh)))


def moba_route_topk_workspace_bytes(q: torch.Tensor, block_size: int, top_k: int,
                                    cu_seqlens=None) -> int:
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    return int(_load().moba_route_topk_workspace_bytes(ctypes.byref(sh)))


def moba_attn_bwd_workspace_bytes(q: torch.Tensor, block_size: int, top_k: int,
                                  cu_seqlens=None) -> int:
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    return int(_load().moba_attn_bwd_workspace_bytes(ctypes.byref(sh)))


@_on_stream
def moba_key_conv(k: torch.Tensor, w: torch.Tensor, block_size: int,
                  mode: str = "plain", cu_seqlens=None, with_centroids: bool = False,
                  out: Optional[torch.Tensor] = None, cent: Optional[torch.Tensor] = None,
                  stream=None):
    """k' = causal depthwise conv of k (w: fp32 [heads, head_dim, W]).

    Returns k' (and the block centroids of k' when ``with_centroids``).
    """
    _dev(k, w)
    sh, keep = _make_shape(k, block_size, 1, cu_seqlens)
    if w.dtype != torch.float32 or w.dim() != 3 or w.shape[0] != k.shape[-2] or w.shape[1] != k.shape[-1]:
        raise MobaError("w must be fp32 [heads, head_dim, width]")
    if out is None:
        out = torch.empty_like(k)
    _like(out, k, "out")
    if out.data_ptr() == k.data_ptr():
        raise MobaError("out must not alias k")
    if with_centroids:
        if cent is None:
            cent = torch.empty(_cent_shape(k, block_size, cu_seqlens), dtype=torch.float32,
                               device=k.device)
        _expect(cent, _cent_shape(k, block_size, cu_seqlens), torch.float32, "cent")
    rc = _load().moba_key_conv(ctypes.byref(sh), _p(k), _p(w), w.shape[2],
                               _CONV_MODES[mode], _p(out),
                               _p(cent if with_centroids else None), _stream(stream))
    _check(rc, "moba_key_conv")
    return (out, cent) if with_centroids else out


def moba_key_conv_bwd_workspace_bytes(k: torch.Tensor, block_size: int, width: int,
                                      cu_seqlens=None) -> int:
    sh, keep = _make_shape(k, block_size, 1, cu_seqlens)
    return int(_load().moba_key_conv_bwd_workspace_bytes(ctypes.byref(sh), int(width)))


@_on_stream
def moba_key_conv_bwd(k: torch.Tensor, w: torch.Tensor, dk_out: torch.Tensor, block_size: int,
                      mode: str = "plain", cu_seqlens=None, workspace: Optional[torch.Tensor] = None,
                      stream=None):
    """Gradients of moba_key_conv given dk_out = dL/dk'.  Returns (dk, dw)."""
    _dev(k, w, dk_out)
    if dk_out.shape != k.shape or dk_out.dtype != k.dtype:
        raise MobaError("dk_out must match k")
    if w.dtype != torch.float32 or w.dim() != 3 or w.shape[0] != k.shape[-2] or w.shape[1] != k.shape[-1]:
        raise MobaError("w must be fp32 [heads, head_dim, width]")
    sh, keep = _make_shape(k, block_size, 1, cu_seqlens)
    W = int(w.shape[2])
    need = moba_key_conv_bwd_workspace_bytes(k, block_size, W, cu_seqlens)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k.device)
    _ws(workspace, need)
    dk = torch.empty_like(k)
    dw = torch.empty_like(w)
    rc = _load().moba_key_conv_bwd(ctypes.byref(sh), _p(k), _p(w), W, _CONV_MODES[mode],
                                   _p(dk_out), _p(dk), _p(dw), _p(workspace), workspace.numel(),
                                   _stream(stream))
    _check(rc, "moba_key_conv_bwd")
    return dk, dw


@_on_stream
def moba_centroids(k: torch.Tensor, block_size: int, cu_seqlens=None,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block means of k: fp32 [total_blocks, heads, head_dim]."""
    _dev(k)
    sh, keep = _make_shape(k, block_size, 1, cu_seqlens)
    if out is None:
        out = torch.empty(_cent_shape(k, block_size, cu_seqlens), dtype=torch.float32,
                          device=k.device)
    _expect(out, _cent_shape(k, block_size, cu_seqlens), torch.float32, "out")
    _check(_load().moba_centroids(ctypes.byref(sh), _p(k), _p(out), _stream(stream)),
           "moba_centroids")
    return out


@_on_stream
def moba_route_topk(q: torch.Tensor, cent: torch.Tensor, block_size: int, top_k: int,
                    cu_seqlens=None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal top-k block ids: int32 [..., heads, top_k], ascending, -1 padded.

    workspace: uint8 device tensor of at least moba_route_topk_workspace_bytes
    (a moba_attn_fwd workspace of that size may be shared); allocated here
    when None."""
    _dev(q, cent)
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    _expect(cent, _cent_shape(q, block_size, cu_seqlens), torch.float32, "cent")
    if out is None:
        out = torch.empty(_rows(q) + (top_k,), dtype=torch.int32, device=q.device)
    _idx(out, q, top_k)
    need = int(_load().moba_route_topk_workspace_bytes(ctypes.byref(sh)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _ws(workspace, need)
    _check(_load().moba_route_topk(ctypes.byref(sh), _p(q), _p(cent), _p(out), _p(workspace),
                                   workspace.numel(), _stream(stream)),
           "moba_route_topk")
    return out


@_on_stream
def moba_route_topk_noalloc(q: torch.Tensor, cent: torch.Tensor, block_size: int, top_k: int,
                            cu_seqlens=None, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """moba_route_topk on the library's fixed per-GPU routing scratch (the C
    call allocates nothing; pass ``out`` to allocate nothing here either).
    Calls that overlap on one GPU race on that scratch."""
    _dev(q, cent)
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    _expect(cent, _cent_shape(q, block_size, cu_seqlens), torch.float32, "cent")
    if out is None:
        out = torch.empty(_rows(q) + (top_k,), dtype=torch.int32, device=q.device)
    _idx(out, q, top_k)
    _check(_load().moba_route_topk_noalloc(ctypes.byref(sh), _p(q), _p(cent), _p(out),
                                           _stream(stream)), "moba_route_topk_noalloc")
    return out


def _workspace(q, block_size, top_k, cu_seqlens, workspace):
    need = moba_attn_fwd_workspace_bytes(q, block_size, top_k, cu_seqlens)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _ws(workspace, need)
    return workspace


@_on_stream
def moba_attn_index(idx, q, block_size, top_k, workspace, cu_seqlens=None, stream=None):
    _dev(q)
    _idx(idx, q, top_k)
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    _ws(workspace, moba_attn_fwd_workspace_bytes(q, block_size, top_k, cu_seqlens))
    _check(_load().moba_attn_index(ctypes.byref(sh), _p(idx), _p(workspace),
                                   workspace.numel(), _stream(stream)), "moba_attn_index")


@_on_stream
def moba_attn_routed(q, k, v, block_size, top_k, workspace, scale=None, cu_seqlens=None,
                     stream=None):
    _qkv(q, k, v)
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    _ws(workspace, moba_attn_fwd_workspace_bytes(q, block_size, top_k, cu_seqlens))
    _check(_load().moba_attn_routed(ctypes.byref(sh), _p(q), _p(k), _p(v),
                                    float(scale or 0.0), _p(workspace), workspace.numel(),
                                    _stream(stream)), "moba_attn_routed")


@_on_stream
def moba_attn_combine(q, k, v, idx, block_size, top_k, workspace, o, lse=None, scale=None,
                      cu_seqlens=None, stream=None):
    _qkv(q, k, v)
    _idx(idx, q, top_k)
    _like(o, q, "o")
    _expect(lse, _rows(q), torch.float32, "lse")
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    _ws(workspace, moba_attn_fwd_workspace_bytes(q, block_size, top_k, cu_seqlens))
    _check(_load().moba_attn_combine(ctypes.byref(sh), _p(q), _p(k), _p(v), _p(idx),
                                     float(scale or 0.0), _p(o), _p(lse), _p(workspace),
                                     workspace.numel(), _stream(stream)), "moba_attn_combine")


@_on_stream
def moba_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                  block_size: int, top_k: int, scale: Optional[float] = None,
                  cu_seqlens=None, workspace: Optional[torch.Tensor] = None,
                  return_lse: bool = True, out: Optional[torch.Tensor] = None,
                  blasst_lambda: Optional[float] = None, return_kept: bool = False,
                  kept_out: Optional[torch.Tensor] = None, stream=None):
    """Attention over the listed blocks + the causal own block.

    blasst_lambda (0..1): skip, per query, the selected blocks whose
    maximum score is below the running maximum + ln(lambda) (BLASST, blocks
    in ascending order, the own block last; moba_attn_fwd_blasst).
    Returns (o, lse) with lse fp32 [..., heads] (None if not requested);
    with blasst_lambda and return_kept, (o, lse, kept_idx): the attended
    selection (int32 like idx, written into kept_out when given), which
    moba_attn_bwd_blasst takes.
    """
    _qkv(q, k, v)
    _idx(idx, q, top_k)
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    if out is None:
        out = torch.empty_like(q)
    _like(out, q, "out")
    lse = torch.empty(_rows(q), dtype=torch.float32, device=q.device) if return_lse else None
    workspace = _workspace(q, block_size, top_k, cu_seqlens, workspace)
    if return_kept and blasst_lambda is None:
        raise MobaError("return_kept needs blasst_lambda")
    if blasst_lambda is not None:
        kept = None
        if return_kept:
            kept = torch.empty_like(idx) if kept_out is None else kept_out
            _like(kept, idx, "kept_out")
        rc = _load().moba_attn_fwd_blasst(ctypes.byref(sh), _p(q), _p(k), _p(v), _p(idx),
                                          float(scale or 0.0), float(blasst_lambda), _p(out),
                                          _p(lse), _p(kept), _p(workspace), workspace.numel(),
                                          _stream(stream))
        _check(rc, "moba_attn_fwd_blasst")
        return (out, lse, kept) if return_kept else (out, lse)
    rc = _load().moba_attn_fwd(ctypes.byref(sh), _p(q), _p(k), _p(v), _p(idx),
                               float(scale or 0.0), _p(out), _p(lse), _p(workspace),
                               workspace.numel(), _stream(stream))
    _check(rc, "moba_attn_fwd")
    return out, lse


def moba_attn_fwd_blasst(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                         block_size: int, top_k: int, blasst_lambda: float, **kw):
    """moba_attn_fwd with the BLASST block skip (see moba_attn_fwd)."""
    return moba_attn_fwd(q, k, v, idx, block_size, top_k, blasst_lambda=blasst_lambda, **kw)


@_on_stream
def moba_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_size: int, top_k: int,
             conv_w: Optional[torch.Tensor] = None, conv_mode: str = "plain",
             cu_seqlens=None, scale: Optional[float] = None,
             workspace: Optional[torch.Tensor] = None, blasst_lambda: Optional[float] = None,
             stream=None):
    """The whole MoBA forward: [key conv] -> centroids -> route -> attention
    (with the BLASST block skip when blasst_lambda is given).

    Returns (o, lse, idx, k_used) where k_used is k' when a conv ran; with
    blasst_lambda, idx is the attended (kept) selection.  With ``stream``
    every step runs (and every buffer is allocated) on it.
    """
    if conv_w is not None:
        kk, cent = moba_key_conv(k, conv_w, block_size, conv_mode, cu_seqlens,
                                 with_centroids=True)
    else:
        kk = k
        cent = moba_centroids(k, block_size, cu_seqlens)
    if workspace is None:
        need = max(moba_attn_fwd_workspace_bytes(q, block_size, top_k, cu_seqlens),
                   moba_route_topk_workspace_bytes(q, block_size, top_k, cu_seqlens), 256)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    idx = moba_route_topk(q, cent, block_size, top_k, cu_seqlens, workspace=workspace)
    if blasst_lambda is not None:
        o, lse, kept = moba_attn_fwd(q, kk, v, idx, block_size, top_k, scale, cu_seqlens, workspace,
                                     blasst_lambda=blasst_lambda, return_kept=True)
        return o, lse, kept, kk
    o, lse = moba_attn_fwd(q, kk, v, idx, block_size, top_k, scale, cu_seqlens, workspace)
    return o, lse, idx, kk


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_size: int, top_k: int,
        conv_w: Optional[torch.Tensor] = None, conv_mode: str = "plain", cu_seqlens=None,
        scale: Optional[float] = None, stream=None):
    """``moba_fwd`` without the convolved keys: returns (o, lse, idx)."""
    o, lse, idx, _ = moba_fwd(q, k, v, block_size, top_k, conv_w=conv_w, conv_mode=conv_mode,
                              cu_seqlens=cu_seqlens, scale=scale, stream=stream)
    return o, lse, idx


@_on_stream
def moba_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                  o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                  block_size: int, top_k: int, scale: Optional[float] = None,
                  cu_seqlens=None, workspace: Optional[torch.Tensor] = None,
                  out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                  stream=None, _entry: str = "moba_attn_bwd"):
    """Gradients (dq, dk, dv) of moba_attn_fwd's output for the selection idx.

    o and lse are that forward's outputs; dout is dL/dO.  bf16 (fast path) or
    fp32 (plain recompute path).
    """
    _dev(q, k, v, idx, o, lse, dout)
    if not (q.shape == k.shape == v.shape == o.shape == dout.shape):
        raise MobaError("q, k, v, o, dout must share one shape")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise MobaError("q, k, v, o, dout must share one dtype")
    if idx.dtype != torch.int32 or tuple(idx.shape) != _rows(q) + (top_k,):
        raise MobaError("idx must be int32 [..., heads, top_k]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != _rows(q):
        raise MobaError("lse must be fp32 [..., heads]")
    sh, keep = _make_shape(q, block_size, top_k, cu_seqlens)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    for g, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _like(g, q, n)
    need = moba_attn_bwd_workspace_bytes(q, block_size, top_k, cu_seqlens)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _ws(workspace, need)
    rc = getattr(_load(), _entry)(ctypes.byref(sh), _p(q), _p(k), _p(v), _p(idx),
                                  float(scale or 0.0), _p(o), _p(lse), _p(dout), _p(dq),
                                  _p(dk), _p(dv), _p(workspace), workspace.numel(),
                                  _stream(stream))
    _check(rc, _entry)
    return dq, dk, dv


def moba_attn_bwd_blasst(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         kept_idx: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                         dout: torch.Tensor, block_size: int, top_k: int, **kw):
    """Gradients of moba_attn_fwd_blasst's output for the decisions it took:
    kept_idx is that call's attended selection (return_kept=True); a row's
    own block takes part only where kept_idx lists it.  Other arguments as
    moba_attn_bwd."""
    return moba_attn_bwd(q, k, v, kept_idx, o, lse, dout, block_size, top_k,
                         _entry="moba_attn_bwd_blasst", **kw)


class _MobaAttention(torch.autograd.Function):
    """Autograd glue: the forward is moba_fwd, the backward moba_attn_bwd
    (then moba_key_conv_bwd when a key convolution ran).  The block
    selection is piecewise constant in q and k, so no gradient reaches the
    router."""

    @staticmethod
    def forward(ctx, q, k, v, conv_w, block_size, top_k, conv_mode, cu_seqlens, scale,
                blasst_lambda):
        o, lse, idx, kk = moba_fwd(q, k, v, block_size, top_k, conv_w, conv_mode,
                                   cu_seqlens, scale, blasst_lambda=blasst_lambda)
        ctx.save_for_backward(q, k, v, conv_w, o, lse, idx, kk)
        ctx.cfg = (block_size, top_k, conv_mode, cu_seqlens, scale, blasst_lambda)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, conv_w, o, lse, idx, kk = ctx.saved_tensors
        block_size, top_k, conv_mode, cu_seqlens, scale, blasst_lambda = ctx.cfg
        bwd = moba_attn_bwd if blasst_lambda is None else moba_attn_bwd_blasst
        dq, dkk, dv = bwd(q, kk, v, idx, o, lse, do.contiguous(), block_size, top_k,
                          scale=scale, cu_seqlens=cu_seqlens)
        dk, dw = dkk, None
        if conv_w is not None:
            dk, dw = moba_key_conv_bwd(k, conv_w, dkk, block_size, conv_mode, cu_seqlens)
        return dq, dk, dv, dw, None, None, None, None, None, None


def moba_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_size: int,
                   top_k: int, conv_w: Optional[torch.Tensor] = None,
                   conv_mode: str = "plain", cu_seqlens=None,
                   scale: Optional[float] = None,
                   blasst_lambda: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MoBA attention as a differentiable op: returns (o, lse).

    Gradients flow to q, k, v and the conv filter (the selection itself
    carries none).  With blasst_lambda the forward applies the BLASST block
    skip and the backward differentiates the kept blocks' softmax (BLASST's
    sparsity-aware training); the skip decisions carry no gradient either.
    """
    return _MobaAttention.apply(q, k, v, conv_w, block_size, top_k, conv_mode, cu_seqlens, scale,
                                blasst_lambda)
