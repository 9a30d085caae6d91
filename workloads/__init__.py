"""Seeded synthetic workloads for the MoBA forward pass.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no convolution, pooling, scoring, selection or attention).
Both the CPU oracle tests and the GPU tests / benchmark take their inputs from
here, so the two sides see identical tensors.

Shapes follow the task definition of "Optimizing Mixture of Block Attention"
(summary page, section "Definizione del Compito"): q, k, v of sequence length
N, split into blocks of B keys, each query keeping k blocks.  Layout is
``[batch, seq, heads, head_dim]`` (varlen: ``[total_tokens, heads, head_dim]``
plus ``cu_seqlens``), head_dim fastest.

Recipe (identical for every config):
  1. ``g = torch.Generator().manual_seed(seed)`` on the CPU;
  2. draw fp32 ``randn`` for q, then k, then v, each of the full shape;
  3. if the config has a key convolution of width W, draw its weights
     ``randn(heads, head_dim, W) * sqrt(1/W)`` (so each weight ~ N(0, 1/W));
  4. apply the planted routing signal if the config has one (C3 only);
  5. round q, k, v to the config dtype (bf16 round-to-nearest-even by torch).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

__all__ = ["Spec", "CONFIGS", "spec", "make", "segments", "eff_flops",
           "routed_pairs", "grad_output", "eff_flops_bwd", "routing_bytes"]


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    seed: int
    batch: int
    seq: int                  # per-batch length (uniform) or total tokens (varlen)
    heads: int
    head_dim: int
    block_size: int
    top_k: int
    dtype: str                # "f32" | "bf16"
    conv_width: int = 0       # 0 = no key convolution
    conv_mode: str = "plain"  # "plain" or "silu_residual" (k + SiLU(conv), the page's form)
    seqlens: Optional[tuple] = None   # varlen lengths (batch must be 1)
    plant: bool = False       # C3's planted per-query-block signal
    sink: bool = False        # every query's router favours block 0 (attention sink)
    desc: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def scaled(self, seq: int, name_suffix: str = "-small") -> "Spec":
        """Same B / k / d / W / structure, shorter sequences (parity sizes)."""
        if self.seqlens is not None:
            tot = sum(self.seqlens)
            lens = tuple(max(1, (l * seq) // tot) for l in self.seqlens)
            # keep the total exactly `seq`
            lens = lens[:-1] + (seq - sum(lens[:-1]),)
            return dataclasses.replace(self, name=self.name + name_suffix,
                                       seq=seq, seqlens=lens)
        return dataclasses.replace(self, name=self.name + name_suffix, seq=seq)


CONFIGS = {
    "C1": Spec("C1", 1, 1, 1024, 1, 64, 64, 4, "f32",
               desc="tiny fp32: b1 H1 N1024 d64 B64 (16 blocks) top-4"),
    "C2": Spec("C2", 2, 1, 8192, 16, 64, 128, 8, "bf16",
               desc="b1 H16 N8192 d64 B128 (64 blocks) top-8 bf16"),
    "C3": Spec("C3", 3, 2, 32768, 16, 64, 128, 8, "bf16", conv_width=3,
               plant=True,
               desc="b2 H16 N32768 d64 B128 top-8 bf16, key conv W=3, "
                    "planted signal"),
    "C4": Spec("C4", 4, 1, 65536, 16, 64, 64, 16, "bf16",
               desc="b1 H16 N65536 d64 B64 (1024 blocks) top-16 bf16"),
    "C5": Spec("C5", 5, 1, 131072, 16, 128, 128, 8, "bf16", conv_width=4,
               seqlens=(65536, 32768, 16384, 16384),
               desc="varlen 4 seqs (65536,32768,16384,16384) H16 d128 B128 "
                    "top-8 bf16, key conv W=4"),
    "H": Spec("H", 6, 2, 65536, 16, 64, 128, 8, "bf16",
              desc="b2 H16 N65536 d64 B128 top-8 bf16 (64K, B=128, top-8)"),
    # the pages' larger-block variants at the same 7/8 sparsity (MoBA-256:
    # B=256 k=4; MoBA-512: B=512 k=2), at the efficiency setting's shape
    "M256": Spec("M256", 8, 2, 65536, 16, 64, 256, 4, "bf16",
                 desc="b2 H16 N65536 d64 B256 top-4 bf16 (MoBA-256)"),
    "M512": Spec("M512", 9, 2, 65536, 16, 64, 512, 2, "bf16",
                 desc="b2 H16 N65536 d64 B512 top-2 bf16 (MoBA-512)"),
    # the pages' best-quality variant "MoBA-128 + kconv5": the key conv in
    # the page's k + SiLU(conv) form with W = 5, at the efficiency shape
    "H5": Spec("H5", 10, 2, 65536, 16, 64, 128, 8, "bf16", conv_width=5,
               conv_mode="silu_residual",
               desc="b2 H16 N65536 d64 B128 top-8 bf16, key conv W=5 k+SiLU(conv) (kconv5)"),
    # long context (the efficiency figure's longest sequence): one 512K
    # sequence, 16 heads, d=64, B=128, top-8
    "L": Spec("L", 7, 1, 524288, 16, 64, 128, 8, "bf16",
              desc="b1 H16 N524288 d64 B128 top-8 bf16 (512K long context)"),
}


def spec(name: str) -> Spec:
    return CONFIGS[name]


def segments(s: Spec) -> List[int]:
    """cu_seqlens over the flattened token axis (uniform batch -> batch segs)."""
    if s.seqlens is not None:
        cu = [0]
        for l in s.seqlens:
            cu.append(cu[-1] + l)
        return cu
    return [b * s.seq for b in range(s.batch + 1)]


def _plant(q: torch.Tensor, k: torch.Tensor, s: Spec, g: torch.Generator):
    """C3 planted signal (plainest reading of the config prose).

    For each batch b, head h and query block i >= 1 (ascending): take the unit
    direction of the block's mean query (fp32, before rounding), draw
    min(4, i) distinct earlier blocks with randperm(i), and add 0.5 * that
    direction to every key of each drawn block.  Plants accumulate.
    """
    B = s.block_size
    nblk = s.seq // B
    for b in range(s.batch):
        for h in range(s.heads):
            for i in range(1, nblk):
                qm = q[b, i * B:(i + 1) * B, h, :].mean(dim=0)
                qhat = qm / qm.norm()
                picks = torch.randperm(i, generator=g)[:min(4, i)]
                for j in picks.tolist():
                    k[b, j * B:(j + 1) * B, h, :] += 0.5 * qhat


def _sink(q: torch.Tensor, k: torch.Tensor, s: Spec, g: torch.Generator):
    """Attention-sink structure: one random unit direction u per head; every
    query gets +2u and every key of block 0 of each sequence gets +4u, so
    block 0 has the highest router score for (nearly) every query and its
    key-block list holds (nearly) all queries of the sequence."""
    u = torch.randn((s.heads, s.head_dim), generator=g, dtype=torch.float32)
    u = u / u.norm(dim=-1, keepdim=True)
    q += 2.0 * u
    B = s.block_size
    if s.seqlens is not None:
        starts = [0]
        for l in s.seqlens[:-1]:
            starts.append(starts[-1] + l)
        for a, l in zip(starts, s.seqlens):
            k[a:a + min(B, l)] += 4.0 * u
    else:
        k[:, :B] += 4.0 * u


def make(s, seed: Optional[int] = None, device="cpu"):
    """Draw the inputs of config `s` (a Spec or a config name).

    Returns a dict with q, k, v (config dtype, on `device`), conv_w (fp32
    [heads, head_dim, W] or None), cu_seqlens (python list or None for
    uniform batches) and the spec.
    """
    if isinstance(s, str):
        s = spec(s)
    g = torch.Generator().manual_seed(s.seed if seed is None else seed)
    if s.seqlens is not None:
        shape = (s.seq, s.heads, s.head_dim)
    else:
        shape = (s.batch, s.seq, s.heads, s.head_dim)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    w = None
    if s.conv_width > 0:
        w = torch.randn((s.heads, s.head_dim, s.conv_width), generator=g,
                        dtype=torch.float32) * math.sqrt(1.0 / s.conv_width)
    if s.plant:
        _plant(q, k, s, g)
    if s.sink:
        _sink(q, k, s, g)
    dt = s.torch_dtype
    out = {
        "q": q.to(dt).to(device),
        "k": k.to(dt).to(device),
        "v": v.to(dt).to(device),
        "conv_w": None if w is None else w.to(device),
        "cu_seqlens": segments(s) if s.seqlens is not None else None,
        "spec": s,
    }
    return out


def grad_output(s, seed: Optional[int] = None, device="cpu") -> torch.Tensor:
    """dL/dO for the attention backward: standard normal, shaped like q, in
    the config dtype, from its own generator (seed + 10007) so the forward
    inputs stay those of make()."""
    if isinstance(s, str):
        s = spec(s)
    g = torch.Generator().manual_seed((s.seed if seed is None else seed) + 10007)
    if s.seqlens is not None:
        shape = (s.seq, s.heads, s.head_dim)
    else:
        shape = (s.batch, s.seq, s.heads, s.head_dim)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(s.torch_dtype).to(device)


def routed_pairs(s: Spec) -> int:
    """Number of (query, routed past block) pairs over all (sequence, head).

    Closed form of the counting in the task definition: a query in block i
    keeps min(k-1, i) past blocks besides its own (past blocks are full).
    """
    total = 0
    B, k = s.block_size, s.top_k
    lens = s.seqlens if s.seqlens is not None else (s.seq,) * s.batch
    for L in lens:
        for i in range((L + B - 1) // B):
            nq = min(B, L - i * B)
            total += nq * min(k - 1, i)
    return total * s.heads


def eff_flops(s: Spec) -> dict:
    """Effective (selected-block, mask-aware) FLOPs of one forward pass.

    Per query t in block i at in-block position p: 4*d*(B*min(k-1,i) + p+1)
    (QK^T and PV, 2 FLOPs per multiply-add each).  The router's scores are not
    counted.  Returns {"routed": ..., "diag": ..., "total": ...}.
    """
    B, k, d = s.block_size, s.top_k, s.head_dim
    lens = s.seqlens if s.seqlens is not None else (s.seq,) * s.batch
    routed = 0
    diag = 0
    for L in lens:
        for i in range((L + B - 1) // B):
            nq = min(B, L - i * B)
            routed += nq * min(k - 1, i) * B
            diag += nq * (nq + 1) // 2
    routed *= 4 * d * s.heads
    diag *= 4 * d * s.heads
    return {"routed": routed, "diag": diag, "total": routed + diag}


def eff_flops_bwd(s: Spec) -> dict:
    """Effective FLOPs of the attention backward: per (query, key) pair the
    recomputed scores, dP, dV, dK and dQ products, 2*d FLOPs each (10*d),
    i.e. 2.5 times the forward's 4*d."""
    f = eff_flops(s)
    return {n: v * 5 // 2 for n, v in f.items()}


def routing_bytes(s: Spec) -> dict:
    """Algorithmic HBM bytes of the routing stages of one forward (every
    tensor moved once): key conv + pooling (k read, k' written, centroids
    written) or pooling alone (k read, centroids written); the router (q
    read, the centroids read once per (sequence, head), idx written); the
    index inversion (idx read, one 4-byte entry written per (query, routed
    block) pair)."""
    esz = 4 if s.dtype == "f32" else 2
    d, H, K = s.head_dim, s.heads, s.top_k
    tokens = sum(s.seqlens) if s.seqlens is not None else s.batch * s.seq
    lens = s.seqlens if s.seqlens is not None else (s.seq,) * s.batch
    blocks = sum((L + s.block_size - 1) // s.block_size for L in lens)
    kv = tokens * H * d * esz
    cent = blocks * H * d * 4
    idx = tokens * H * K * 4
    out = {"pool": kv + cent}
    if s.conv_width > 0:
        out = {"conv_pool": 2 * kv + cent}
    out["route"] = kv + cent + idx
    out["index"] = idx + routed_pairs(s) * 4
    return out
