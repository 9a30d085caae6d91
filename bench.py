"""Benchmark of the MoBA forward on one MI355X.

One step = one whole forward pass over one batch of synthetic input:
[key conv + pooling | pooling] -> routing -> index inversion -> routed
attention -> own block + merge, every stage a HIP kernel of libmoba_amd.so.
Inputs sit in HBM before the timed region; outputs and the workspace are
preallocated.  Default workload: 2 x 65536 tokens, 16 heads, d = 64, B = 128,
top-8, bf16 (the pages' 64K / B=128 / k=8 efficiency setting).

value = effective TFLOP/s = F_eff / t_step, F_eff counting only the selected
blocks' QK^T and PV (4 d FLOPs per attended key, own block token-causal).
The JSON line also carries the roofline of the dominant kernel (routed
attention, timed live with HIP events on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads  # noqa: E402

METRIC = "MoBA fwd effective TFLOP/s at N=64K B=128 top-8 bf16; % of MFMA bf16 peak"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_routed_attn_H.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_long_key_amd", "csrc", "attn.hip")


def _src_hash() -> str:
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(per_launch_algo_bytes):
    """HBM bytes per launch of the routed kernel from committed PMC counters,
    or None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attn_src_sha256_16") != _src_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(spec, x, nthreads=None, max_slices=32):
    """The CPU oracle (as it stands) on a bounded sample: the first
    `max_slices` (sequence, head) slices of the workload (all 32 at the
    default workload, i.e. the whole forward), each a full forward of one
    head of one sequence, on up to 16 threads (one slice per thread at a
    time)."""
    import numpy as np

    import oracle

    avail = len(os.sched_getaffinity(0))
    threads = nthreads or min(16, avail)
    n = max(1, min(max_slices, spec.batch * spec.heads))
    b_sl = []
    H = spec.heads
    q = x["q"].float().numpy()
    k = x["k"].float().numpy()
    v = x["v"].float().numpy()
    for r in range(n):
        b, h = divmod(r, H)
        b_sl.append((b, h))
    # stack the sampled slices as one "batch" of n sequences with one head
    qs = np.ascontiguousarray(np.stack([q[b, :, h] for b, h in b_sl])[:, :, None, :])
    ks = np.ascontiguousarray(np.stack([k[b, :, h] for b, h in b_sl])[:, :, None, :])
    vs = np.ascontiguousarray(np.stack([v[b, :, h] for b, h in b_sl])[:, :, None, :])
    w = None
    if x["conv_w"] is not None:
        raise NotImplementedError("cpu baseline sample covers conv-free workloads")
    cu = [i * spec.seq for i in range(n + 1)]
    t0 = time.perf_counter()
    oracle.forward(qs.reshape(-1, 1, spec.head_dim), ks.reshape(-1, 1, spec.head_dim),
                   vs.reshape(-1, 1, spec.head_dim), spec.block_size, spec.top_k, cu,
                   conv_w=w, nthreads=threads)
    dt = time.perf_counter() - t0
    f_sample = workloads.eff_flops(spec)["total"] * n / (spec.batch * spec.heads)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": f_sample / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{n} of {spec.batch * spec.heads} (sequence, head) slices, full forward "
                  f"(centroids, routing, attention) in fp64 C on {threads} threads; "
                  f"{dt:.1f} s; cpu: {model}",
        "seconds": dt,
    }


def _calib_copy(args, dev):
    """One plain device copy of --calib-copy-mib MiB (a kernel of known size
    for scaling the HBM byte counters)."""
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="H", choices=sorted(workloads.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="fwd (default): the forward pass; bwd: the attention "
                         "backward (moba_attn_bwd) for the forward's selection")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a "
                         "known-size kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import block_sparse_long_key_amd as moba

    if args.which == "bwd":
        return bench_bwd(args, moba)
    spec = workloads.spec(args.config)
    x = workloads.make(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(dev)
    cu = x["cu_seqlens"]
    B, K = spec.block_size, spec.top_k
    nb = moba.moba_total_blocks(q, B, cu)
    cent = torch.empty((nb, spec.heads, spec.head_dim), dtype=torch.float32, device=dev)
    kc = torch.empty_like(k) if w is not None else None
    idx = torch.empty(q.shape[:-1] + (K,), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, moba.moba_attn_fwd_workspace_bytes(q, B, K, cu),
                         moba.moba_route_topk_workspace_bytes(q, B, K, cu)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    names = (["conv_pool"] if w is not None else ["pool"]) + ["route", "index", "routed_attn",
                                                            "diag_combine"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        if w is not None:
            moba.moba_key_conv(k, w, B, spec.conv_mode, cu, with_centroids=True, out=kc, cent=cent)
            kk = kc
        else:
            moba.moba_centroids(k, B, cu, out=cent)
            kk = k
        mark(1)
        moba.moba_route_topk(q, cent, B, K, cu, out=idx, workspace=ws)
        mark(2)
        moba.moba_attn_index(idx, q, B, K, ws, cu)
        mark(3)
        moba.moba_attn_routed(q, kk, v, B, K, ws, None, cu)
        mark(4)
        moba.moba_attn_combine(q, kk, v, idx, B, K, ws, o, lse, None, cu)
        mark(5)

    _calib_copy(args, dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: whole steps, bracketed by syncs
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_steps = [e[0].elapsed_time(e[5]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    stage_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
                for j, n in enumerate(names)}

    fl = workloads.eff_flops(spec)
    value = fl["total"] / (ms_step * 1e-3) / 1e12
    routed_ms = stage_ms["routed_attn"]
    routed_tflops = fl["routed"] / (routed_ms * 1e-3) / 1e12
    pairs = workloads.routed_pairs(spec)
    traffic = _traffic(pairs) if args.config == "H" else None

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic (seeded i.i.d. N(0,1) q/k/v, CPU torch.Generator)",
        "config": {"workload": f"moba_fwd {spec.name}: {spec.desc}",
                   "batch": spec.batch, "seq_len": spec.seq, "heads": spec.heads,
                   "head_dim": spec.head_dim, "block_size": B, "top_k": K,
                   "key_conv_width": spec.conv_width, "key_conv_mode": spec.conv_mode,
                   "F_eff": fl["total"]},
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "stage_ms": {n: round(t, 4) for n, t in stage_ms.items()},
        "event_ms_per_step": round(sum(ms_steps) / len(ms_steps), 4),
        "event_ms_median": round(sorted(ms_steps)[len(ms_steps) // 2], 4),
        "event_ms_min": round(min(ms_steps), 4),
        "event_ms_max": round(max(ms_steps), 4),
        "roofline": {
            "kernel": "routed_attn_kernel (moba_attn_routed)",
            "bound": "mfma",
            "achieved": round(routed_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(routed_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": fl["routed"],
            "avg_launch_ms": round(routed_ms, 4),
            # the kernel is bound by its HBM traffic in practice: the same
            # bytes over the same time
            "traffic_GBps": (round(traffic / (routed_ms * 1e-3) / 1e9, 1)
                             if traffic else None),
        },
    }
    if not args.no_cpu_baseline and spec.conv_width == 0:
        out["cpu_baseline"] = cpu_baseline(spec, x)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_bwd(args, moba):
    """One step = one moba_attn_bwd call (index inversion, D = dO.O, the
    per-key-block list kernel and the dq merge) on the forward's selection,
    o and lse, which are computed once before the timed region; with a key
    convolution, also moba_key_conv_bwd (dk' -> dk, dw)."""
    spec = workloads.spec(args.config)
    x = workloads.make(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(dev)
    do = workloads.grad_output(spec).to(dev)
    cu = x["cu_seqlens"]
    B, K = spec.block_size, spec.top_k
    o, lse, idx, kk = moba.moba_fwd(q, k, v, B, K, conv_w=w, conv_mode=spec.conv_mode, cu_seqlens=cu)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(256, moba.moba_attn_bwd_workspace_bytes(q, B, K, cu)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    _calib_copy(args, dev)

    wsc = None
    if w is not None:
        wsc = torch.empty(max(256, moba.moba_key_conv_bwd_workspace_bytes(k, B, w.shape[2], cu)),
                          dtype=torch.uint8, device=dev)

    def step():
        moba.moba_attn_bwd(q, kk, v, idx, o, lse, do, B, K, cu_seqlens=cu, workspace=ws,
                           out=(dq, dk, dv))
        if w is not None:
            # dL/dk' -> dL/dk and dL/dw through the key convolution
            moba.moba_key_conv_bwd(k, w, dk, B, spec.conv_mode, cu_seqlens=cu, workspace=wsc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps
    ms_ev = [a.elapsed_time(b) for a, b in evs]
    fl = workloads.eff_flops_bwd(spec)
    value = fl["total"] / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "MoBA attention bwd effective TFLOP/s (10 d FLOPs per attended key)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1) q/k/v/dO, CPU torch.Generator)",
        "config": {"workload": f"moba_attn_bwd {spec.name}: {spec.desc}",
                   "batch": spec.batch, "seq_len": spec.seq, "heads": spec.heads,
                   "head_dim": spec.head_dim, "block_size": B, "top_k": K,
                   "F_eff_bwd": fl["total"]},
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "event_ms_median": round(sorted(ms_ev)[len(ms_ev) // 2], 4),
        "event_ms_min": round(min(ms_ev), 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
