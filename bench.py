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


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(spec, x, nthreads=None, budget_s=10.0):
    """The CPU oracle (as it stands) on a bounded sample of the workload: the
    whole forward (key conv when the workload has one, centroids, routing,
    attention) of whole sequences with every head, on up to 16 threads (one
    (sequence, head) at a time per thread).  Sequences are timed one after
    another in their order until budget_s seconds have been spent or all of
    them are done, so a slow host times fewer of them; the value is the
    sampled sequences' effective FLOPs over their time.  A sequence longer
    than 131072 tokens is cut to its first 131072 (the full routing of the
    512K-token sequence alone would take minutes).  C1 (one head, 1024
    tokens) is also timed on one thread."""
    import dataclasses

    import oracle

    avail = len(os.sched_getaffinity(0))
    threads = min(nthreads or min(16, avail), spec.heads)
    H = spec.heads
    w = x["conv_w"]
    mode = 0 if spec.conv_mode == "plain" else 1
    rb = spec.dtype == "bf16"
    cap = 131072
    # the workload's sequences as (q, k, v) token slices [L, H, d]
    if spec.seqlens is not None:
        cu = x["cu_seqlens"]
        seqs = [tuple(x[n][cu[i]:cu[i + 1]] for n in ("q", "k", "v")) for i in range(len(cu) - 1)]
    else:
        seqs = [tuple(x[n][b] for n in ("q", "k", "v")) for b in range(spec.batch)]
    cut = any(t[0].shape[0] > cap for t in seqs)
    seqs = [tuple(a[:cap] for a in t) for t in seqs]

    def run(t, th):
        q, k, v = (a.float().contiguous() for a in t)
        L = q.shape[0]
        t0 = time.perf_counter()
        oracle.forward(q, k, v, spec.block_size, spec.top_k, [0, L], conv_w=w, conv_mode=mode,
                       round_bf16=rb, nthreads=th)
        return time.perf_counter() - t0

    def flops(L):
        one = dataclasses.replace(spec, batch=1, seq=L, seqlens=None)
        return workloads.eff_flops(one)["total"]

    dt, f_sample, ntok, done = 0.0, 0, 0, 0
    for t in seqs:
        dt += run(t, threads)
        f_sample += flops(t[0].shape[0])
        ntok += t[0].shape[0]
        done += 1
        if dt >= budget_s:
            break
    steps = ("key conv, " if w is not None else "") + "centroids, routing, attention"
    what = (f"{done} of the {len(seqs)} sequence(s)" + (f" (each cut to its first {cap} tokens)" if cut else "")
            + f", {ntok} tokens")
    out = {
        "value": f_sample / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{what}, all {H} heads: full forward ({steps}) in fp64 C on {threads} "
                  f"threads; {dt:.1f} s (sequences are added until {budget_s:.0f} s are spent); "
                  f"cpu: {_cpu_model()}",
        "seconds": dt,
    }
    if spec.name == "C1":
        dt1 = sum(run(t, 1) for t in seqs[:done])
        out["single_thread"] = {"value": f_sample / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                                "seconds": dt1}
    return out


def _memory(dev, workspace_bytes):
    """Device memory of the step: the workspace, and torch's peak allocated
    bytes over the warm-up and timed steps (inputs, outputs, centroids, idx
    and workspaces: the library itself allocates nothing)."""
    return {"workspace_bytes": int(workspace_bytes),
            "peak_allocated_bytes": int(torch.cuda.max_memory_allocated(dev)),
            "peak_allocated_GiB": round(torch.cuda.max_memory_allocated(dev) / 2**30, 3)}


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
    ap.add_argument("--blasst-lambda", type=float, default=None,
                    help="time the forward with the BLASST block skip at this lambda "
                         "(moba_attn_fwd_blasst as one stage after routing)")
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
    blasst = args.blasst_lambda is not None
    if blasst:
        names = names[:2] + ["attn_blasst"]

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
        if blasst:
            moba.moba_attn_fwd_blasst(q, kk, v, idx, B, K, args.blasst_lambda, cu_seqlens=cu,
                                      workspace=ws, out=o)
            mark(3)
            return
        moba.moba_attn_index(idx, q, B, K, ws, cu)
        mark(3)
        moba.moba_attn_routed(q, kk, v, B, K, ws, None, cu)
        mark(4)
        moba.moba_attn_combine(q, kk, v, idx, B, K, ws, o, lse, None, cu)
        mark(5)

    _calib_copy(args, dev)
    torch.cuda.reset_peak_memory_stats(dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: whole steps, bracketed by syncs
    nev = len(names) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_steps = [e[0].elapsed_time(e[nev - 1]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    stage_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
                for j, n in enumerate(names)}

    fl = workloads.eff_flops(spec)
    value = fl["total"] / (ms_step * 1e-3) / 1e12
    routed_ms = stage_ms["attn_blasst" if blasst else "routed_attn"]
    routed_flops = fl["total"] if blasst else fl["routed"]
    routed_tflops = routed_flops / (routed_ms * 1e-3) / 1e12
    pairs = workloads.routed_pairs(spec)
    traffic = _traffic(pairs) if args.config == "H" and not blasst else None
    # the routing stages against the HBM roofline: algorithmic bytes (every
    # tensor moved once) over the event-timed stage time
    rbytes = workloads.routing_bytes(spec)
    if blasst:
        rbytes.pop("index")
    routing = {}
    for n, b in rbytes.items():
        t = stage_ms[n] * 1e-3
        routing[n] = {"ms": round(stage_ms[n], 4), "alg_bytes": b,
                      "GBps": round(b / t / 1e9, 1),
                      "pct_of_hbm_peak": round(100 * b / t / 1e9 / PEAK_HBM_GBS, 1)}

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
        "config": {"workload": f"moba_fwd {spec.name}: {spec.desc}"
                               + (f", BLASST lambda={args.blasst_lambda}" if blasst else ""),
                   "batch": spec.batch, "seq_len": spec.seq, "heads": spec.heads,
                   "head_dim": spec.head_dim, "block_size": B, "top_k": K,
                   "key_conv_width": spec.conv_width, "key_conv_mode": spec.conv_mode,
                   "F_eff": fl["total"]},
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "stage_ms": {n: round(t, 4) for n, t in stage_ms.items()},
        "routing_hbm": routing,
        "event_ms_per_step": round(sum(ms_steps) / len(ms_steps), 4),
        "event_ms_median": round(sorted(ms_steps)[len(ms_steps) // 2], 4),
        "event_ms_min": round(min(ms_steps), 4),
        "event_ms_max": round(max(ms_steps), 4),
        "roofline": {
            "kernel": ("moba_attn_fwd_blasst (index + routed + own block and merge)" if blasst
                       else "routed_attn_kernel (moba_attn_routed)"),
            "bound": "mfma",
            "achieved": round(routed_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(routed_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": routed_flops,
            "avg_launch_ms": round(routed_ms, 4),
            # the kernel is bound by its HBM traffic in practice: the same
            # bytes over the same time
            "traffic_GBps": (round(traffic / (routed_ms * 1e-3) / 1e9, 1)
                             if traffic else None),
        },
    }
    out["memory"] = _memory(dev, ws.numel())
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(spec, x)
    print(json.dumps(out), flush=True)


def _attended_keys(kept, cu, B):
    """(query, key) pairs a kept selection attends: B keys per listed past
    block (a past block is always whole) plus the causal own-block keys of
    the rows that list their own block.  Runs on the device, untimed."""
    T, H, K = kept.shape
    tl = torch.empty(T, dtype=torch.int64, device=kept.device)
    for a, b in zip(cu[:-1], cu[1:]):
        tl[a:b] = torch.arange(b - a, device=kept.device)
    own = (tl // B)[:, None, None]
    past = ((kept >= 0) & (kept < own)).sum()
    own_rows = (kept == own).any(-1)
    causal = (tl % B + 1)[:, None].expand(T, H)
    return int(past) * B + int(causal[own_rows].sum())


def bench_bwd(args, moba):
    """One step = one moba_attn_bwd call (index inversion, D = dO.O, the
    per-key-block list kernel and the dq merge) on the forward's selection,
    o and lse, which are computed once before the timed region; with a key
    convolution, also moba_key_conv_bwd (dk' -> dk, dw).  With
    --blasst-lambda the forward is the BLASST one and the step is
    moba_attn_bwd_blasst on its kept selection; FLOPs count the kept pairs."""
    spec = workloads.spec(args.config)
    x = workloads.make(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    w = None if x["conv_w"] is None else x["conv_w"].to(dev)
    do = workloads.grad_output(spec).to(dev)
    cu = x["cu_seqlens"]
    B, K = spec.block_size, spec.top_k
    blasst = args.blasst_lambda is not None
    o, lse, idx, kk = moba.moba_fwd(q, k, v, B, K, conv_w=w, conv_mode=spec.conv_mode, cu_seqlens=cu,
                                    blasst_lambda=args.blasst_lambda)
    bwd = moba.moba_attn_bwd_blasst if blasst else moba.moba_attn_bwd
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
        bwd(q, kk, v, idx, o, lse, do, B, K, cu_seqlens=cu, workspace=ws, out=(dq, dk, dv))
        if w is not None:
            # dL/dk' -> dL/dk and dL/dw through the key convolution
            moba.moba_key_conv_bwd(k, w, dk, B, spec.conv_mode, cu_seqlens=cu, workspace=wsc)

    torch.cuda.reset_peak_memory_stats(dev)
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
    if blasst:
        cu_tok = workloads.segments(spec)
        fl = {"total": 10 * spec.head_dim * _attended_keys(idx.reshape(-1, spec.heads, K), cu_tok, B)}
    value = fl["total"] / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "MoBA attention bwd effective TFLOP/s (10 d FLOPs per attended key)"
                  + (f", BLASST lambda={args.blasst_lambda} (kept pairs only)" if blasst else ""),
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
        "data": "synthetic (seeded i.i.d. N(0,1) q/k/v/dO, CPU torch.Generator)",
        "config": {"workload": f"{'moba_attn_bwd_blasst' if blasst else 'moba_attn_bwd'} "
                               f"{spec.name}: {spec.desc}",
                   "batch": spec.batch, "seq_len": spec.seq, "heads": spec.heads,
                   "head_dim": spec.head_dim, "block_size": B, "top_k": K,
                   "F_eff_bwd": fl["total"]},
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "event_ms_median": round(sorted(ms_ev)[len(ms_ev) // 2], 4),
        "event_ms_min": round(min(ms_ev), 4),
        "memory": _memory(dev, ws.numel() + (wsc.numel() if wsc is not None else 0)),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
