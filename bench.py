#!/usr/bin/env python3
"""Throughput of one sparse-linear attention layer forward through libsla on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan13b_sla]

A step is one pass of the whole hot path over one batch of synthetic input already
resident in HBM: pooled scores, block map, linear key states, marginal sums and the
attention kernel with its fused linear epilogue, on one stream (the key states run first when
they also write the key block means, so the pooling pass reads only Q; --overlap runs the key
states and marginal sums on a second HIP stream beside the scores and the block map).  Prints
one JSON line.

value = effective TFLOP/s = dense-equivalent attention FLOPs (4 B Hq Nv^2 d, halved when
causal) / measured time per layer; ms_per_step = milliseconds per layer forward.
The roofline entry covers the pass that takes the most time, measured with HIP events
recorded on the stream its kernels are launched on, over the timed steps.
cpu_baseline times the CPU oracle on a bounded sample (whole heads) of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SLA fwd ms/layer + effective TFLOP/s, B1 H12 N32768 d128 bf16, 5% crit"


def metric_for(w):
    """The headline metric for its own workload; the same form, naming the shape, for the others."""
    if w.name == "wan13b_sla":
        return METRIC
    mode = {"sla": "SLA", "salad": "SALAD", "nsa": "NSA-style selected + window"}[w.mode]
    sparsity = (f"{w.kh_bp / 100:g}% crit" if w.mode != "nsa" else f"{w.n_sel} selected + {w.window}-token window")
    return (f"{mode} fwd ms/layer + effective TFLOP/s, B{w.B} H{w.Hq}/{w.Hkv} N{w.N} d{w.d} "
            f"{'bf16' if w.dtype == 'bf16' else 'fp32'}, {sparsity}")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak
PEAK_FP64_TFLOPS = 78.6       # MI355X fp64 (vector and matrix cores)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAKS = {"mfma": PEAK_BF16_TFLOPS, "fp64": PEAK_FP64_TFLOPS, "hbm": PEAK_HBM_GBS}
PASSES = ["pool", "scores", "block_map", "kv_reduce", "marginal_states", "attention"]
KERNEL_SOURCES = {
    "pool": "pool_scores.hip", "scores": "pool_scores.hip", "block_map": "block_map.hip",
    "kv_reduce": "kv_reduce.hip", "marginal_states": "marginal.hip", "attention": "attn_fwd.hip",
}
# the kernel whose counters stand for each pass (a substring of its name in rocprofv3 output)
PASS_KERNEL = {"attention": "attn_fwd_kernel", "marginal_states": "marginal_gemm_kernel",
               "kv_reduce": "kv_state_kernel", "pool": "pool_kernel", "scores": "scores_kernel",
               "block_map": "classify_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pass_work(w, layer):
    """Algorithmic work of one launch of each pass: (bound, bytes or FLOPs)."""
    B, Hq, Hkv, d, Nv, nb = w.B, w.Hq, w.Hkv, w.d, w.Nv, w.nb
    eb = 2 if w.dtype == "bf16" else 4
    Hs = Hkv if layer.group else Hq
    rows = B * Hs * nb
    n_crit_entries = int(layer.maps["crit_rowptr"][-1].item())
    n_marg_entries = int(layer.maps["marg_rowptr"][-1].item()) if "marg_rowptr" in layer.maps else 0
    G = Hq // Hkv
    heads_per_row = G if layer.group else 1
    pair_flops = 4.0 * 64 * 64 * d                 # QK^T and PV of one 64 x 64 block pair
    work = {}
    # Q (and K, unless the key-state pass pools it) in, fp32 block means out
    pooled = Hq if getattr(layer, "fuse_key_pooling", False) else Hq + Hkv
    work["pool"] = ("hbm", B * pooled * (Nv * d * eb + nb * d * 4))
    # pooled scores on the fp64 matrix cores: 2 d FLOP per (row, candidate) pair
    work["scores"] = ("fp64", 2.0 * rows * nb * d * (Hq // Hkv if layer.group else 1))
    work["block_map"] = ("hbm", rows * nb * 4 + (n_crit_entries + n_marg_entries) * 4 + rows * 20)
    if layer.lin == 1:
        # K, V in; one bf16 state + fp32 z (+ the fp32 key block mean when fused) per key block out
        kmean = d * 4 if getattr(layer, "fuse_key_pooling", False) else 0
        work["kv_reduce"] = ("hbm", 2 * B * Hkv * Nv * d * eb + B * Hkv * nb * (d * d * 2 + d * 4 + kmean))
        # mask product S = M H: reads every bf16 state and z once, writes bf16 row sums + fp32 u
        work["marginal_states"] = ("hbm", B * Hkv * nb * (d * d * 2 + d * 4) + rows * (d * d * 2 + d * 4))
    elif layer.lin == 2:
        kmean = B * Hkv * nb * d * 4 if getattr(layer, "fuse_key_pooling", False) else 0
        work["kv_reduce"] = ("hbm", 2 * B * Hkv * Nv * d * eb + B * Hkv * (d * d + d) * 4 + kmean)
        work["marginal_states"] = ("hbm", 0)
    else:
        work["kv_reduce"] = ("hbm", 0)
        work["marginal_states"] = ("hbm", 0)
    attn = n_crit_entries * heads_per_row * pair_flops
    if layer.lin != 0:
        attn += B * Hq * nb * 64 * 2.0 * d * d    # linear epilogue phi(Q) S per query block
    if getattr(layer, "proj_w", None) is not None:
        attn += B * Hq * nb * 64 * 2.0 * d * d    # Proj: O_l W^T per query block
    work["attention"] = ("mfma", attn)
    return work, n_crit_entries * heads_per_row


def proj_weights(w, kind):
    """Seeded Proj weight (one [d, d] for all heads, or one per head) and bias, fp32 CPU tensors."""
    import numpy as np
    import torch
    r = np.random.default_rng(w.seed + 77)
    shape = (w.d, w.d) if kind == "shared" else (w.Hq, w.d, w.d)
    W = r.standard_normal(shape).astype(np.float32) / np.float32(np.sqrt(w.d))
    b = (0.1 * r.standard_normal(shape[:-1])).astype(np.float32)
    return torch.from_numpy(W), torch.from_numpy(b)


def kernel_source_digest(pass_name):
    path = os.path.join(ROOT, "block_sparse_linear_mean_amd", "csrc", KERNEL_SOURCES[pass_name])
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(pass_name, workload):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernel source.

    The summary file profiles/hbm_counters_<workload>.txt holds one line per pass
      TRAFFIC pass=<name> bytes_per_launch=<int> kernel_source_sha=<hex16>
    written from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE), calibrated with a copy kernel.
    """
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    m = re.search(rf"TRAFFIC pass={pass_name} bytes_per_launch=(\d+) kernel_source_sha=([0-9a-f]+)", open(path).read())
    if not m or m.group(2) != kernel_source_digest(pass_name):
        return None
    return int(m.group(1))


def host_cpu():
    """(cores this process may run on, CPU model name) of the host."""
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(cores), model


def cpu_baseline(w, q, k, v, wg, heads, proj_w=None, proj_b=None, smooth_k=False):
    """The CPU oracle as it stands, on whole heads of the same workload (and options), extrapolated
    to all heads."""
    import numpy as np
    from oracle import sla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                           or [1])
    except Exception:
        blas_threads = 1
    heads = max(1, min(heads, w.Hkv))
    G = w.Hq // w.Hkv
    Q = q[:, :heads * G].float().numpy()
    K = k[:, :heads].float().numpy()
    V = v[:, :heads].float().numpy()
    wgn = None if wg is None else wg[:heads * G].numpy()
    t0 = time.perf_counter()
    pw = pb = None
    if proj_w is not None:
        pw = proj_w.numpy() if proj_w.dim() == 2 else proj_w[:heads * G].numpy()
        pb = proj_b.numpy() if proj_b.dim() == 1 else proj_b[:heads * G].numpy()
    f = orc.Forward(Q, K, V, n_valid=w.Nv, mode=w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp, n_sel=w.n_sel,
                    window=w.window, w_gate=wgn, proj_w=pw, proj_b=pb, smooth_k=smooth_k)
    f.output()
    dt = time.perf_counter() - t0
    full = dt * (w.Hkv / heads)
    cores, model = host_cpu()
    return {
        "value": round(w.dense_flops() / full / 1e12, 6),
        "unit": "TFLOP/s (effective, dense-equivalent)",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": model,
        "blas_threads": int(blas_threads),
        "sample": (f"{heads} of {w.Hkv} KV heads ({heads * G} query heads), every query block, full forward "
                   f"in {dt:.1f} s, scaled x{w.Hkv / heads:g} to the whole layer ({full:.1f} s); "
                   f"float64 numpy oracle on {cores} host cores ({model}), its matrix products on "
                   f"{blas_threads} BLAS thread(s)"),
        "ms_per_layer": round(full * 1e3, 1),
    }


def captured_mass(w, qd, kd, vd):
    """Mean over valid query rows of the dense softmax mass that falls on the row's critical
    blocks, exp(lse_critical - lse_dense), with the tokens in row-major and in Hilbert order (the
    reordering remark of the pages: a more coherent block raises the mass a fixed budget captures).
    Both log-sum-exps come from the library's forward (the dense one with every block critical)."""
    import torch
    import block_sparse_linear_mean_amd as sla
    if w.mode != "sla" or getattr(w, "grid", None) is None:
        return None
    out = {}
    for name, order in (("row-major", None), ("hilbert", sla.sla_hilbert_order(*w.grid))):
        lay = sla.SlaForward(qd, kd, vd, w.Nv, "sla", kh_bp=w.kh_bp, kl_bp=w.kl_bp, training=True, token_order=order)
        lay.run()
        dense = sla.SlaForward(qd, kd, vd, w.Nv, "sla", kh_bp=10000, kl_bp=0, training=True, token_order=order)
        dense.run()
        mass = torch.exp(lay.lse[:, :, :w.Nv] - dense.lse[:, :, :w.Nv])
        out[name] = round(float(mass.mean()), 4)
        out[name + "_p10"] = round(float(torch.quantile(mass.flatten()[::97].float(), 0.1)), 4)
        del lay, dense
        torch.cuda.empty_cache()
        log(f"bench: captured dense mass ({name}) = {out[name]}")
    return out


def bench_nsa3(args, w, qd, kd, vd):
    """Time NSA with its three branches (compressed 32/16 tokens, 16 selected blocks, 512-token window,
    gated merge) on an NSA workload: pooled scores, the selection map and sla_nsa3_fwd per step."""
    import torch
    import block_sparse_linear_mean_amd as sla
    if w.mode != "nsa":
        raise SystemExit("--nsa-branches 3 needs an nsa workload")
    layer = sla.SlaForward(qd, kd, vd, w.Nv, "nsa", n_sel=w.n_sel, window=0)
    g = torch.Generator(device="cpu").manual_seed(11)
    wg = (torch.randn((3, w.Hq, w.d), generator=g) / w.d ** 0.5).to(qd.device)
    B, Hq, N, d = qd.shape
    ws = torch.empty(sla.sla_nsa3_workspace_bytes(B, Hq, w.Hkv, N, d, 0 if w.dtype == "bf16" else 1, w.Nv,
                                                  w.window, 32, 16), device=qd.device, dtype=torch.uint8)
    out = torch.empty_like(qd)
    steps = {"pool_scores": layer.pool_scores, "block_map": layer.block_map,
             "nsa3": lambda: sla.sla_nsa3_fwd(qd, kd, vd, w.Nv, layer.maps, wg, window=w.window, out=out, workspace=ws)}
    for _ in range(args.warmup):
        for fn in steps.values():
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        ev[s_][0].record()
        for i, fn in enumerate(steps.values()):
            fn()
            ev[s_][i + 1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    pass_ms = {name: sum(ev[s_][i].elapsed_time(ev[s_][i + 1]) for s_ in range(args.steps)) / args.steps
               for i, name in enumerate(steps)}
    log("bench: per-pass ms " + ", ".join(f"{k_}={v_:.4f}" for k_, v_ in pass_ms.items()) + f"; wall {ms_step:.4f}")
    print(json.dumps({
        "metric": "NSA (compressed + selected + window, gated) fwd ms/layer + effective TFLOP/s",
        "value": round(w.dense_flops() / (ms_step / 1e3) / 1e12, 3),
        "unit": "TFLOP/s (effective, dense-equivalent causal)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic (seeded)",
        "config": {"workload": w.name, "branches": 3, "cmp_block": 32, "cmp_stride": 16, "n_sel": w.n_sel,
                   "window": w.window},
        "passes": {k_: round(v_, 5) for k_, v_ in pass_ms.items()},
    }))


def backward_numbers(w, qd, kd, vd, steps, warmup):
    """One training forward, then `warmup` untimed and `steps` timed backward calls on a fixed seeded
    dO: wall and HIP-event ms per backward, executed FLOPs (as bench_backward states them), the
    critical pairs and the achieved TFLOP/s."""
    import torch
    import block_sparse_linear_mean_amd as sla
    from workloads import make_inputs
    wg = make_inputs(w)[3] if w.mode == "salad" else None
    layer = sla.SlaForward(qd, kd, vd, w.Nv, w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp, n_sel=w.n_sel,
                           window=w.window, w_gate=wg, training=True)
    layer.run()
    g = torch.Generator(device="cpu").manual_seed(7)
    dout = torch.randn(qd.shape, generator=g).to(device=qd.device, dtype=qd.dtype)
    grads = (torch.empty(qd.shape, device=qd.device, dtype=torch.float32),
             torch.empty(kd.shape, device=qd.device, dtype=torch.float32),
             torch.empty(kd.shape, device=qd.device, dtype=torch.float32))
    for _ in range(warmup):
        layer.backward(dout, grads=grads)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for s_ in range(steps):
        layer.backward(dout, grads=grads)
        ev[s_ + 1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    ms_gpu = ev[0].elapsed_time(ev[-1]) / steps
    entries = int(layer.maps["crit_rowptr"][-1].item())
    pairs = entries * (w.Hq // w.Hkv if layer.group else 1)
    d, nb, BH, BK = w.d, w.nb, w.B * w.Hq, w.B * w.Hkv
    flops = pairs * 7 * 2.0 * 64 * 64 * d
    if layer.lin != sla.SLA_LIN_NONE:
        flops += BH * nb * 3 * 2.0 * 64 * d * d + BK * nb * 2 * 2.0 * 64 * d * d
        flops += BH * 2.0 * (nb if layer.lin == sla.SLA_LIN_MARGINAL else 1) * nb * d * d
    achieved = flops / (ms_gpu / 1e3) / 1e12
    return dict(ms_per_step=ms_step, gpu_ms=ms_gpu, flops=flops, pairs=pairs, achieved=achieved)


def other_workloads(dev, steps, warmup):
    """The layer forward of the salad and nsa_prefill workloads and the backward of wan13b_sla, each
    on its own seeded inputs in this process (wall ms per step over `steps` after `warmup`), so that
    the default run times them beside the headline."""
    import torch
    import block_sparse_linear_mean_amd as sla
    from workloads import WORKLOADS, make_inputs
    out = {}
    for name in ("salad", "nsa_prefill"):
        w = WORKLOADS[name]
        log(f"bench: other workload {name}: inputs")
        q, k, v, wg = make_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        layer = sla.SlaForward(qd, kd, vd, w.Nv, w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp, n_sel=w.n_sel,
                               window=w.window, w_gate=None if wg is None else wg.to(dev))
        for _ in range(warmup):
            layer.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            layer.run()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        out[name] = {"pass": "forward", "ms_per_step": round(ms, 5),
                     "value": round(w.dense_flops() / (ms / 1e3) / 1e12, 3),
                     "unit": "TFLOP/s (effective, dense-equivalent)", "metric": metric_for(w)}
        log(f"bench: {name} forward {ms:.4f} ms/layer")
        del layer, qd, kd, vd
        torch.cuda.empty_cache()
    w = WORKLOADS["wan13b_sla"]
    log("bench: other workload wan13b_sla backward: inputs")
    q, k, v, _ = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    r = backward_numbers(w, qd, kd, vd, steps, warmup)
    out["wan13b_sla_backward"] = {"pass": "backward (dQ, dK, dV)", "ms_per_step": round(r["ms_per_step"], 5),
                                  "gpu_ms": round(r["gpu_ms"], 5), "executed_flops": r["flops"],
                                  "mfma_frac": round(r["achieved"] / PEAK_BF16_TFLOPS, 4)}
    log(f"bench: wan13b_sla backward {r['ms_per_step']:.4f} ms/layer")
    del qd, kd, vd
    torch.cuda.empty_cache()
    out["note"] = f"{warmup} warm-up and {steps} timed steps each, wall clock, after the headline's timed region"
    return out


def bench_backward(args, w, qd, kd, vd):
    """Time the backward (dQ, dK, dV, and dw_gate for SALAD, of one layer for its block map) and
    print one JSON line.

    The forward runs once in training mode (it also keeps each row's log-sum-exp); each timed step
    is one backward call on a fixed seeded dO.  Executed FLOPs: per critical (query head, key block)
    pair the seven 64 x 64 x d products of the sparse backward (S and dP in both the dQ and the
    dK/dV kernels, dQ, dK, dV); with a linear branch, per query block the three 64 x d x d products
    of the query side and per key block the two of the key side, plus the transposed mask product
    over the state gradients (2 nb^2 d^2 per head; gated: 2 nb d^2, one row per head).
    """
    r = backward_numbers(w, qd, kd, vd, args.steps, args.warmup)
    ms_step, ms_gpu, flops, pairs, achieved = r["ms_per_step"], r["gpu_ms"], r["flops"], r["pairs"], r["achieved"]
    dense = 2.5 * w.dense_flops()          # dense-equivalent backward: 2.5x the forward's products
    log(f"bench: backward {ms_gpu:.4f} ms/layer (HIP events), wall {ms_step:.4f}; executed {flops / 1e9:.1f} GFLOP")
    print(json.dumps({
        "metric": metric_for(w).replace(" fwd ", " bwd ").replace("effective TFLOP/s", "effective TFLOP/s (dQ, dK, dV)"),
        "value": round(dense / (ms_step / 1e3) / 1e12, 3),
        "unit": "TFLOP/s (effective, dense-equivalent backward = 2.5x forward)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded)", "config": {"workload": w.name, "pass": "backward", "critical_pairs": pairs},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "sla_attn_bwd_ext (all kernels)", "algorithmic_per_launch": flops,
                     "avg_launch_ms": round(ms_gpu, 5)},
    }))


# ----------------------------------------------------------------------------- profile summaries
# Text summaries of rocprofv3 output (run on the host after a profiled run; no GPU needed).

def _read_csv(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def _short(name, n=70):
    return name if len(name) <= n else name[:n - 3] + "..."


def summarize_trace(directory, command, note):
    """Per-kernel call count and durations (us) from a --kernel-trace run's *kernel_trace.csv."""
    rows = _read_csv(directory, "kernel_trace.csv")
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"# rocprofv3 kernel trace summary: {note}", f"# command: {command}",
           "# durations in microseconds, one row per kernel, from the run's kernel_trace.csv",
           f"{'kernel':72s} {'calls':>6s} {'total_us':>11s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{_short(name, 72):72s} {len(d):6d} {sum(d):11.1f} {sum(d) / len(d):9.2f} "
                   f"{min(d):9.2f} {max(d):9.2f}")
    return "\n".join(out) + "\n"


def summarize_counters(fetch_dir, write_dir, workload, copy_mib, commands, passes=None):
    """HBM traffic per launch of each pass's kernel from FETCH_SIZE and WRITE_SIZE runs (KiB per
    dispatch), each scaled by the ratio of known to counted bytes of an elementwise copy of copy_mib MiB.
    One TRAFFIC line per pass whose kernel appears in both runs."""
    import statistics

    def per_kernel(directory, counter):
        vals = {}
        for r in _read_csv(directory, "counter_collection.csv"):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)

    def pick(vals, match):
        names = [n for n in vals if match(n)]
        return (names[0], statistics.median(vals[names[0]])) if names else (None, None)

    is_copy = lambda n: "MulFunctor" in n or ("elementwise" in n and "mul" in n.lower())
    ck_f, copy_f = pick(fetch, is_copy)
    ck_w, copy_w = pick(write, is_copy)
    if ck_f is None or ck_w is None:
        raise SystemExit("no calibration copy kernel in the counter runs (run with --copy-calibration-mb)")
    fac_f, fac_w = copy_bytes / copy_f, copy_bytes / copy_w
    out = [f"# HBM traffic per launch of each pass's kernel, workload {workload}",
           f"# fetch run: {commands[0]}", f"# write run: {commands[1]}",
           f"# calibration kernel: {_short(ck_f, 60)}, {copy_mib} MiB read + {copy_mib} MiB written per launch",
           f"copy   FETCH_SIZE {copy_f:.0f} B counted / {copy_bytes} B known -> factor {fac_f:.4f}",
           f"copy   WRITE_SIZE {copy_w:.0f} B counted / {copy_bytes} B known -> factor {fac_w:.4f}"]
    for pass_name in passes or PASSES:
        key = PASS_KERNEL[pass_name]
        kn, kf = pick(fetch, lambda n: key in n)
        _, kw = pick(write, lambda n: key in n)
        if kn is None or kw is None:
            continue
        traffic = int(round(kf * fac_f + kw * fac_w))
        out += [f"{pass_name}: {_short(kn, 70)}",
                f"  FETCH_SIZE median {kf:.0f} B/launch (scaled {kf * fac_f:.0f}); "
                f"WRITE_SIZE median {kw:.0f} B/launch (scaled {kw * fac_w:.0f})",
                f"TRAFFIC pass={pass_name} bytes_per_launch={traffic} kernel_source_sha={kernel_source_digest(pass_name)}"]
    return "\n".join(out) + "\n"


def cold_steps(layer, args, dev):
    """Layer time with the caches cold: before each step a 512 MiB scratch write evicts L2 and
    MALL (256 MB), so the inputs come from HBM.  Median over the steps (HIP events)."""
    import torch
    scratch = torch.empty(512 << 20, device=dev, dtype=torch.uint8)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    ev_att = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s_ in range(args.steps):
        scratch.fill_(s_ & 255)
        ev[s_][0].record()
        layer.run(events={"attention": ev_att[s_]})
        ev[s_][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    att = sorted(a.elapsed_time(b) for a, b in ev_att)
    del scratch
    return {"ms_per_step_median": round(ms[len(ms) // 2], 5), "attention_ms_median": round(att[len(att) // 2], 5),
            "flush": "512 MiB scratch write before each step"}


def achievable_peaks(dev, attention_ms, attention_flops):
    """Context for the roofline fractions, measured in the same process: a device copy of 1 GiB
    (read + write), a large bf16 GEMM (8192^3, the vendor library) and the vendor's dense
    FlashAttention at B1 H12 N8192 d128, with the attention pass's rate as a fraction of each."""
    import torch
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    n = 1 << 28
    src = torch.ones(n, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src), 10)
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    gemm_ms = timed(lambda: torch.matmul(a, b), 10)
    del a, b
    gemm_tf = 2 * m ** 3 / (gemm_ms / 1e3) / 1e12
    att_tf = attention_flops / (attention_ms / 1e3) / 1e12
    res = {"copy_GBps": round(2 * n * 4 / (copy_ms / 1e3) / 1e9, 1), "gemm_bf16_TFLOPs": round(gemm_tf, 1),
           "gemm_shape": [m, m, m], "attention_frac_of_gemm": round(att_tf / gemm_tf, 4)}
    # the vendor's dense FlashAttention (torch SDPA, flash backend only) at B1 H12 N8192 d128 bf16
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        g = torch.Generator(device=dev).manual_seed(0)
        q, k, v = (torch.randn(1, 12, 8192, 128, device=dev, dtype=torch.bfloat16, generator=g) for _ in range(3))
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            sdpa_ms = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v), 10)
        sdpa_tf = 4.0 * 12 * 8192 ** 2 * 128 / (sdpa_ms / 1e3) / 1e12
        res.update({"sdpa_flash_dense_TFLOPs": round(sdpa_tf, 1), "sdpa_shape": [1, 12, 8192, 128],
                    "attention_frac_of_sdpa": round(att_tf / sdpa_tf, 4)})
        del q, k, v
    except (RuntimeError, ImportError) as e:
        res["sdpa_flash_dense_TFLOPs"] = None
        log(f"bench: no flash SDPA for the context line ({e})")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan13b_sla")
    ap.add_argument("--cpu-sample-heads", type=int, default=12)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip timing the salad and nsa_prefill forwards and the wan13b_sla backward")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the cold-cache steps and the copy / GEMM reference measurements")
    ap.add_argument("--backward", action="store_true", help="time the layer backward instead")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one HIP graph of the layer (one host launch per step)")
    ap.add_argument("--overlap", action="store_true",
                    help="run the key states and marginal sums on a second stream, overlapping scores and map")
    ap.add_argument("--token-order", choices=["row-major", "hilbert"], default="row-major",
                    help="run the layer on Q, K, V gathered along a 3-D Hilbert curve of the latent grid")
    ap.add_argument("--proj", choices=["none", "shared", "per-head"], default="none",
                    help="SLA only: the learned projection of the linear branch (seeded random weights and bias)")
    ap.add_argument("--smooth-k", action="store_true", help="SLA/SALAD: keys of the linear branch centred by their mean")
    ap.add_argument("--nsa-branches", type=int, choices=[2, 3], default=2,
                    help="3: time NSA with its compressed branch and gated merge (nsa workloads)")
    ap.add_argument("--captured-mass", action="store_true",
                    help="also report the dense attention mass the critical blocks capture (row-major and Hilbert)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (calibrates HBM byte counters)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="print a kernel-trace summary of a rocprofv3 run")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the HBM-traffic summary of every pass's kernel from two rocprofv3 --pmc runs")
    ap.add_argument("--command", action="append", default=[], help="profiling command(s) to record")
    ap.add_argument("--note", default="")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, (args.command or ["?"])[0], args.note), end="")
        return
    if args.summarize_counters:
        cmds = (args.command + ["?", "?"])[:2]
        print(summarize_counters(*args.summarize_counters, args.workload, args.copy_calibration_mb, cmds), end="")
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU only: the library has no multi-GPU path "
               f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).")
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        log(msg)
        sys.exit(2)

    import torch
    import block_sparse_linear_mean_amd as sla
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    log(f"bench: generating {w.name} inputs")
    q, k, v, wg = make_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if args.backward:
        bench_backward(args, w, qd, kd, vd)
        return
    if args.nsa_branches == 3:
        bench_nsa3(args, w, qd, kd, vd)
        return
    order = None
    if args.token_order == "hilbert":
        if getattr(w, "grid", None) is None:
            raise SystemExit("--token-order hilbert needs a workload with a latent grid")
        order = sla.sla_hilbert_order(*w.grid)
    proj_w = proj_b = None
    if args.proj != "none":
        if w.mode != "sla":
            raise SystemExit("--proj applies to the SLA workloads")
        proj_w, proj_b = proj_weights(w, args.proj)
    if args.smooth_k and w.mode == "nsa":
        raise SystemExit("--smooth-k applies to a linear branch (SLA, SALAD)")
    layer = sla.SlaForward(qd, kd, vd, w.Nv, w.mode, kh_bp=w.kh_bp, kl_bp=w.kl_bp, n_sel=w.n_sel,
                           window=w.window, w_gate=wg, token_order=order,
                           proj_w=None if proj_w is None else proj_w.to(dev),
                           proj_b=None if proj_b is None else proj_b.to(dev), smooth_k=args.smooth_k)
    passes_run = (["reorder"] if order is not None else []) + PASSES + (["restore"] if order is not None else [])
    log(f"bench: {args.warmup} warm-up steps")
    for _ in range(args.warmup):
        layer.run(overlap=args.overlap)
    torch.cuda.synchronize()

    mk = lambda: {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in passes_run}

    def instrumented(n_steps):
        """n_steps layer steps with an event pair around every pass (on the stream it runs on) and
        around every step: (mean ms per pass, mean ms per step, per-step ms)."""
        ev = [mk() for _ in range(n_steps)]
        ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
        for s_ in range(n_steps):
            ev_step[s_][0].record()
            layer.run(overlap=args.overlap, events=ev[s_])
            ev_step[s_][1].record()
        torch.cuda.synchronize()
        per_pass = {name: sum(ev[s_][name][0].elapsed_time(ev[s_][name][1]) for s_ in range(n_steps)) / n_steps
                    for name in passes_run}
        per_step = [a.elapsed_time(b) for a, b in ev_step]
        return per_pass, sum(per_step) / n_steps, per_step

    # the dominant pass, from a short instrumented run before the timed region
    pre_ms, _, _ = instrumented(min(args.steps, 5))
    dom = max(PASSES, key=lambda n: pre_ms[n])
    # timed region: the plain layer, with one event pair around the dominant pass only (its launch
    # duration for the roofline, measured live; a pair around every pass costs ~0.04 ms per layer)
    ev_dom = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    graph = layer.capture() if args.graph else None
    log(f"bench: {args.steps} timed steps" + (" (replays of one HIP graph of the layer)" if graph else ""))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            layer.run(overlap=args.overlap, events={dom: ev_dom[s]})
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # with a graph the dominant pass's launch time comes from the instrumented run before it
    dom_ms = pre_ms[dom] if graph is not None else sum(a.elapsed_time(b) for a, b in ev_dom) / args.steps
    # per-pass breakdown: a separate instrumented run of as many steps, after the timed region
    pass_ms, step_gpu_ms, per_step = instrumented(args.steps)
    gpu_ms = step_gpu_ms
    log("bench: per-pass ms (instrumented run) " + ", ".join(f"{k_}={v_:.4f}" for k_, v_ in pass_ms.items()) +
        f"; step {step_gpu_ms:.4f} (events); timed region: wall {ms_step:.4f} ms/step, {dom} {dom_ms:.4f} ms")

    work, pairs = pass_work(w, layer)
    bound, amount = work[dom]
    t_dom = dom_ms / 1e3
    if bound == "hbm":
        achieved = amount / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        achieved = amount / t_dom / 1e12
        roof = {"bound": bound, "achieved": round(achieved, 3), "peak": PEAKS[bound], "unit": "TFLOP/s"}
    roof["frac"] = round(achieved / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom, w.name)
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = amount
    roof["avg_launch_ms"] = round(dom_ms, 5)

    if order is not None:
        # a row gather of Q, K, V and a row scatter of O: 2 * bytes of each tensor
        eb = 2 if w.dtype == "bf16" else 4
        work["reorder"] = ("hbm", 3 * 2 * w.B * w.Hq * w.N * w.d * eb)
        work["restore"] = ("hbm", 2 * w.B * w.Hq * w.N * w.d * eb)
    passes = {}
    for name in passes_run:
        b_, a_ = work[name]
        t_ = pass_ms[name] / 1e3
        if a_ and t_ > 0:
            frac = (a_ / t_ / 1e9 / PEAK_HBM_GBS) if b_ == "hbm" else (a_ / t_ / 1e12 / PEAKS[b_])
        else:
            frac = None
        passes[name] = {"ms": round(pass_ms[name], 5), "bound": b_,
                        "roofline_frac": None if frac is None else round(frac, 4)}
        if name in PASS_KERNEL and a_:
            passes[name]["algorithmic_per_launch"] = a_
            passes[name]["traffic"] = measured_traffic(name, w.name)
    if "marginal_states" in passes and layer.lin == 1 and pass_ms["marginal_states"] > 0:
        # the 0/1-mask product: matrix-core FLOPs (2 nb^2 d^2 per head, the dense mask) and HBM bytes
        t_ = pass_ms["marginal_states"] / 1e3
        heads = w.B * (w.Hkv if layer.group else w.Hq)
        mflops = 2.0 * heads * w.nb * w.nb * (w.d * w.d + w.d)
        passes["marginal_states"]["mfma_frac"] = round(mflops / t_ / 1e12 / PEAK_BF16_TFLOPS, 4)
        passes["marginal_states"]["hbm_frac"] = passes["marginal_states"]["roofline_frac"]
        passes["marginal_states"]["mask_product_flops"] = mflops
    if "scores" in passes and pass_ms["scores"] > 0:
        # the pooled scores also write nb^2 fp32 per map row
        rows = w.B * (w.Hkv if layer.group else w.Hq) * w.nb
        passes["scores"]["hbm_frac"] = round(rows * w.nb * 4 / (pass_ms["scores"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)

    value = w.dense_flops() / (ms_step / 1e3) / 1e12
    cfg = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "n_valid": w.Nv, "d": w.d,
           "block": 64, "mode": w.mode, "causal": w.causal}
    if w.mode == "sla":
        cfg.update(kh_pct=w.kh_bp / 100, kl_pct=w.kl_bp / 100, n_crit=layer.n_crit, n_negl=layer.n_negl)
    elif w.mode == "salad":
        cfg.update(kh_pct=w.kh_bp / 100, n_crit=layer.n_crit, linear="all keys, gated")
    else:
        cfg.update(n_sel=w.n_sel, window=w.window)
    cfg["critical_pairs"] = pairs
    if order is not None:
        cfg["token_order"] = "hilbert"
    metric = metric_for(w)
    if args.proj != "none":
        cfg["proj"] = args.proj
        metric += f", + Proj ({args.proj})"
    if args.smooth_k:
        cfg["smooth_k"] = True
        metric += ", smooth-K"
    if args.graph:
        cfg["hip_graph"] = True
    result = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s (effective, dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Wan2.1-shaped Fourier-feature Q/K, Gaussian V)" if w.generator == "video"
        else "synthetic (seeded)",
        "config": cfg,
        "roofline": roof,
        "passes": passes,
        "gpu_ms_per_step": round(gpu_ms, 5),
    }
    per_step = sorted(per_step)
    result["gpu_ms_per_step_median"] = round(per_step[len(per_step) // 2], 5)
    result["gpu_ms_per_step_min"] = round(per_step[0], 5)
    result["passes_note"] = ("passes and gpu_ms_per_step*: a separate run of as many steps with an event pair "
                             "around every pass and step, after the timed region")
    if not args.no_context:
        result["cold"] = cold_steps(layer, args, dev)
        result["achievable"] = achievable_peaks(dev, pass_ms["attention"], work["attention"][1])
    if (not args.no_others and w.name == "wan13b_sla" and order is None and args.proj == "none"
            and not args.smooth_k and not args.graph and not args.overlap):
        result["other_workloads"] = other_workloads(dev, 10, 3)
    if args.captured_mass:
        result["captured_mass"] = captured_mass(w, qd, kd, vd)
    if args.copy_calibration_mb:
        # an elementwise kernel that reads and writes exactly n * 4 bytes each (a plain DtoD copy
        # may go to a blit path that the counters do not see)
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"bench: copy calibration, 3 elementwise copies of {args.copy_calibration_mb} MiB")
    if not args.no_cpu_baseline:
        log(f"bench: cpu baseline (oracle) on {args.cpu_sample_heads} head(s)")
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, wg, args.cpu_sample_heads, proj_w, proj_b, args.smooth_k)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
