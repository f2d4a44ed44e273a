#!/usr/bin/env python3
"""Benchmark: exact attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one pass of the whole hot path over one batch: fa_fwd, then the three
backward kernels (fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq), on synthetic seeded
inputs already resident in HBM. The default workload is the Llama-shaped causal case
(B=4, H=32, N=4096, d=128, bf16). Prints one JSON line.

FLOP model (algorithmic work, not what the kernels happen to execute): one "GEMM
unit" is 2*B*H*N^2*d, halved under causal masking. Forward = 2 units (QK^T, PV);
backward = 5 units (recomputed QK^T, dO V^T, P^T dO, dS^T Q, dS K), i.e. 2.5x the
forward. Per kernel: fwd 2 units, dkdv 4, dq 1 (its recomputation of S and dP is the
price of a dQ pass without atomics and is not counted), preprocess 0.

The CPU baseline times the fp64 oracle on a bounded sample of the same workload
(whole heads, forward + backward), on the host cores, and reports the same FLOP
model per second.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s, bf16 d=128 N=4096 causal; % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA, published (twice bf16)
CSRC = os.path.join(ROOT, "exact_io_aware_attention_amd", "csrc")

# HBM traffic per launch of a kernel, from two rocprofv3 --pmc passes over this script
# (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) on the named workload, each scaled by
# the ratio that the same counter shows for a copy kernel of known size run in the same
# process (--calibrate-copy-mib). Reported only while the kernel sources still hash to
# the value they had when the counters were taken; otherwise null.
TRAFFIC = {
    ("c3", "fwd"): {"bytes": 724759552, "fetch_kib": 287332.9, "write_kib": 133120.0,
                  "fetch_factor": 2.0, "write_factor": 1.0,
                  "sources_sha256": "864d63ae2d056263a4906f8659a463a4b0d4130391f1d42b2dfc0f7678990e44",
                  "profile": "profiles/attention_fwd_bwd_c3.md"},
    ("c3", "bwd_preprocess"): {"bytes": 274770234, "fetch_kib": 132120.1, "write_kib": 4096.0,
                  "fetch_factor": 2.0, "write_factor": 1.0,
                  "sources_sha256": "864d63ae2d056263a4906f8659a463a4b0d4130391f1d42b2dfc0f7678990e44",
                  "profile": "profiles/attention_fwd_bwd_c3.md"},
    ("c3", "bwd_dkdv"): {"bytes": 964896062, "fetch_kib": 340076.2, "write_kib": 262144.0,
                  "fetch_factor": 2.0, "write_factor": 1.0,
                  "sources_sha256": "864d63ae2d056263a4906f8659a463a4b0d4130391f1d42b2dfc0f7678990e44",
                  "profile": "profiles/attention_fwd_bwd_c3.md"},
    ("c3", "bwd_dq"): {"bytes": 898215941, "fetch_kib": 373054.3, "write_kib": 131072.0,
                  "fetch_factor": 2.0, "write_factor": 1.0,
                  "sources_sha256": "864d63ae2d056263a4906f8659a463a4b0d4130391f1d42b2dfc0f7678990e44",
                  "profile": "profiles/attention_fwd_bwd_c3.md"},
}


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def traffic_for(workload: str, kernel: str):
    t = TRAFFIC.get((workload, kernel))
    if t is None or t["sources_sha256"] != sources_sha256():
        return None
    return t


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_unit(B, H, N, d, causal, lengths=None):
    if lengths is not None:
        return sum(2.0 * H * L * L * d * (0.5 if causal else 1.0) for L in lengths)
    return 2.0 * B * H * N * N * d * (0.5 if causal else 1.0)


def standard_attention(q, k, v, do, scale: float, causal: bool, reps: int = 3):
    """Standard (materialising) attention on the same GPU, for comparison: S = scale Q K^T
    and P = softmax(S) are written to HBM as full N x N matrices (bf16 GEMMs with fp32
    accumulation via torch.matmul, softmax in fp32), and the backward is the textbook
    chain rule on those stored matrices. Every matmul gets contiguous operands. Returns
    fwd/bwd times (median of `reps`, HIP events on the current stream), the peak device
    memory the two passes allocate, and O for a sanity check."""
    import torch
    B, N, H, d = q.shape
    qh, kh, vh, doh = (t.permute(0, 2, 1, 3).contiguous() for t in (q, k, v, do))  # (B, H, N, d)
    kt = kh.transpose(-1, -2).contiguous()
    vt = vh.transpose(-1, -2).contiguous()
    mask = torch.ones(N, N, device=q.device, dtype=torch.bool).triu_(1) if causal else None

    def fwd():
        s = torch.matmul(qh, kt).float().mul_(scale)
        if mask is not None:
            s.masked_fill_(mask, float("-inf"))
        p = torch.softmax(s, dim=-1).to(q.dtype)
        del s
        return p, torch.matmul(p, vh)

    def bwd(p, o):
        dv = torch.matmul(p.transpose(-1, -2).contiguous(), doh)
        dp = torch.matmul(doh, vt).float()
        dd = (doh.float() * o.float()).sum(-1, keepdim=True)
        ds = (p.float() * (dp - dd)).to(q.dtype)
        del dp
        dq = torch.matmul(ds, kh).float().mul_(scale)
        dk = torch.matmul(ds.transpose(-1, -2).contiguous(), qh).float().mul_(scale)
        return dq, dk, dv

    stream = torch.cuda.current_stream()
    tf, tb = [], []
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o = None
    for _ in range(reps + 1):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        p, o = fwd()
        e1.record(stream)
        grads = bwd(p, o)
        e2.record(stream)
        torch.cuda.synchronize()
        tf.append(e0.elapsed_time(e1))
        tb.append(e1.elapsed_time(e2))
        del p, grads
    peak = torch.cuda.max_memory_allocated() - base
    med = lambda x: sorted(x[1:])[len(x[1:]) // 2]
    return {"fwd_ms": med(tf), "bwd_ms": med(tb), "peak_extra_bytes": int(peak)}, o.permute(0, 2, 1, 3)


def decode_bench(reps: int = 20):
    """fa_fwd_decode on the decode workloads: median time of `reps` calls (HIP events on
    the launch stream) and the achieved rate of the algorithmic bytes (K and V read
    once, Q read, O and LSE written) against the HBM peak."""
    import torch
    import exact_io_aware_attention_amd as fa
    import workloads as W
    res = {}
    for name, w in sorted(W.DECODE_WORKLOADS.items()):
        q, k, v = (t.cuda() for t in W.make_decode_inputs(w))
        B, Nq, H, d = q.shape
        Nk = k.shape[1]
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
        ws_bytes = fa.fa_fwd_decode_workspace_bytes(B, H, Nq, Nk, d, 0)
        ws = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
        sp = torch.cuda.current_stream().cuda_stream

        def call():
            st = fa.fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                                  Nk, d, w.scale, int(w.causal), 0, ws.data_ptr(), ws_bytes, fa.FA_DTYPE_BF16, sp)
            if st != fa.FA_OK:
                raise fa.FAError(st, "fa_fwd_decode")

        for _ in range(3):
            call()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        algo = 2 * B * Nk * H * d * 2 + 2 * B * Nq * H * d * 2 + B * H * Nq * 4
        gbs = algo / (ms * 1e-3) / 1e9
        res[name] = {"workload": w.description, "batch": B, "heads": H, "seqlen_q": Nq, "seqlen_k": Nk,
                     "head_dim": d, "causal": w.causal, "ms": round(ms, 4), "algorithmic_bytes": algo,
                     "achieved_gbs": round(gbs, 1), "hbm_peak_gbs": PEAK_HBM_GBS,
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "bound": "hbm"}
        del q, k, v, o, lse, ws
    return res


def fp8_bench(reps: int = 20):
    """fa_fwd_fp8 on the 8-bit workloads: median time of `reps` calls (HIP events on the
    launch stream) and the forward's algorithmic FLOPs (2 GEMM units, halved under causal)
    per second against the fp8 MFMA peak."""
    import torch
    import exact_io_aware_attention_amd as fa
    import workloads as W
    res = {}
    for name, w in sorted(W.FP8_WORKLOADS.items()):
        q8, k8, v8 = (t.cuda() for t in W.make_fp8_inputs(w))
        B, N, H, d = q8.shape
        o = torch.empty((B, N, H, d), device=q8.device, dtype=torch.bfloat16)
        lse = torch.empty((B, H, N), device=q8.device, dtype=torch.float32)
        sp = torch.cuda.current_stream().cuda_stream

        def call():
            st = fa.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                               w.scale, w.descale_q, w.descale_k, w.descale_v, int(w.causal), sp)
            if st != fa.FA_OK:
                raise fa.FAError(st, "fa_fwd_fp8")

        for _ in range(3):
            call()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        flops = 2 * (2.0 * B * H * N * N * d) * (0.5 if w.causal else 1.0)
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"workload": w.description, "batch": B, "heads": H, "seqlen": N, "head_dim": d,
                     "causal": w.causal, "ms": round(ms, 4), "tflops": round(tf, 2), "bound": "mfma",
                     "peak_tflops": PEAK_FP8_TFLOPS, "frac_of_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        del q8, k8, v8, o, lse
    return res


def cpu_baseline(inp, w, budget_s: float):
    """Time the oracle (fp64, NumPy) on whole heads of the workload until ~budget_s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = len(os.sched_getaffinity(0))
    B, H = inp.q.shape[0], inp.q.shape[2]
    heads = [(b, h) for b in range(B) for h in range(H)]
    flops = 0.0
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        q, k, v, do = (oracle.to_f64(t[b, :, h, :]) for t in (inp.q, inp.k, inp.v, inp.do))
        oracle.head_forward(q, k, v, w.scale, w.causal)
        oracle.head_backward(q, k, v, do, w.scale, w.causal)
        N, d = q.shape
        flops += 7 * gemm_unit(1, 1, N, d, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (batch, head) pairs of {w.name}, fp64 forward + backward "
                  f"(oracle materialises the full N x N scores), {dt:.1f} s wall",
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work (0: skip)")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch (not varlen)")
    ap.add_argument("--seqlen", type=int, default=None, help="override the workload's sequence length (not varlen)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurements")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit forward measurement")
    ap.add_argument("--no-standard", action="store_true",
                    help="skip the standard-attention comparison (materialised N x N scores)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the warmup, run a plain fp32 copy kernel (y = -x) over this many MiB, "
                         "three times, as the known-size reference for HBM byte counters")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): every (sequence, head) pair is "
              "independent, so more GPUs would each run these kernels on their share of the heads; no "
              "cross-GPU path is implemented", file=sys.stderr)
        return 2

    import torch
    import exact_io_aware_attention_amd as fa
    import workloads as W

    fa.load_library()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    w = W.get(a.workload)
    log(f"bench: generating {w.name} inputs")
    if (a.batch is not None or a.seqlen is not None) and w.varlen:
        print("--batch/--seqlen apply to fixed-length workloads only", file=sys.stderr)
        return 2
    inp = W.make_inputs(w, batch=a.batch, seqlen=a.seqlen)
    resized = a.batch is not None or a.seqlen is not None
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (inp.q, inp.k, inp.v, inp.do))
    cu = inp.cu_seqlens.to(dev) if inp.cu_seqlens is not None else None
    B, N, H, d, T = inp.batch, inp.seqlen, w.heads, w.head_dim, inp.total_tokens
    dt_code = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_FP32
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N) if cu is None else (H, T), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_bytes(B, H, N, d, int(cu is not None), T)
    ws = torch.empty(ws_bytes, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    cup = cu.data_ptr() if cu is not None else None
    causal = int(w.causal)

    def check(st, name):
        if st != fa.FA_OK:
            raise fa.FAError(st, name)

    def k_fwd():
        check(fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                        w.scale, causal, cup, T, dt_code, sp), "fa_fwd")

    def k_pre():
        check(fa.fa_bwd_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws_bytes, B, H, N,
                                   d, w.scale, cup, T, dt_code, sp), "fa_bwd_preprocess")

    def k_dkdv():
        check(fa.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             ws.data_ptr(), ws_bytes, dk.data_ptr(), dv.data_ptr(), B, H, N, d, w.scale,
                             causal, cup, T, dt_code, sp), "fa_bwd_dkdv")

    def k_dq():
        check(fa.fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                           ws.data_ptr(), ws_bytes, dq.data_ptr(), B, H, N, d, w.scale, causal, cup, T,
                           dt_code, sp), "fa_bwd_dq")

    kernels = [("fwd", k_fwd), ("bwd_preprocess", k_pre), ("bwd_dkdv", k_dkdv), ("bwd_dq", k_dq)]
    if a.calibrate_copy_mib > 0:
        n = a.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # reads and writes calibrate_copy_mib MiB each
        torch.cuda.synchronize()
        log(f"bench: copy calibration, {a.calibrate_copy_mib} MiB read + {a.calibrate_copy_mib} MiB written "
            f"per launch, 3 launches")
        del src, dst
    log(f"bench: warmup {a.warmup}")
    for _ in range(a.warmup):
        for _, fn in kernels:
            fn()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(a.steps)]
    log(f"bench: timing {a.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        ev[s][0].record(stream)
        for i, (_, fn) in enumerate(kernels):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(a.steps)) / a.steps
           for i, (name, _) in enumerate(kernels)}
    step_ms = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(a.steps)) / a.steps
    log("bench: per-kernel ms " + json.dumps({k_: round(v_, 4) for k_, v_ in per.items()}))

    unit = gemm_unit(B, H, N, d, w.causal, inp.lengths)
    fwd_fl, bwd_fl = 2 * unit, 5 * unit
    algo = {"fwd": 2 * unit, "bwd_preprocess": 0.0, "bwd_dkdv": 4 * unit, "bwd_dq": 1 * unit}
    bwd_ms = per["bwd_preprocess"] + per["bwd_dkdv"] + per["bwd_dq"]
    value = (fwd_fl + bwd_fl) / (step_ms * 1e-3) / 1e12
    dom = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda n: per[n])
    achieved = algo[dom] / (per[dom] * 1e-3) / 1e12
    tr = None if resized else traffic_for(w.name, dom)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid normal inputs)",
        "config": {
            "workload": f"{w.name}: {w.description}" + (" (resized)" if resized else ""),
            "batch": B, "heads": H, "seq_len": N, "head_dim": d, "causal": bool(w.causal),
            "global_batch": B, "parallelism": "single GPU",
        },
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(per["fwd"], 4), "tflops": round(fwd_fl / (per["fwd"] * 1e-3) / 1e12, 2),
                "frac_of_peak": round(fwd_fl / (per["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_fl / (bwd_ms * 1e-3) / 1e12, 2),
                "frac_of_peak": round(bwd_fl / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in per.items()},
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if tr is None else tr["bytes"],
        },
    }
    if tr is not None:
        out["roofline"]["traffic_detail"] = {
            "hbm_bytes_per_launch": tr["bytes"], "fetch_kib": tr["fetch_kib"], "write_kib": tr["write_kib"],
            "fetch_factor": tr["fetch_factor"], "write_factor": tr["write_factor"],
            "achieved_hbm_gbs": round(tr["bytes"] / (per[dom] * 1e-3) / 1e9, 1),
            "profile": tr["profile"]}
    need = 3 * B * H * N * N * 4  # fp32 scores + bf16 copies, roughly
    total_mem = torch.cuda.get_device_properties(0).total_memory
    if not a.no_standard and w.varlen is False and w.dtype == "bf16" and need > total_mem // 2:
        out["standard_attention"] = {"skipped": f"needs about {need / 2**30:.0f} GiB for the N x N matrices "
                                                f"(device: {total_mem / 2**30:.0f} GiB)"}
    elif not a.no_standard and w.varlen is False and w.dtype == "bf16":
        # The same step with standard attention; its memory is what this library avoids.
        log("bench: standard attention (materialised scores) for comparison")
        st, o_std = standard_attention(q, k, v, do, w.scale, bool(w.causal))
        ours_fwd, ours_bwd = per["fwd"], bwd_ms
        out["standard_attention"] = {
            "fwd_ms": round(st["fwd_ms"], 4), "bwd_ms": round(st["bwd_ms"], 4),
            "speedup_fwd": round(st["fwd_ms"] / ours_fwd, 2), "speedup_bwd": round(st["bwd_ms"] / ours_bwd, 2),
            "peak_extra_gib": round(st["peak_extra_bytes"] / 2**30, 2),
            "ours_workspace_gib": round(ws_bytes / 2**30, 4),
            "o_max_abs_diff": round(float((o_std.float() - o.float()).abs().max()), 4),
        }
        del o_std
        torch.cuda.empty_cache()
    if not a.no_decode:
        log("bench: decode workloads")
        out["decode"] = decode_bench()
    if not a.no_fp8:
        log("bench: 8-bit forward")
        out["fp8_forward"] = fp8_bench()
    if a.cpu_budget > 0 and w.varlen is False:
        log(f"bench: CPU oracle baseline (~{a.cpu_budget:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(inp, w, a.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
