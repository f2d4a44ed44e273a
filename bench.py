#!/usr/bin/env python3
"""Benchmark: exact attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

A step is one pass of the whole hot path over one batch: fa_fwd, then the backward as
fa_bwd runs it (fa_bwd_dq_stats: the dQ pass, which also forms the row statistics; then
fa_bwd_dkdv), on synthetic seeded inputs already resident in HBM. The default workload is the Llama-shaped causal case
(B=4, H=32, N=4096, d=128, bf16). Prints one JSON line.

FLOP model (algorithmic work, not what the kernels happen to execute): one "GEMM
unit" is 2*B*H*N^2*d, halved under causal masking. Forward = 2 units (QK^T, PV);
backward = 5 units (recomputed QK^T, dO V^T, P^T dO, dS^T Q, dS K), i.e. 2.5x the
forward. Per kernel: fwd 2 units, dkdv 4, dq 1 (its recomputation of S and dP is the
price of a dQ pass without atomics and is not counted).

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
BF16_FLOP_PER_CLK_CU = 4096  # dense bf16 MFMA FLOP per clock per compute unit (gfx950)
# The headline targets: the forward at >= 50 % and the backward at >= 35 % of the bf16
# dense MFMA peak on the Llama-shaped causal workload.
TARGET_FRAC = {"fwd": 0.50, "bwd": 0.35}
CSRC = os.path.join(ROOT, "exact_io_aware_attention_amd", "csrc")

# Memory traffic per launch of a kernel (bytes between L2 and the memory fabric: HBM and
# the Infinity Cache in front of it, which these counters cannot tell apart), from two
# rocprofv3 --pmc passes over this script on the named workload: reads as the sum over
# TCC_EA0_RDREQ_32B/_64B/_128B of requests x size, writes as WRITE_SIZE. The same passes
# count the library's copy kernel (--calibrate-copy-mib 1024) at 1.0000 GiB read and
# 1.0000 GiB written per launch, so the scale factors are 1. (FETCH_SIZE counts a 128-byte
# read request as 64 bytes, half of these kernels' reads.) Reported only while the
# kernel's sources hash to the value they had when the counters were taken; else null.
TRAFFIC = {
    ("c3", "fwd"): {"read_bytes": 503496832, "write_bytes": 136314880, "factor": 1.0,
                  "sources_sha256": "3273f60472fad0d613cfddf8eb09ddc58614d7a4ded4f456c1bd667c5fefd26e",
                  "profile": "profiles/attention_fwd_bwd_c3.md"},
    ("c3", "bwd_dq"): {"read_bytes": 785595456, "write_bytes": 138412096, "factor": 1.0,
                  "sources_sha256": "b446bb7000ef9a451b97c7a1865b0bca6512193d1f73b33394e2c8a4926a3304",
                  "profile": "profiles/attention_fwd_bwd_c3.md"},
    ("c3", "bwd_dkdv"): {"read_bytes": 675768000, "write_bytes": 268435456, "factor": 1.0,
                  "sources_sha256": "b446bb7000ef9a451b97c7a1865b0bca6512193d1f73b33394e2c8a4926a3304",
                  "profile": "profiles/attention_fwd_bwd_c3.md"},
}

# The sources each kernel is built from: its counters stay valid while these are unchanged.
KERNEL_SOURCES = {
    "fwd": ("fa_fwd.hip", "fa_common.h", "fa_launch.h"),
    "bwd_dkdv": ("fa_bwd.hip", "fa_common.h", "fa_launch.h"),
    "bwd_dq": ("fa_bwd.hip", "fa_common.h", "fa_launch.h"),
}


def sources_sha256(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(workload: str, kernel: str):
    t = TRAFFIC.get((workload, kernel))
    if t is None or kernel not in KERNEL_SOURCES or t["sources_sha256"] != sources_sha256(kernel):
        return None
    return t


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_unit(B, H, N, d, causal, lengths=None):
    if lengths is not None:
        return sum(2.0 * H * L * L * d * (0.5 if causal else 1.0) for L in lengths)
    return 2.0 * B * H * N * N * d * (0.5 if causal else 1.0)


def standard_attention(q, k, v, do, scale: float, causal: bool, reps: int = 3):
    """Standard attention on the same GPU, for comparison: the N x N matrices S, P and dP
    are written to HBM and read back, as the pages describe the method being improved
    upon. Plain PyTorch bf16: batched GEMMs (fp32 accumulation, bf16 results) and bf16
    elementwise/softmax kernels, each operand laid out as its GEMM wants it before the
    timed region (Q pre-scaled by the softmax scale, K^T, V^T, dO^T, Q^T contiguous), so
    nothing is transposed or converted inside it. Per step:
      forward   S = (scale Q) K^T            GEMM, writes S (bf16)
                S[hidden] = -inf             in place, causal only (reads and writes S)
                P = softmax(S)               reads S, writes P (bf16)
                O = P V                      GEMM, reads P
      backward  dV^T = dO^T P                GEMM, reads P
                dP = dO V^T                  GEMM, writes dP (bf16)
                D = rowsum(dO * O)           small
                dS = P * (dP - D)            in place on dP (two passes: reads dP/P, writes dP)
                dQ = scale dS K, dK^T = scale Q^T dS   GEMMs, read dS
    Returns fwd/bwd times (median of `reps` after one untimed pass, HIP events on the
    current stream), the peak device memory the two passes allocate, and O."""
    import torch
    B, N, H, d = q.shape
    bf = q.dtype
    qh = (q.float() * scale).to(bf).permute(0, 2, 1, 3).contiguous()          # (B, H, N, d)
    kh, vh, doh = (t.permute(0, 2, 1, 3).contiguous() for t in (k, v, do))
    kt, vt, dot = (t.transpose(-1, -2).contiguous() for t in (kh, vh, doh))   # (B, H, d, N)
    qt = q.permute(0, 2, 3, 1).contiguous()                                   # Q^T (B, H, d, N)
    mask = torch.ones(N, N, device=q.device, dtype=torch.bool).triu_(1) if causal else None

    def fwd():
        s = torch.matmul(qh, kt)
        if mask is not None:
            s.masked_fill_(mask, float("-inf"))
        p = torch.softmax(s, dim=-1)
        del s
        return p, torch.matmul(p, vh)

    def bwd(p, o):
        dvt = torch.matmul(dot, p)
        dp = torch.matmul(doh, vt)
        dd = (doh.float() * o.float()).sum(-1, keepdim=True).to(bf)
        dp.sub_(dd).mul_(p)                        # dS, in place
        dq = torch.matmul(dp, kh).mul_(scale)
        dkt = torch.matmul(qt, dp).mul_(scale)
        return dq, dkt, dvt

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
    # HBM bytes the N x N matrices alone force per step, counting each read or write of
    # S, P, dP once (bf16): forward S write, S read and P write (softmax), P read (PV),
    # plus a read and a write of S for the causal mask; backward P read (dV), dP write,
    # dP read + write (- D), dP and P read + dP write (* P), dS read twice (dQ, dK).
    nn = 2.0 * B * H * N * N
    nxn = nn * ((4 + (2 if causal else 0)) + 9)
    return {"fwd_ms": med(tf), "bwd_ms": med(tb), "peak_extra_bytes": int(peak),
            "nxn_bytes_per_step": nxn, "passes": reps + 1}, o.permute(0, 2, 1, 3)


def time_calls(call, reps: int = 20, rounds: int = 5):
    """Two timings of a library call on the current stream (HIP events): the steady-state
    time per call, as the median over `rounds` of `reps` back-to-back calls (the way the
    step is timed), and the median time of a single call that starts on an idle GPU (what
    a lone call waits, launch and ramp-up included)."""
    import torch
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    batch = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        batch.append(e0.elapsed_time(e1) / reps)
    single = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        single.append(e0.elapsed_time(e1))
    return sorted(batch)[len(batch) // 2], sorted(single)[len(single) // 2]


def decode_bench(reps: int = 20):
    """fa_fwd_decode on the decode workloads: the steady-state time per call (and a lone
    call's, see time_calls) and the achieved rate of the algorithmic bytes (K and V read
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

        ms, ms_single = time_calls(call, reps)
        algo = 2 * B * Nk * H * d * 2 + 2 * B * Nq * H * d * 2 + B * H * Nq * 4
        gbs = algo / (ms * 1e-3) / 1e9
        res[name] = {"workload": w.description, "batch": B, "heads": H, "seqlen_q": Nq, "seqlen_k": Nk,
                     "head_dim": d, "causal": w.causal, "ms": round(ms, 4), "ms_single_call": round(ms_single, 4),
                     "algorithmic_bytes": algo,
                     "achieved_gbs": round(gbs, 1), "hbm_peak_gbs": PEAK_HBM_GBS,
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "bound": "hbm"}
        del q, k, v, o, lse, ws
    return res


def fp8_bench(reps: int = 20, batch=None, seqlen=None):
    """fa_fwd_fp8 on the 8-bit workloads: the steady-state time per call (and a lone
    call's, see time_calls) and the forward's algorithmic FLOPs (2 GEMM units, halved
    under causal) per second against the fp8 MFMA peak."""
    import torch
    import exact_io_aware_attention_amd as fa
    import workloads as W
    res = {}
    for name, w in sorted(W.FP8_WORKLOADS.items()):
        q8, k8, v8 = (t.cuda() for t in W.make_fp8_inputs(w, batch=batch, seqlen=seqlen))
        B, N, H, d = q8.shape
        o = torch.empty((B, N, H, d), device=q8.device, dtype=torch.bfloat16)
        lse = torch.empty((B, H, N), device=q8.device, dtype=torch.float32)
        sp = torch.cuda.current_stream().cuda_stream

        def call():
            st = fa.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                               w.scale, w.descale_q, w.descale_k, w.descale_v, int(w.causal), sp)
            if st != fa.FA_OK:
                raise fa.FAError(st, "fa_fwd_fp8")

        ms, ms_single = time_calls(call, reps)
        flops = 2 * (2.0 * B * H * N * N * d) * (0.5 if w.causal else 1.0)
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"workload": w.description + (" (resized)" if batch or seqlen else ""),
                     "batch": B, "heads": H, "seqlen": N, "head_dim": d,
                     "causal": w.causal, "ms": round(ms, 4), "ms_single_call": round(ms_single, 4),
                     "tflops": round(tf, 2), "bound": "mfma",
                     "peak_tflops": PEAK_FP8_TFLOPS, "frac_of_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        del q8, k8, v8, o, lse
    return res


def atomic_bwd_bench(fa, tensors, dims, det_ms: float, reps: int = 10):
    """fa_bwd_atomic (dQ by fp32 atomics from the dK/dV kernel, then a conversion) on the
    step's inputs, against the deterministic backward's time: the measured alternative to
    the separate dQ pass (head_dim 128, bf16 only)."""
    import torch
    q, k, v, o, lse, do, cup = tensors
    B, H, N, d, T, scale, causal, sp = dims
    wsb = fa.fa_bwd_atomic_workspace_bytes(B, H, N, d, int(cup is not None), T)
    ws = torch.empty(wsb, device=q.device, dtype=torch.uint8)
    g = [torch.empty_like(q) for _ in range(3)]

    def call():
        st = fa.fa_bwd_atomic(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                              g[0].data_ptr(), g[1].data_ptr(), g[2].data_ptr(), ws.data_ptr(), wsb, B, H, N, d, scale,
                              causal, cup, T, fa.FA_DTYPE_BF16, sp)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_bwd_atomic")
    for _ in range(3):
        call()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"ms": round(ms, 4), "deterministic_ms": round(det_ms, 4), "ratio_to_deterministic": round(ms / det_ms, 3),
            "workspace_gib": round(wsb / 2**30, 3),
            "note": "fa_bwd_atomic: row statistics + accumulator clear, the fused dK/dV/dQ kernel, dQ conversion"}


def ceilings(reps: int = 5):
    """The device's own figures and measured ceilings: compute units and maximum engine
    clock as the HIP runtime reports them (the dense bf16 MFMA peak follows as CUs x 4096
    FLOP/clk x clock), then three loops timed with HIP events on the launch stream (median
    of `reps`): independent bf16 MFMA chains in every SIMD, independent v_exp_f32 and fp32
    FMA chains in every lane (the vector-ALU roof of the softmax), LDS operand reads, one
    MFMA chain per wave with vector work between its MFMAs (how much of it the matrix pipe
    hides), independent MFMA chains with the forward's vector mix per MFMA (the MFMA rate
    that mix allows at one and two waves per SIMD), and a 1 GiB copy."""
    import torch
    import exact_io_aware_attention_amd as fa
    info = fa.fa_device_info(torch.cuda.current_device())
    cus, clk_khz = info["compute_units"], info["max_clock_khz"]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    def ok(st, name):
        if st != fa.FA_OK:
            raise fa.FAError(st, name)

    mblocks, miters = 4 * cus, 2000         # four waves per SIMD, four chains per wave, ~1 ms
    vblocks, viters = 32 * cus, 1000
    out = torch.empty(max(mblocks, vblocks) * 256, device="cuda", dtype=torch.float32)
    t_mfma = timed(lambda: ok(fa.fa_ubench_mfma_bf16(out.data_ptr(), mblocks, miters, sp), "mfma"))
    m8iters = miters // 2                   # the 8-bit MFMA does four times the FLOPs in twice the time
    t_mfma8 = timed(lambda: ok(fa.fa_ubench_mfma_fp8(out.data_ptr(), mblocks, m8iters, sp), "mfma fp8"))
    t_exp = timed(lambda: ok(fa.fa_ubench_valu(out.data_ptr(), vblocks, viters, 0, sp), "exp"))
    t_fma = timed(lambda: ok(fa.fa_ubench_valu(out.data_ptr(), vblocks, viters, 1, sp), "fma"))
    lblocks, liters = 2 * cus, 4000          # two 64 KiB workgroups per CU (two waves per SIMD)
    t_ldsr = timed(lambda: ok(fa.fa_ubench_lds(out.data_ptr(), lblocks, liters, 0, sp), "lds rows"))
    t_ldst = timed(lambda: ok(fa.fa_ubench_lds(out.data_ptr(), lblocks, liters, 1, sp), "lds transposed"))
    # One dependent MFMA chain per wave with n independent vector operations after each
    # MFMA: cycles per MFMA (at the reported clock) at one and two waves per SIMD, with the
    # accumulator in VGPRs or AGPRs; 32 cycles is the matrix pipe's rate.
    citers = 2000
    coexec = {}
    for wps in (1, 2):
        for nv, op in ((0, 1), (4, 1), (8, 1), (2, 0), (4, 0)):
            for ag in (0, 1):
                t = timed(lambda: ok(fa.fa_ubench_mfma_valu(out.data_ptr(), wps * cus, citers, nv, ag, op, sp),
                                     "mfma+valu"))
                key = f"{wps}w_{'exp' if op == 0 else 'fma'}{nv}_{'agpr' if ag else 'vgpr'}"
                coexec[key] = round(t * 1e-3 * clk_khz * 1e3 / (wps * citers * 4), 1)
    # The forward's instruction mix (one exponential and three FMAs per MFMA) without its
    # dependences, LDS reads or barriers, four independent MFMA chains per wave, at one and
    # two waves per SIMD: the share of the MFMA peak that mix allows, beside the MFMAs alone.
    xiters = 4000
    mix = {}
    for wps in (1, 2):
        for m in (0, 1):
            t = timed(lambda: ok(fa.fa_ubench_mfma_mix(out.data_ptr(), wps * cus, xiters, m, sp), "mfma mix"))
            fl = wps * cus * 4 * xiters * 4 * 32768.0
            mix[f"{wps}w_{'softmax_mix' if m else 'mfma_only'}_frac_of_peak"] = round(
                fl / (t * 1e-3) / (cus * BF16_FLOP_PER_CLK_CU * clk_khz * 1e3), 3)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: ok(fa.fa_ubench_copy(src.data_ptr(), dst.data_ptr(), nbytes, 16 * cus, sp), "copy"))
    del src, dst, out
    torch.cuda.empty_cache()
    mfma_flops = mblocks * 4 * miters * 8 * 32768.0
    lane_ops = vblocks * 256 * viters * 8.0
    clk_hz = clk_khz * 1e3
    return {
        "device": info,
        "peak_bf16_tflops_from_clock": round(cus * BF16_FLOP_PER_CLK_CU * clk_hz / 1e12, 1),
        "mfma_bf16_loop_tflops": round(mfma_flops / (t_mfma * 1e-3) / 1e12, 1),
        "mfma_fp8_loop_tflops": round(mblocks * 4 * m8iters * 8 * 131072.0 / (t_mfma8 * 1e-3) / 1e12, 1),
        "exp_gops": round(lane_ops / (t_exp * 1e-3) / 1e9, 1),
        "exp_lane_ops_per_clk_cu": round(lane_ops / (t_exp * 1e-3) / clk_hz / cus, 2),
        "fma_fp32_tflops": round(2 * lane_ops / (t_fma * 1e-3) / 1e12, 1),
        "fma_lane_ops_per_clk_cu": round(lane_ops / (t_fma * 1e-3) / clk_hz / cus, 2),
        "copy_gbs": round(2 * nbytes / (t_copy * 1e-3) / 1e9, 1),
        # LDS operand reads (1 KiB per wave each: one ds_read_b128, or two 512-byte
        # ds_read_b64_tr_b16) per clock per CU and in bytes per second: what bounds an
        # MFMA whose 32x16 bf16 operand comes from LDS
        "lds_row_operands_per_clk_cu": round(lblocks * 4 * liters * 8 / (t_ldsr * 1e-3) / clk_hz / cus, 4),
        "lds_tr_operands_per_clk_cu": round(lblocks * 4 * liters * 8 / (t_ldst * 1e-3) / clk_hz / cus, 4),
        "lds_row_tbs": round(lblocks * 4 * liters * 8 * 1024 / (t_ldsr * 1e-3) / 1e12, 1),
        "lds_tr_tbs": round(lblocks * 4 * liters * 8 * 1024 / (t_ldst * 1e-3) / 1e12, 1),
        "mfma_chain_cycles_per_mfma": coexec,
        "mfma_with_forward_mix": mix,
        "ms": {"mfma": round(t_mfma, 4), "mfma_fp8": round(t_mfma8, 4), "exp": round(t_exp, 4), "fma": round(t_fma, 4), "copy": round(t_copy, 4),
               "lds_rows": round(t_ldsr, 4), "lds_tr": round(t_ldst, 4)},
        "note": "rates per clock use the reported maximum clock; the clock under load may be lower",
    }


def cpu_baseline(inp, w, budget_s: float):
    """Time the oracle (fp64, NumPy) on whole heads of the workload until ~budget_s."""
    import numpy as np
    import oracle
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max([i.get("num_threads", 1) for i in blas] or [1])
    except Exception:  # pragma: no cover - informational only
        blas_threads = len(os.sched_getaffinity(0))
    B, H = inp.q.shape[0], inp.q.shape[2]
    heads = [(b, h) for b in range(B) for h in range(H)]
    flops = 0.0
    done = 0
    N0 = inp.q.shape[1]
    if 8.0 * N0 * N0 > 4e9:
        # One head's fp64 score matrix would exceed 4 GB (the long-context workload): time
        # the oracle on 256 seeded query rows per head instead, O and dQ of those rows
        # (forward 2 and dQ 3 products of 256 x N x d: 10 * 256 * N * d FLOP per head).
        import workloads as W
        rows = W.sample_rows(w.seed, N0, 256)
        t0 = time.perf_counter()
        for b, h in heads:
            q, k, v, do = (oracle.to_f64(t[b, :, h, :]) for t in (inp.q, inp.k, inp.v, inp.do))
            oracle.forward_rows(q, k, v, w.scale, w.causal, rows)
            oracle.backward_query_rows(q, k, v, do, w.scale, w.causal, rows)
            flops += 10.0 * rows.size * N0 * q.shape[1]
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        return {
            "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"256 seeded query rows (O and dQ) of {done} of {len(heads)} heads of {w.name}, fp64, "
                      f"{dt:.1f} s wall; FLOPs counted for those rows only (10 x 256 x N x d per head)",
            "host_cpus": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "blas": [{"vendor": i.get("internal_api"), "version": i.get("version"),
                      "threads": i.get("num_threads"), "library": os.path.basename(i.get("filepath", ""))}
                     for i in blas],
        }
    if inp.cu_seqlens is not None:
        # packed batch: whole (sequence, head) pairs, causal within each sequence
        cu = inp.cu_seqlens.tolist()
        H = inp.q.shape[1]
        heads = [(s, h) for s in range(len(cu) - 1) for h in range(H)]

        def view(t, s, h):
            return oracle.to_f64(t[cu[s]:cu[s + 1], h, :])
    else:
        def view(t, b, h):
            return oracle.to_f64(t[b, :, h, :])
    t0 = time.perf_counter()
    for b, h in heads:
        q, k, v, do = (view(t, b, h) for t in (inp.q, inp.k, inp.v, inp.do))
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
        "sample": f"{done} of {len(heads)} ({'sequence' if inp.cu_seqlens is not None else 'batch'}, head) pairs "
                  f"of {w.name}, fp64 forward + backward "
                  f"(oracle materialises the full N x N scores), {dt:.1f} s wall",
        "host_cpus": len(os.sched_getaffinity(0)),
        "os_cpu_count": os.cpu_count(),
        "blas": [{"vendor": i.get("internal_api"), "version": i.get("version"),
                  "threads": i.get("num_threads"), "library": os.path.basename(i.get("filepath", ""))}
                 for i in blas],
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
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (MFMA loop, exponential and FMA rates, copy)")
    ap.add_argument("--no-standard", action="store_true",
                    help="skip the standard-attention comparison (materialised N x N scores)")
    ap.add_argument("--no-atomic", action="store_true",
                    help="skip timing fa_bwd_atomic (dQ by fp32 atomics) beside the deterministic backward")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before the warmup, run the library's copy kernel over this many MiB, three times, "
                         "as the known-size reference for the byte counters")
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

    def k_dq_stats():
        check(fa.fa_bwd_dq_stats(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                 lse.data_ptr(), ws.data_ptr(), ws_bytes, dq.data_ptr(), B, H, N, d, w.scale, causal,
                                 cup, T, dt_code, sp), "fa_bwd_dq_stats")

    def k_dkdv():
        check(fa.fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             ws.data_ptr(), ws_bytes, dk.data_ptr(), dv.data_ptr(), B, H, N, d, w.scale,
                             causal, cup, T, dt_code, sp), "fa_bwd_dkdv")

    # The step: the forward, then the backward as fa_bwd runs it (the dQ pass, which also
    # forms the row statistics, then dK/dV), each stage timed on its own.
    kernels = [("fwd", k_fwd), ("bwd_dq", k_dq_stats), ("bwd_dkdv", k_dkdv)]
    if a.calibrate_copy_mib > 0:
        # The library's copy kernel (16-byte loads and stores per lane, like the kernels'
        # tile copies): it reads and writes calibrate_copy_mib MiB per launch, the known
        # sizes that the byte counters of the attention kernels are scaled against.
        nbytes = a.calibrate_copy_mib * (1 << 20)
        src = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            check(fa.fa_ubench_copy(src.data_ptr(), dst.data_ptr(), nbytes, 4096, sp), "fa_ubench_copy")
        torch.cuda.synchronize()
        log(f"bench: copy calibration (ub_copy_kernel), {a.calibrate_copy_mib} MiB read + "
            f"{a.calibrate_copy_mib} MiB written per launch, 3 launches")
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

    def pass_summary(name, flops, ms):
        tf = flops / (ms * 1e-3) / 1e12
        frac = tf / PEAK_BF16_TFLOPS
        return {"ms": round(ms, 4), "tflops": round(tf, 2), "frac_of_peak": round(frac, 4),
                "target_frac": TARGET_FRAC[name], "target_met": bool(frac >= TARGET_FRAC[name]),
                "target_ms": round(flops / (TARGET_FRAC[name] * PEAK_BF16_TFLOPS * 1e12) * 1e3, 4)}

    unit = gemm_unit(B, H, N, d, w.causal, inp.lengths)
    fwd_fl, bwd_fl = 2 * unit, 5 * unit
    algo = {"fwd": 2 * unit, "bwd_dkdv": 4 * unit, "bwd_dq": 1 * unit}
    # each operand read once and each result written once (X = one (tokens, heads, d) tensor,
    # S = one fp32 row statistic per (head, token))
    X = T * H * d * q.element_size()
    S = T * H * 4
    algo_bytes = {"fwd": 3 * X + X + S, "bwd_dq": 5 * X + S + X + 2 * S, "bwd_dkdv": 4 * X + 2 * S + 2 * X}
    bwd_ms = per["bwd_dkdv"] + per["bwd_dq"]
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
        "fwd": pass_summary("fwd", fwd_fl, per["fwd"]),
        "bwd": pass_summary("bwd", bwd_fl, bwd_ms),
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in per.items()},
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if tr is None else tr["read_bytes"] + tr["write_bytes"],
        },
    }
    if tr is not None:
        tb = tr["read_bytes"] + tr["write_bytes"]
        out["roofline"]["traffic_detail"] = {
            "fabric_bytes_per_launch": tb, "read_bytes": tr["read_bytes"], "write_bytes": tr["write_bytes"],
            "counter_scale_factor": tr["factor"],
            "algorithmic_bytes_per_launch": algo_bytes[dom],
            "ratio_to_algorithmic": round(tb / algo_bytes[dom], 3),
            "achieved_gbs": round(tb / (per[dom] * 1e-3) / 1e9, 1),
            "note": "bytes between L2 and the memory fabric (HBM plus the Infinity Cache in front of it)",
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
        e = q.element_size()
        # this library's operand bytes per step: forward reads Q, K, V and writes O, LSE;
        # backward reads Q, K, V, O, dO (+ statistics) and writes dQ, dK, dV
        ours_bytes = (4 + 8) * B * N * H * d * e + 16 * B * H * N
        ours_fwd, ours_bwd = per["fwd"], bwd_ms
        out["standard_attention"] = {
            "fwd_ms": round(st["fwd_ms"], 4), "bwd_ms": round(st["bwd_ms"], 4),
            "speedup_fwd": round(st["fwd_ms"] / ours_fwd, 2), "speedup_bwd": round(st["bwd_ms"] / ours_bwd, 2),
            "peak_extra_gib": round(st["peak_extra_bytes"] / 2**30, 2),
            "ours_workspace_gib": round(ws_bytes / 2**30, 4),
            "o_max_abs_diff": round(float((o_std.float() - o.float()).abs().max()), 4),
            "nxn_bytes_per_step": st["nxn_bytes_per_step"],
            "ours_operand_bytes_per_step": ours_bytes,
            "dispatch_passes": st["passes"],
            "note": "bf16 PyTorch: S, P, dP materialised in HBM; operand layouts prepared outside the "
                    "timed region; Q pre-scaled in bf16",
        }
        del o_std
        torch.cuda.empty_cache()
    if not a.no_atomic and d == 128 and w.dtype == "bf16":
        log("bench: backward with dQ by fp32 atomics (fa_bwd_atomic)")
        out["bwd_atomic"] = atomic_bwd_bench(fa, (q, k, v, o, lse, do, cup),
                                             (B, H, N, d, T, w.scale, causal, sp), bwd_ms)
    if not a.no_ceilings:
        log("bench: measured ceilings")
        c = ceilings()
        out["ceilings"] = c
        out["roofline"]["peak_from_device_clock"] = c["peak_bf16_tflops_from_clock"]
        out["roofline"]["peak_measured_mfma_loop"] = c["mfma_bf16_loop_tflops"]
        out["roofline"]["frac_of_measured"] = round(achieved / c["mfma_bf16_loop_tflops"], 4)
        # The softmax's exponentials against the measured v_exp_f32 rate: one per visible
        # score in the forward (B H N^2 / 2 under causal), a lower bound on its time.
        n_exp = unit / (2.0 * d)
        out["ceilings"]["fwd_exp_bound_ms"] = round(n_exp / (c["exp_gops"] * 1e9) * 1e3, 4)
    if not a.no_decode:
        log("bench: decode workloads")
        out["decode"] = decode_bench()
    if not a.no_fp8:
        log("bench: 8-bit forward")
        out["fp8_forward"] = fp8_bench(batch=a.batch, seqlen=a.seqlen)
        if "ceilings" in out:
            loop8 = out["ceilings"]["mfma_fp8_loop_tflops"]
            for leg in out["fp8_forward"].values():
                leg["peak_measured_mfma_loop"] = loop8
                leg["frac_of_measured"] = round(leg["tflops"] / loop8, 4)
    if a.cpu_budget > 0:
        log(f"bench: CPU oracle baseline (~{a.cpu_budget:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(inp, w, a.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
