"""Benchmark of the dense GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

A step is one C = A @ B in fp32, M = N = K = 4096, row-major, not transposed,
A and B iid uniform[-1, 1) (seed 1), already resident in device memory; the
timed region is exactly K steps on one stream, bracketed by device
synchronisation, after W untimed steps (and at least 100 ms of them).  Every
input is generated and uploaded before the first timed launch.

Also measured (same method, extra keys of the one JSON line), each with every
output of a timed call checked against the CPU oracle:
  fp16_2048 / bf16_2048  16-bit operands, fp32 accumulation, 16-bit output at
                         2048^3, nn/tn/nt (entries N(0,1)/sqrt(K), seed 2);
  sgemm_512              SGEMM 512^3 nn (uniform, seed 0);
  sgemm_ragged           C = 1.5 op(A) op(B) - 0.5 C at 4095x4097x1031 and
                         8192x256x8192, four transpose pairs, ld + 8 (seed 4);
  attention_heads, epilogue, lora_step  the strided-batch, fused-epilogue and
                         LoRA-step workloads (timings).

`roofline` is for the fp32 kernel: achieved TFLOP/s = 2*M*N*K per launch /
mean launch duration, timed with events recorded on the stream the kernel runs
on, against the MI355X dense fp32 matrix peak (157.3 TFLOP/s), and against the
matrix-core rate the control probe measures on the same box.  `control` holds
the control benchmarks (matrix-core peak with the shader clock under load, and
a plain copy) and whether they are within 10% of their references;
`per_launch_us` and `cold_us` give per-launch medians, best and worst, and the
median after a 512 MiB cache scrub.  `power` holds the board's socket power
and shader clock (from amd-smi) while fp32 4096^3, fp16 2048^3 nn and the
fp16 matrix-core probe run back to back for 4 s each (skipped under a
profiler, like the other amd-smi readings).  `cpu_baseline` times the CPU oracle
(plain fp64 triple loop, the host cores this process may use) on a bounded
sample of the same workload: whole rows of C.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F32 = 157.3      # TFLOP/s, MI355X dense fp32 matrix
PEAK_F16 = 2516.6     # TFLOP/s, MI355X dense fp16 matrix
HBM_PEAK = 8000.0     # GB/s

# Control benchmarks and their references.  "Metal GEMM Kernels for LoRA
# Training on Apple Silicon", section 9: a performance figure is trusted only
# while a control benchmark stays within 10% of its reference.  The matrix-core
# probes' references are the published peaks.  No figure is published for what
# a plain copy sustains (a read + write stream does not approach the 8 TB/s HBM
# peak), so the copy's reference is the rate measured here: 4.47-4.67 TB/s on
# every box this library was measured on, 56-58% of the peak.  The line also
# reports the copy as a fraction of the peak.
REF_MFMA_F32 = PEAK_F32
REF_MFMA_F16 = PEAK_F16
REF_COPY_GBS = 4600.0
CONTROL_TOL = 0.10

# What `traffic` counts: bytes the L2 caches exchange with the memory fabric
# per launch (read requests by size + write requests by size, from rocprofv3
# TCC_EA0 counters).  The 256 MB Infinity Cache sits behind that interface, so
# its hits are included: the figure is an upper bound on HBM traffic.
TRAFFIC_SOURCE = "L2-to-fabric bytes per launch (TCC_EA0 read/write requests x request size; includes Infinity Cache hits)"


def tflops(M, N, K, seconds):
    return 2.0 * M * N * K / seconds / 1e12


def measured_traffic(kernel, ta, tb, M, N):
    """HBM bytes per dispatch of this kernel on an M x N output from the
    committed counter summary (profiles/hbm_traffic.txt, keyed by kernel,
    transpose pair and workgroup count), or None when that summary was taken
    from other kernel sources than the ones built now."""
    import hashlib
    import glob
    import dense_gemm_amd as dg
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    # the GEMM kernels' sources only: the dispatcher (api.cpp) picks kernels but
    # does not change what a given kernel moves, and probe.hip holds no GEMM
    for f in sorted(glob.glob(os.path.join(ROOT, "dense_gemm_amd", "csrc", "*.hip")) +
                    glob.glob(os.path.join(ROOT, "dense_gemm_amd", "csrc", "*.hpp"))):
        if os.path.basename(f) != "probe.hip":
            h.update(open(f, "rb").read())
    table = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.rsplit("=", 1)
            table[k.strip()] = v.strip()
    if table.get("sources") != h.hexdigest()[:16]:
        return None
    tm, tn = dg.dg_kernel_tile_m(kernel), dg.dg_kernel_tile_n(kernel)
    wgs = -(-M // tm) * -(-N // tn)
    key = f"{dg.dg_kernel_name(kernel)} {'t' if ta else 'n'}{'t' if tb else 'n'} wgs={wgs}"
    return int(float(table[key])) if key in table else None


def time_launches(fn, stream, reps):
    """Mean duration of one launch (s), from events on `stream` around reps launches."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / reps


def warm(fn, min_count=10, min_s=0.1):
    """Untimed launches of fn until at least min_count have run and at least
    min_s seconds have passed (the shader clock ramps up under sustained
    load; a few launches after an idle gap run slow).  Returns the count."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < min_count or time.perf_counter() - t0 < min_s:
        for _ in range(max(1, min_count)):
            fn()
        n += max(1, min_count)
        torch.cuda.synchronize()
    return n


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_check(dtype, got, ref, ab, alpha=1.0, beta=0.0, c0=None):
    """Every output of a timed launch against the CPU oracle: max err/bound
    and the number of violations."""
    import oracle
    worst, bad = oracle.compare(dtype, got, ref, ab, alpha, beta, c0)
    return {"outputs": int(got.size), "max_err_over_bound": round(worst, 4), "violations": bad}


def per_launch(fn, stream, n):
    """Per-launch durations (µs) from an event pair around each of n launches
    on `stream`: median, best and worst."""
    import statistics
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    for a, b in pairs:
        a.record(stream)
        fn()
        b.record(stream)
    pairs[-1][1].synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in pairs]
    return {"median": round(statistics.median(us), 2), "best": round(min(us), 2),
            "worst": round(max(us), 2), "launches": n}


def cold_launches(fn, stream, n, scrub):
    """Median duration (µs) of n launches, each after `scrub` (a 512 MiB
    buffer, twice the Infinity Cache) is rewritten on the same stream, so the
    operands come from HBM instead of the caches."""
    import statistics
    import torch
    us = []
    for i in range(n):
        scrub.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        us.append(a.elapsed_time(b) * 1e3)
    return round(statistics.median(us), 2)


def control_probes(dev, stream):
    """The control benchmarks (libdense_gemm_probe.so): matrix-core peak of the
    fp32 and fp16 instructions the GEMMs use, with the shader clock while they
    run, and the plain-copy HBM rate; each against its reference.  Beside
    them, not gated: the fp16 matrix-core rate on pseudo-random operands that
    change every instruction, at the clock the part holds under that load."""
    import statistics
    import torch

    import dense_gemm_amd.probe as pr

    sptr = stream.cuda_stream
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count   # two waves per SIMD
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    khz = pr.dgp_wall_clock_khz()
    res = {}
    for name, kind, iters in (("mfma_f32", pr.DGP_MFMA_F32, 8000), ("mfma_f16", pr.DGP_MFMA_F16, 16000),
                              ("mfma_f16_random", pr.DGP_MFMA_F16_RANDOM, 16000)):
        def f(kind=kind, iters=iters):
            rc = pr.dgp_mfma_peak(kind, wgs, iters, sink.data_ptr(), clocks.data_ptr(), sptr)
            if rc != 0:
                raise RuntimeError(f"dgp_mfma_peak failed ({rc}, hip {pr.dgp_last_hip_error()})")
        f()
        torch.cuda.synchronize()
        t = min(time_launches(f, stream, 3) for _ in range(3))
        c = clocks.view(wgs, 2).cpu().numpy()
        ratio = statistics.median(float(x) / float(y) for x, y in c if y > 0)
        res[name] = {"tflops": round(pr.dgp_mfma_flops(kind, wgs, iters) / t / 1e12, 1),
                     "clock_mhz": round(ratio * khz / 1e3) if khz > 0 else None}
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def cp():
        rc = pr.dgp_copy(src.data_ptr(), dst.data_ptr(), nbytes, sptr)
        if rc != 0:
            raise RuntimeError(f"dgp_copy failed ({rc}, hip {pr.dgp_last_hip_error()})")
    cp()
    torch.cuda.synchronize()
    t = min(time_launches(cp, stream, 5) for _ in range(2))
    assert bool(torch.equal(src[:: 1 << 20], dst[:: 1 << 20]))
    del src, dst
    gbs = 2 * nbytes / t / 1e9
    ok = (res["mfma_f32"]["tflops"] >= (1 - CONTROL_TOL) * REF_MFMA_F32
          and res["mfma_f16"]["tflops"] >= (1 - CONTROL_TOL) * REF_MFMA_F16
          and gbs >= (1 - CONTROL_TOL) * REF_COPY_GBS)
    return {"mfma_f32_tflops": res["mfma_f32"]["tflops"], "mfma_f32_clock_mhz": res["mfma_f32"]["clock_mhz"],
            "mfma_f16_tflops": res["mfma_f16"]["tflops"], "mfma_f16_clock_mhz": res["mfma_f16"]["clock_mhz"],
            # not gated: the matrix cores on operands that change every
            # instruction, as in a GEMM on random data (power sets the clock)
            "mfma_f16_random_tflops": res["mfma_f16_random"]["tflops"],
            "mfma_f16_random_clock_mhz": res["mfma_f16_random"]["clock_mhz"],
            "copy_gbs": round(gbs, 1), "copy_frac_of_hbm_peak": round(gbs / HBM_PEAK, 3),
            "references": {"mfma_f32_tflops": REF_MFMA_F32, "mfma_f16_tflops": REF_MFMA_F16,
                           "copy_gbs": REF_COPY_GBS, "tolerance": CONTROL_TOL},
            "within_tolerance": bool(ok)}


def lora_step(dev, stream, reps, out="f16"):
    """Times the 18 GEMMs of one LoRA MLP-block step (512 tokens, d_model 2048,
    FFN 5632, rank 32; fp16 operands, fp32 accumulation) back to back on one
    stream, and each GEMM on its own (events around repeated launches).  Each
    GEMM goes through dg_gemm_splitk with the library's choice of K split
    (skinny and low-rank products are split, the others are not).  out: the
    type of every C, "f16" (rounded once) or "f32" (the fp32 result written
    as is, "Metal GEMM Kernels for LoRA Training", section 4)."""
    import numpy as np
    import torch

    import dense_gemm_amd as dg
    import synth

    sptr = stream.cuda_stream
    code = dg.DG_F16_F32ACC if out == "f16" else dg.DG_F16_F32OUT
    ctype = torch.float16 if out == "f16" else torch.float32
    calls = []
    # one split-K workspace for the whole step (the calls are ordered on one stream)
    wsb = max(dg.dg_gemm_splitk_workspace_size(M, N, dg.dg_gemm_splitk_choose(ta, tb, M, N, K, code))
              for _, M, N, K, ta, tb, _, _ in synth.LORA_GEMMS)
    ws = torch.empty(max(wsb, 16) // 4, dtype=torch.float32, device=dev)
    for idx, (name, M, N, K, ta, tb, beta, _) in enumerate(synth.LORA_GEMMS):
        a, b, c0 = synth.lora_problem(idx, seed=3, out=out)
        A = torch.from_numpy(np.ascontiguousarray(a.T if ta else a)).to(dev)
        B = torch.from_numpy(np.ascontiguousarray(b.T if tb else b)).to(dev)
        C = torch.from_numpy(c0).to(dev) if c0 is not None else torch.empty((M, N), dtype=ctype, device=dev)
        lda, ldb = (M if ta else K), (K if tb else N)
        k = dg.dg_select_kernel(ta, tb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), N,
                                code)

        splits = dg.dg_gemm_splitk_choose(ta, tb, M, N, K, code)

        def f(ta=ta, tb=tb, M=M, N=N, K=K, A=A, B=B, C=C, lda=lda, ldb=ldb, beta=beta, stream_ptr=None):
            rc = dg.dg_gemm_splitk(ta, tb, M, N, K, 1.0, A.data_ptr(), lda, B.data_ptr(), ldb, beta,
                                   C.data_ptr(), N, code,
                                   sptr if stream_ptr is None else stream_ptr, 0, ws.data_ptr(),
                                   ws.numel() * 4)
            if rc != 0:
                raise dg.GemmError(rc)
        calls.append((name, M, N, K, f, dg.dg_kernel_name(k) + (f" splitk{splits}" if splits > 1 else "")))

    def step():
        for c in calls:
            c[4]()

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    t_step = time_launches(step, stream, reps)
    flops = sum(2.0 * M * N * K for _, M, N, K, _, _ in calls)

    # the same step captured once in a HIP graph and replayed: the library
    # only enqueues kernels on the caller's stream (no allocation, no memset),
    # so a whole step records; replay takes the host's per-launch cost off the
    # GPU's critical path
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for name, M, N, K, f, _ in calls:
            f(stream_ptr=torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t_graph = time_launches(graph.replay, stream, reps)
    per = []
    for name, M, N, K, f, kname in calls:
        # a few-microsecond kernel: several windows, the best one (a single
        # short window can be set by host-side jitter instead of the GPU)
        t = min(time_launches(f, stream, max(reps, 200)) for _ in range(3))
        per.append({"gemm": name, "M": M, "N": N, "K": K, "us": round(t * 1e6, 2),
                    "tflops": round(2.0 * M * N * K / t / 1e12, 2), "kernel": kname})
    return {"output": out, "step_ms": round(t_step * 1e3, 4), "gflop": round(flops / 1e9, 3),
            "tflops": round(flops / t_step / 1e12, 2),
            "tokens_per_s": round(512 / t_step, 1),
            "graph_step_ms": round(t_graph * 1e3, 4), "graph_tflops": round(flops / t_graph / 1e12, 2),
            "per_gemm": per}


def lora_step_paired(dev, stream, reps, check=True):
    """The 18 GEMMs of lora_step, with each pair of synth.LORA_PAIRS run as one
    strided-batch launch of dg_gemm_ex (batch 2: the two problems stored one
    after the other), and the other products as in lora_step: 14 launches
    for the same 72.38 GFLOP, fp16 C.  A batch of two fills more of the GPU
    than either half (gate and up: 352 tiles of 128x128 against 176), and a
    launch saves the few microseconds between dependent kernels.  Every
    output of the paired launches is checked against the oracle."""
    import numpy as np
    import torch

    import dense_gemm_amd as dg
    import synth

    sptr = stream.cuda_stream
    code = dg.DG_F16_F32ACC
    paired = {i for pr in synth.LORA_PAIRS for i in pr}
    wsb = max(dg.dg_gemm_splitk_workspace_size(M, N, dg.dg_gemm_splitk_choose(ta, tb, M, N, K, code))
              for _, M, N, K, ta, tb, _, _ in synth.LORA_GEMMS)
    ws = torch.empty(max(wsb, 16) // 4, dtype=torch.float32, device=dev)
    calls, pairs = [], []
    for idx, (name, M, N, K, ta, tb, beta, _) in enumerate(synth.LORA_GEMMS):
        if idx in paired:
            continue
        a, b, c0 = synth.lora_problem(idx, seed=3)
        A = torch.from_numpy(np.ascontiguousarray(a.T if ta else a)).to(dev)
        B = torch.from_numpy(np.ascontiguousarray(b.T if tb else b)).to(dev)
        C = torch.from_numpy(c0).to(dev) if c0 is not None else torch.empty((M, N), dtype=torch.float16, device=dev)
        lda, ldb = (M if ta else K), (K if tb else N)

        def f(ta=ta, tb=tb, M=M, N=N, K=K, A=A, B=B, C=C, lda=lda, ldb=ldb, beta=beta):
            rc = dg.dg_gemm_splitk(ta, tb, M, N, K, 1.0, A.data_ptr(), lda, B.data_ptr(), ldb, beta,
                                   C.data_ptr(), N, code, sptr, 0, ws.data_ptr(), ws.numel() * 4)
            if rc != 0:
                raise dg.GemmError(rc)
        calls.append((idx, f))
    for i0, i1 in synth.LORA_PAIRS:
        name, M, N, K, ta, tb, beta, _ = synth.LORA_GEMMS[i0]
        probs = [synth.lora_problem(i, seed=3) for i in (i0, i1)]
        A = torch.from_numpy(np.stack([np.ascontiguousarray(a.T if ta else a) for a, _, _ in probs])).to(dev)
        B = torch.from_numpy(np.stack([np.ascontiguousarray(b.T if tb else b) for _, b, _ in probs])).to(dev)
        C0 = (torch.from_numpy(np.stack([c0 for _, _, c0 in probs])).to(dev) if beta != 0.0 else None)
        C = C0.clone() if C0 is not None else torch.empty((2, M, N), dtype=torch.float16, device=dev)
        lda, ldb = (M if ta else K), (K if tb else N)

        def f(ta=ta, tb=tb, M=M, N=N, K=K, A=A, B=B, C=C, lda=lda, ldb=ldb, beta=beta):
            rc = dg.dg_gemm_ex(ta, tb, M, N, K, 1.0, A.data_ptr(), lda, M * K, B.data_ptr(), ldb, K * N,
                               beta, C.data_ptr(), N, M * N, 2, None, dg.DG_EPI_NONE, code, sptr)
            if rc != 0:
                raise dg.GemmError(rc)
        calls.append((i0, f))
        pairs.append((i0, i1, f, C, C0, probs))
    calls.sort(key=lambda c: c[0])          # the step's order, a pair at its first product

    def step():
        for _, f in calls:
            f()

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    t_step = time_launches(step, stream, reps)
    flops = sum(2.0 * M * N * K for _, M, N, K, _, _, _, _ in synth.LORA_GEMMS)
    res = {"launches": len(calls), "step_ms": round(t_step * 1e3, 4), "gflop": round(flops / 1e9, 3),
           "tflops": round(flops / t_step / 1e12, 2), "tokens_per_s": round(512 / t_step, 1)}
    if check:
        import oracle
        parity = []
        for i0, i1, f, C, C0, probs in pairs:
            name, M, N, K, ta, tb, beta, _ = synth.LORA_GEMMS[i0]
            if C0 is not None:
                C.copy_(C0)
            f()
            torch.cuda.synchronize()
            got = C.float().cpu().numpy()
            for h, (a, b, c0) in enumerate(probs):
                ref, ab = oracle.gemm(False, False, M, N, K, 1.0, a, K, b, N, beta, c0, N)
                r = oracle_check("f16", got[h], ref, ab, 1.0, beta, c0)
                parity.append({"gemm": synth.LORA_GEMMS[(i0, i1)[h]][0], **r})
        res["parity"] = parity
    return res


def _dev_tensor(x, dtype, dev):
    """A host array of the given storage type as a device tensor (bf16 from
    its uint16 bit patterns)."""
    import numpy as np
    import torch
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def bf16_square(dev, stream, reps, check=True):
    """bf16 operands, fp32 accumulation, bf16 output at 2048^3, nn/tn/nt, with
    the fp16 workload's recipe (N(0,1)/sqrt(K), seed 2); every output of the
    timed calls against the oracle."""
    import torch

    import dense_gemm_amd as dg
    import synth
    S = 2048
    a, b, _ = synth.problem(S, S, S, "bf16", "normal_sqrtk", 2)
    res = {"peak": PEAK_F16, "unit": "TFLOP/s"}
    outs = {}
    for name, ta, tb in (("nn", 0, 0), ("tn", 1, 0), ("nt", 0, 1)):
        A = _dev_tensor(a.T if ta else a, "bf16", dev)
        B = _dev_tensor(b.T if tb else b, "bf16", dev)
        C = torch.empty((S, S), dtype=torch.bfloat16, device=dev)
        k = dg.dg_select_kernel(ta, tb, S, S, S, A.data_ptr(), S, B.data_ptr(), S, C.data_ptr(), S,
                                dg.DG_BF16_F32ACC)

        def f(ta=ta, tb=tb, A=A, B=B, C=C):
            rc = dg.dg_gemm(ta, tb, S, S, S, 1.0, A.data_ptr(), S, B.data_ptr(), S, 0.0,
                            C.data_ptr(), S, dg.DG_BF16_F32ACC, stream.cuda_stream)
            if rc != 0:
                raise dg.GemmError(rc)

        warm(f, 20, 0.1)
        t = min(time_launches(f, stream, reps) for _ in range(3))
        ach = tflops(S, S, S, t)
        res[name] = {"tflops": round(ach, 2), "frac": round(ach / PEAK_F16, 4),
                     "kernel_us": round(t * 1e6, 2), "kernel": dg.dg_kernel_name(k)}
        torch.cuda.synchronize()
        outs[name] = C.float().cpu().numpy()
    if check:
        import oracle
        ref, ab = oracle.gemm(False, False, S, S, S, 1.0, a, S, b, S, 0.0, None, S)
        for name in outs:
            res[name]["parity"] = oracle_check("bf16", outs[name], ref, ab)
    return res


def attention_heads(dev, stream, reps):
    """The six per-head products of attention (head-major Q, K, V; "Metal GEMM
    Kernels for LoRA Training", section 8) for 512 tokens and 32 heads of 64,
    fp16, each one strided-batched call over the heads."""
    import torch

    import dense_gemm_amd as dg
    import synth
    T, D, H = 512, 64, 32
    products = [("S = Q K^T", T, T, D, 0, 1), ("O = P V", T, D, T, 0, 0),
                ("dV = P^T dO", T, D, T, 1, 0), ("dP = dO V^T", T, T, D, 0, 1),
                ("dQ = dS K", T, D, T, 0, 0), ("dK = dS^T Q", T, D, T, 1, 0)]
    st = synth.Stream(40)
    per, total_t, total_f = [], 0.0, 0.0
    for name, M, N, K, ta, tb in products:
        sa, sb = M * K, K * N
        A = _dev_tensor(synth.round_to(st.normal((H * sa,)), "f16"), "f16", dev)
        B = _dev_tensor(synth.round_to(st.normal((H * sb,)) / K ** 0.5, "f16"), "f16", dev)
        C = torch.empty((H, M, N), dtype=torch.float16, device=dev)
        lda, ldb = (M if ta else K), (K if tb else N)

        def f(M=M, N=N, K=K, ta=ta, tb=tb, A=A, B=B, C=C, lda=lda, ldb=ldb, sa=sa, sb=sb):
            rc = dg.dg_gemm_ex(ta, tb, M, N, K, 1.0, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb,
                               0.0, C.data_ptr(), N, M * N, H, None, dg.DG_EPI_NONE,
                               dg.DG_F16_F32ACC, stream.cuda_stream)
            if rc != 0:
                raise dg.GemmError(rc)

        for _ in range(10):
            f()
        torch.cuda.synchronize()
        t = time_launches(f, stream, reps)
        fl = 2.0 * M * N * K * H
        total_t += t
        total_f += fl
        per.append({"product": name, "M": M, "N": N, "K": K, "heads": H,
                    "variant": ("t" if ta else "n") + ("t" if tb else "n"),
                    "us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 2)})
    return {"tokens": T, "head_dim": D, "heads": H, "dtype": "f16",
            "total_us": round(total_t * 1e6, 2), "tflops": round(total_f / total_t / 1e12, 2),
            "per_product": per}


def epilogue_cost(dev, stream, reps):
    """The MLP up-projection (512 x 5632 x 2048, nt, fp16) with and without the
    fused bias + gelu epilogue: the epilogue's cost is the difference."""
    import torch

    import dense_gemm_amd as dg
    import synth
    M, N, K = 512, 5632, 2048
    st = synth.Stream(41)
    X = _dev_tensor(synth.round_to(st.normal((M, K)), "f16"), "f16", dev)
    W = _dev_tensor(synth.round_to(st.normal((N, K), 0.02), "f16"), "f16", dev)
    bias = _dev_tensor(synth.round_to(st.normal((N,), 0.5), "f16"), "f16", dev)
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    res = {"M": M, "N": N, "K": K, "variant": "nt", "dtype": "f16"}
    for name, bp, epi in (("plain", None, dg.DG_EPI_NONE), ("bias_gelu", bias.data_ptr(), dg.DG_EPI_GELU),
                          ("bias_relu", bias.data_ptr(), dg.DG_EPI_RELU)):
        def f(bp=bp, epi=epi):
            rc = dg.dg_gemm_ex(0, 1, M, N, K, 1.0, X.data_ptr(), K, 0, W.data_ptr(), K, 0, 0.0,
                               Y.data_ptr(), N, 0, 1, bp, epi, dg.DG_F16_F32ACC, stream.cuda_stream)
            if rc != 0:
                raise dg.GemmError(rc)

        for _ in range(10):
            f()
        torch.cuda.synchronize()
        t = min(time_launches(f, stream, reps) for _ in range(3))
        res[name + "_us"] = round(t * 1e6, 2)
    return res


def sgemm_512(dev, stream, reps):
    """SGEMM 512^3 nn, fp32, uniform[-1, 1) (seed 0): one launch's time, its
    fraction of the fp32 matrix peak, and every output against the oracle."""
    import torch

    import dense_gemm_amd as dg
    import oracle
    import synth
    S = 512
    a, b, _ = synth.problem(S, S, S, "f32", "uniform", 0)
    A, B = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    C = torch.empty((S, S), dtype=torch.float32, device=dev)
    k = dg.dg_select_kernel(0, 0, S, S, S, A.data_ptr(), S, B.data_ptr(), S, C.data_ptr(), S, dg.DG_F32)

    def f():
        rc = dg.dg_gemm(0, 0, S, S, S, 1.0, A.data_ptr(), S, B.data_ptr(), S, 0.0, C.data_ptr(), S,
                        dg.DG_F32, stream.cuda_stream)
        if rc != 0:
            raise dg.GemmError(rc)

    warm(f, 20)
    t = min(time_launches(f, stream, reps) for _ in range(3))
    ach = tflops(S, S, S, t)
    ref, ab = oracle.gemm(False, False, S, S, S, 1.0, a, S, b, S, 0.0, None, S)
    return {"workload": "SGEMM fp32 nn M=N=K=512 alpha=1 beta=0", "kernel": dg.dg_kernel_name(k),
            "kernel_us": round(t * 1e6, 2), "tflops": round(ach, 2), "frac": round(ach / PEAK_F32, 4),
            "per_launch_us": per_launch(f, stream, 50),
            "parity": oracle_check("f32", C.cpu().numpy(), ref, ab)}


def sgemm_ragged(dev, stream, reps):
    """The fp32 full-form workloads: C = 1.5 op(A) op(B) - 0.5 C with M, N, K
    = 4095, 4097, 1031 and 8192, 256, 8192, all four transpose pairs, every
    row stride padded by 8 (NaN in the padding), uniform[-1, 1) (seed 4).
    Per variant: the kernel, its time and fraction of the fp32 peak, and every
    output of one call from C0 against the oracle (one oracle run per shape:
    the variants share their logical operands)."""
    import numpy as np
    import torch

    import dense_gemm_amd as dg
    import oracle
    import synth
    alpha, beta = 1.5, -0.5
    out = {}
    for M, N, K in ((4095, 4097, 1031), (8192, 256, 8192)):
        a, b, c0 = synth.problem(M, N, K, "f32", "uniform", 4, with_c0=True)
        C0, ldc = synth.store(c0, False, N + 8)
        ref, ab = oracle.gemm(False, False, M, N, K, alpha, np.ascontiguousarray(a), K,
                              np.ascontiguousarray(b), N, beta, c0, N)
        res = {}
        for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
            sa, lda = synth.store(a, bool(ta), (M if ta else K) + 8)
            sb, ldb = synth.store(b, bool(tb), (K if tb else N) + 8)
            A, B = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
            Cd = torch.from_numpy(C0).to(dev)
            k = dg.dg_select_kernel(ta, tb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                    Cd.data_ptr(), ldc, dg.DG_F32)

            def f(ta=ta, tb=tb, A=A, B=B, C=Cd, lda=lda, ldb=ldb):
                rc = dg.dg_gemm(ta, tb, M, N, K, alpha, A.data_ptr(), lda, B.data_ptr(), ldb, beta,
                                C.data_ptr(), ldc, dg.DG_F32, stream.cuda_stream)
                if rc != 0:
                    raise dg.GemmError(rc)

            # one call from C0, checked; then the timed calls (which keep
            # updating C in place: C <- 1.5 AB - 0.5 C stays bounded)
            f()
            torch.cuda.synchronize()
            got = Cd.cpu().numpy()
            parity = oracle_check("f32", got[:, :N], ref, ab, alpha, beta, c0)
            # the stated bound taken literally, 2e-5 * sum_k |a_ik b_kj| + 1e-6,
            # without the alpha and beta terms
            parity["literal_max_err_over_bound"] = oracle_check("f32", got[:, :N], ref, ab)[
                "max_err_over_bound"]
            parity["c_padding_untouched"] = bool(np.isnan(got[:, N:]).all())
            warm(f, 5)
            t = min(time_launches(f, stream, reps) for _ in range(3))
            ach = tflops(M, N, K, t)
            res[("t" if ta else "n") + ("t" if tb else "n")] = {
                "kernel": dg.dg_kernel_name(k), "kernel_us": round(t * 1e6, 2),
                "tflops": round(ach, 2), "frac": round(ach / PEAK_F32, 4), "parity": parity}
            del A, B, Cd
        out[f"{M}x{N}x{K}"] = res
    return {"alpha": alpha, "beta": beta, "ld_pad": 8, **out}


def f16_k_sweep(dev, stream, reps):
    """fp16 M = N = 2048 over K = 64 .. 8192 (nn, tn, nt; the library's
    kernel, event-timed back to back): the launch's time splits into a part
    independent of K (launch, prologue, K-group sum, C stores) and a cost per
    64-deep K slab, read off as the slope between the two largest K."""
    import torch

    import dense_gemm_amd as dg
    S = 2048
    Ks = (64, 128, 256, 512, 1024, 2048, 4096, 8192)
    out = {}
    g = torch.Generator(device=dev).manual_seed(5)
    for name, ta, tb in (("nn", 0, 0), ("tn", 1, 0), ("nt", 0, 1)):
        us = {}
        for K in Ks:
            A = (torch.randn((K, S) if ta else (S, K), device=dev, generator=g) / 8).half()
            B = (torch.randn((S, K) if tb else (K, S), device=dev, generator=g) / 8).half()
            C = torch.empty((S, S), device=dev, dtype=torch.float16)
            lda, ldb = (S if ta else K), (K if tb else S)

            def f(ta=ta, tb=tb, K=K, A=A, B=B, C=C, lda=lda, ldb=ldb):
                rc = dg.dg_gemm(ta, tb, S, S, K, 1.0, A.data_ptr(), lda, B.data_ptr(), ldb, 0.0,
                                C.data_ptr(), S, dg.DG_F16_F32ACC, stream.cuda_stream)
                if rc != 0:
                    raise dg.GemmError(rc)

            warm(f, 20, 0.05)
            us[K] = round(min(time_launches(f, stream, reps) for _ in range(3)) * 1e6, 2)
        slab = (us[8192] - us[4096]) / ((8192 - 4096) // 64)
        out[name] = {"us_by_k": us, "us_per_slab": round(slab, 4),
                     "k_independent_us": round(us[2048] - slab * (2048 // 64), 2)}
    return out


def slab_probe(dev, stream, slabs=2000):
    """The slab probe (libdense_gemm_probe.so, dgp_slab_probe): one workgroup
    per CU doing the per-slab work of the fp16 2048^3 tile without its data
    flow -- per SIMD and slab 8 KB of direct loads into LDS, 16 KB of
    fragment reads from LDS and 16 MFMAs.  Per slab: shader cycles and
    nanoseconds, the medians over the workgroups of the first wave's
    s_memtime and s_memrealtime spans, from the second of two launches.
      l2        each combination of the parts, loading contiguous 32 KB
                windows of a 1 MiB source that stays in L2;
      patterns  loads alone and all three parts for load patterns between
                that and the GEMM's: contiguous or panel rows 4 KB apart (the
                row stride of K = 2048 fp16 operands), 1, 6 or 12 groups per
                XCD and slab (6 x 32 KB is the 2048^3 tiles' 192 KB of A and
                B panels per XCD and slab), from a source that fits L2 or a
                64 MiB one that fits only the Infinity Cache; all three
                parts also with one slab of loads in flight at each slab's
                start instead of two."""
    import statistics
    import torch

    import dense_gemm_amd.probe as pr

    sptr = stream.cuda_stream
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
    khz = pr.dgp_wall_clock_khz()
    L, M, R = pr.DGP_SLAB_LOADS, pr.DGP_SLAB_MFMA, pr.DGP_SLAB_READS

    def run(mode, windows, pitch, src):
        for _ in range(2):
            rc = pr.dgp_slab_probe(mode, wgs, slabs, windows, pitch, src.data_ptr(), src.numel() * 4,
                                   sink.data_ptr(), clocks.data_ptr(), sptr)
            if rc != 0:
                raise RuntimeError(f"dgp_slab_probe failed ({rc}, hip {pr.dgp_last_hip_error()})")
        torch.cuda.synchronize()
        c = clocks.view(wgs, 2).cpu().tolist()
        cyc = statistics.median(x for x, _ in c) / slabs
        ns = statistics.median(y for _, y in c) / slabs / khz * 1e6 if khz > 0 else None
        return {"cycles": round(cyc, 1), "ns": None if ns is None else round(ns, 1)}

    mib = 1 << 18                                                       # floats per MiB
    small = torch.ones(mib, dtype=torch.float32, device=dev)
    l2 = {name: run(mode, 1, 128, small) for name, mode in (
        ("loads", L), ("mfma", M), ("reads", R), ("loads+mfma", L | M), ("loads+reads", L | R),
        ("reads+mfma", R | M), ("loads+reads+mfma", L | R | M))}
    del small
    patterns = {}
    # (name, windows, pitch, MiB): 8 groups of 1 MiB at pitch 4 KB = one
    # fixed group per XCD, resident in its L2
    for name, windows, pitch, size in (("contiguous, 1 group, L2", 1, 128, 1),
                                       ("rows 4 KB apart, 1 group, L2", 1, 4096, 8),
                                       ("contiguous, 6 groups, 64 MiB", 6, 128, 64),
                                       ("rows 4 KB apart, 6 groups, 64 MiB", 6, 4096, 64),
                                       ("rows 4 KB apart, 12 groups, 64 MiB", 12, 4096, 64)):
        src = torch.ones(size * mib, dtype=torch.float32, device=dev)
        D = pr.DGP_SLAB_DEPTH1
        patterns[name] = {"loads": run(L, windows, pitch, src), "loads+reads+mfma": run(L | R | M, windows, pitch, src),
                          "loads+reads+mfma, one slab in flight": run(L | R | M | D, windows, pitch, src)}
        del src
    # the GEMM tiles' own loads: A and B panels of a 16 x 16 tile grid, the
    # nt operands of 2048 x 2048 x K, tiles dealt to XCDs in the library's
    # order, 1 .. 16 tile rows per group (the 128 x 128 kernel takes 4); the
    # source holds ones (half of the fp16 operands zero) unless stated
    gemm = {}
    T = int(round(wgs ** 0.5))
    if T * T == wgs:
        P = pr.DGP_SLAB_PANELS
        for K in (2048, 8192):
            src = torch.ones(2 * T * 128 * 2 * K // 4, dtype=torch.float32, device=dev)
            for gm in (1, 2, 4, 8, 16):
                if gm <= T:
                    gemm[f"K={K}, {gm} tile rows per group"] = run(L | R | M | P, gm, 2 * K, src)
            # the lanes of a row fetching its chunks in the GEMM's XOR order
            Z = pr.DGP_SLAB_SWIZZLE
            gemm[f"K={K}, 4 tile rows per group, swizzled lanes"] = run(L | R | M | P | Z, 4, 2 * K, src)
            # the same over random fp16 operands (as the GEMM's), which the
            # matrix cores multiply at a lower clock
            g = torch.Generator(device=dev).manual_seed(6)
            src.copy_((torch.randn(src.numel() * 2, device=dev, generator=g) / 8).half().view(torch.float32))
            gemm[f"K={K}, 4 tile rows per group, swizzled lanes, random fp16"] = run(L | R | M | P | Z, 4, 2 * K, src)
            del src
    return {"workgroups": wgs, "slabs": slabs, "mfma_cycles_per_slab_at_peak": 16 * 32,
            "cycles_per_slab_l2": l2, "cycles_per_slab_by_load_pattern": patterns,
            "gemm_tile_panels": gemm}


def under_profiler():
    """True when rocprofv3 runs this process (it exports ROCPROF_* variables).
    Its library is preloaded into every child process too, where it can set
    up the GPU before the child's own program starts; the amd-smi children
    are skipped then."""
    return any(k.startswith("ROCPROF_") for k in os.environ)


def smi_clocks(index=0):
    """Clock state from `amd-smi metric --clock --json` (a child process): the
    median current shader clock over the XCDs, its range, whether it is
    locked, and the memory clock.  None when the tool is missing or fails,
    or under a profiler.  The tool starts in about a second, so it sees the
    GPU idle between launches; the clock under load is the control probe's."""
    import subprocess
    if under_profiler():
        return None
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                           text=True, timeout=30)
        data = json.loads(r.stdout)
        gpus = data["gpu_data"] if isinstance(data, dict) else data
        clk = next(g for g in gpus if g.get("gpu") == index)["clock"]

        def val(x):
            return x["value"] if isinstance(x, dict) else None

        gfx = [val(v["clk"]) for k, v in clk.items() if k.startswith("gfx_")]
        gfx = sorted(x for x in gfx if x is not None)
        g0 = clk.get("gfx_0", {})
        mem = clk.get("mem_0", {})
        return {"gfx_mhz_median": gfx[len(gfx) // 2] if gfx else None,
                "gfx_min_mhz": val(g0.get("min_clk")), "gfx_max_mhz": val(g0.get("max_clk")),
                "gfx_locked": g0.get("clk_locked"), "mem_mhz": val(mem.get("clk"))}
    except Exception:
        return None


def parse_power_clock(text, index=0):
    """(socket power in W, median of the XCDs' current shader clocks in MHz)
    of GPU `index` from the JSON that `amd-smi metric --power --clock --json`
    prints, or None when either is missing."""
    import statistics
    try:
        data = json.loads(text)
    except ValueError:
        return None
    gpus = data["gpu_data"] if isinstance(data, dict) else data
    g = next((x for x in gpus if isinstance(x, dict) and x.get("gpu") == index), None)
    if g is None:
        return None
    pw = g.get("power", {}).get("socket_power", {})
    clk = [v["clk"]["value"] for k, v in g.get("clock", {}).items()
           if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
           and isinstance(v["clk"].get("value"), (int, float))]
    if not isinstance(pw, dict) or not isinstance(pw.get("value"), (int, float)) or not clk:
        return None
    return pw["value"], statistics.median(clk)


def power_under_load(fn, stream, seconds=4.0, skip=1.5, index=0):
    """Board power and shader clock while `fn` (one launch) runs back to back
    for `seconds`: `amd-smi metric --power --clock --json` in a child process,
    called again and again from a host thread (about 10 samples a second).
    The tool reports a window that lags the load by about a second, so
    samples from the first `skip` seconds are dropped.  Returns the medians
    of the socket power (W) and of the XCDs' current shader clocks (MHz), the
    sample count and the mean time per launch over the window, or None when
    the tool is missing or fails."""
    import statistics
    import subprocess
    import threading

    import torch
    samples = []
    stop = threading.Event()
    t0 = time.perf_counter()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"],
                                   capture_output=True, text=True, timeout=30)
            except Exception:
                return
            if time.perf_counter() - t0 < skip:
                continue
            pc = parse_power_clock(r.stdout, index)
            if pc is None:
                return
            samples.append(pc)

    th = threading.Thread(target=sampler)
    th.start()
    n = 0
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn()
        n += 50
        torch.cuda.synchronize()
    end.record(stream)
    end.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    return {"socket_power_w": statistics.median(p for p, _ in samples),
            "gfx_mhz": statistics.median(c for _, c in samples), "samples": len(samples),
            "us_per_launch": round(start.elapsed_time(end) * 1e3 / n, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-f16", action="store_true", help="skip the 16-bit measurements")
    ap.add_argument("--no-lora", action="store_true", help="skip the LoRA-step GEMM sequence")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the SGEMM 512^3 and ragged full-form legs")
    ap.add_argument("--k-sweep", action="store_true",
                    help="also time fp16 M=N=2048 over K = 64 .. 8192 (cost per K slab and "
                         "the K-independent part)")
    ap.add_argument("--no-aux", action="store_true",
                    help="skip the attention-heads and fused-epilogue legs")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the oracle checks of the timed outputs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache launches (for hardware-counter passes, whose "
                         "per-kernel averages would otherwise mix cold and warm launches)")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the board power and clock samples under sustained load")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 256 MiB device-to-device copy (a kernel of known traffic, "
                         "to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library is a single-GPU kernel library)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dense_gemm_amd as dg
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    # ---- inputs: generated and resident in device memory before any timing ----
    M = N = K = 4096
    a, b, _ = synth.problem(M, N, K, "f32", "uniform", 1)
    A = torch.from_numpy(a).to(dev)
    B = torch.from_numpy(b).to(dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    S = 2048
    a16, b16, _ = (None, None, None) if args.no_f16 else synth.problem(S, S, S, "f16", "normal_sqrtk", 2)
    torch.cuda.synchronize()

    smi_before = smi_clocks()
    control = control_probes(dev, stream)

    if args.copy_calibration:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- fp32 4096^3 nn: the step ------------------------------------------------
    kernel = dg.dg_select_kernel(0, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                                 dg.DG_F32)

    def step():
        rc = dg.dg_gemm(0, 0, M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C.data_ptr(),
                        N, dg.DG_F32, sptr)
        if rc != 0:
            raise dg.GemmError(rc)

    # W untimed steps, and at least 100 ms of them (the control probes above
    # keep the GPU busy up to here; the clock still settles under this load)
    warmup_launches = warm(step, args.warmup, 0.1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    launch_s = time_launches(step, stream, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    value = tflops(M, N, K, wall / args.steps)
    achieved = tflops(M, N, K, launch_s)
    f32_launches = per_launch(step, stream, 20)
    scrub = None if args.no_cold else torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=dev)
    f32_cold_us = None if args.no_cold else cold_launches(step, stream, 5, scrub)   # 512 MiB scrub
    smi_after = smi_clocks()

    out = {
        "metric": "TFLOP/s + % of MFMA peak: fp32 4096^3 nn; fp16->fp32 2048^3 nn/tn/nt",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches": warmup_launches,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (uniform[-1,1) fp32, seed 1, SplitMix64)",
        "config": {"workload": "SGEMM fp32 row-major nn M=N=K=4096 alpha=1 beta=0",
                   "M": M, "N": N, "K": K, "kernel": dg.dg_kernel_name(kernel)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_F32,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F32, 4),
                     "traffic": measured_traffic(kernel, 0, 0, M, N),
                     "traffic_source": TRAFFIC_SOURCE,
                     "algorithmic_bytes": 3 * M * N * 4, "kernel_ms": round(launch_s * 1e3, 4),
                     "frac_of_probe_peak": round(achieved / control["mfma_f32_tflops"], 4),
                     "probe_clock_mhz": control["mfma_f32_clock_mhz"]},
        "per_launch_us": f32_launches,
        "cold_us": f32_cold_us,
        "control": control,
        "smi_clocks": {"before": smi_before, "after_fp32": smi_after},
    }
    if not control["within_tolerance"]:
        out["gate"] = ("a control benchmark is more than 10% from its reference: "
                       "the figures of this line are not trusted")

    # ---- fp16 2048^3 nn / tn / nt ---------------------------------------------
    if not args.no_f16:
        res = {}
        outs = {}
        for name, ta, tb in (("nn", 0, 0), ("tn", 1, 0), ("nt", 0, 1)):
            As = torch.from_numpy(np.ascontiguousarray(a16.T if ta else a16)).to(dev)
            Bs = torch.from_numpy(np.ascontiguousarray(b16.T if tb else b16)).to(dev)
            Cs = torch.empty((S, S), dtype=torch.float16, device=dev)
            k16 = dg.dg_select_kernel(ta, tb, S, S, S, As.data_ptr(), S, Bs.data_ptr(), S,
                                      Cs.data_ptr(), S, dg.DG_F16_F32ACC)

            def step16(ta=ta, tb=tb, As=As, Bs=Bs, Cs=Cs):
                rc = dg.dg_gemm(ta, tb, S, S, S, 1.0, As.data_ptr(), S, Bs.data_ptr(), S, 0.0,
                                Cs.data_ptr(), S, dg.DG_F16_F32ACC, sptr)
                if rc != 0:
                    raise dg.GemmError(rc)

            warm(step16, 20, 0.1)
            reps = max(args.steps, 200)
            t16 = min(time_launches(step16, stream, reps) for _ in range(3))
            ach = tflops(S, S, S, t16)
            res[name] = {"tflops": round(ach, 2), "frac": round(ach / PEAK_F16, 4),
                         "frac_of_probe_peak": round(ach / control["mfma_f16_tflops"], 4),
                         # against the matrix cores alone on operands that change every
                         # instruction (the clock the part holds on such data)
                         "frac_of_random_operand_probe": round(ach / control["mfma_f16_random_tflops"], 4),
                         "kernel_us": round(t16 * 1e6, 2), "kernel": dg.dg_kernel_name(k16),
                         "traffic": measured_traffic(k16, ta, tb, S, S),
                         "algorithmic_bytes": 3 * S * S * 2,
                         "per_launch_us": per_launch(step16, stream, 100),
                         "cold_us": None if args.no_cold else cold_launches(step16, stream, 20, scrub)}
            torch.cuda.synchronize()
            outs[name] = Cs.float().cpu().numpy()
            del As, Bs, Cs
        if not args.no_check:
            # the variants share their logical operands: one oracle run
            import oracle
            ref, ab = oracle.gemm(False, False, S, S, S, 1.0, a16, S, b16, S, 0.0, None, S)
            for name in outs:
                res[name]["parity"] = oracle_check("f16", outs[name], ref, ab)
            del ref, ab
        out["fp16_2048"] = {"peak": PEAK_F16, "unit": "TFLOP/s", **res}
        del outs

    # ---- board power and shader clock under sustained load ---------------------
    # (the fp16 matrix rate on this workload's data is set by the power and
    # clock the part holds, not by the specification's 2.4 GHz)
    if not args.no_power and under_profiler():
        out["power"] = {"skipped": "under a profiler (its library is preloaded into the amd-smi "
                                   "child processes)"}
    elif not args.no_power:
        pw = {"source": "amd-smi metric --power --clock: socket power and the median of the XCDs' "
                        "shader clocks, medians over the samples of a 4 s window of back-to-back "
                        "launches after its first 1.5 s"}
        pw["fp32_4096_nn"] = power_under_load(step, stream)
        if not args.no_f16:
            An = torch.from_numpy(a16).to(dev)
            Bn = torch.from_numpy(b16).to(dev)
            Cn = torch.empty((S, S), dtype=torch.float16, device=dev)

            def step16nn():
                rc = dg.dg_gemm(0, 0, S, S, S, 1.0, An.data_ptr(), S, Bn.data_ptr(), S, 0.0,
                                Cn.data_ptr(), S, dg.DG_F16_F32ACC, sptr)
                if rc != 0:
                    raise dg.GemmError(rc)
            pw["fp16_2048_nn"] = power_under_load(step16nn, stream)
            del An, Bn, Cn
            import dense_gemm_amd.probe as pr
            wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
            sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
            clk = torch.zeros(wgs * 2, dtype=torch.int64, device=dev)
            for name, kind in (("mfma_f16_probe_random_operands", pr.DGP_MFMA_F16_RANDOM),
                               ("mfma_f16_probe_constant_operands", pr.DGP_MFMA_F16)):
                def pf(kind=kind):
                    rc = pr.dgp_mfma_peak(kind, wgs, 2000, sink.data_ptr(), clk.data_ptr(), sptr)
                    if rc != 0:
                        raise RuntimeError(f"dgp_mfma_peak failed ({rc})")
                pw[name] = power_under_load(pf, stream)
            del sink, clk
        out["power"] = pw

    # ---- bf16 2048^3 nn / tn / nt (same recipe as fp16) ------------------------
    if not args.no_f16:
        out["bf16_2048"] = bf16_square(dev, stream, max(args.steps, 200), not args.no_check)

    if args.k_sweep:
        out["f16_k_sweep"] = f16_k_sweep(dev, stream, 100)

    # ---- the fp16 tile's slab work without the GEMM (load path against MFMAs)
    if not args.no_f16:
        out["slab_probe"] = slab_probe(dev, stream)

    # ---- SGEMM 512^3 and the ragged full-form workloads -------------------------
    if not args.no_extra:
        out["sgemm_512"] = sgemm_512(dev, stream, max(args.steps, 200))
        out["sgemm_ragged"] = sgemm_ragged(dev, stream, max(args.steps // 2, 10))

    # ---- attention per-head products (strided batch over heads) ----------------
    if not args.no_f16 and not args.no_aux:
        out["attention_heads"] = attention_heads(dev, stream, max(args.steps, 50))

    # ---- fused epilogue on the MLP up-projection -----------------------------
    if not args.no_f16 and not args.no_aux:
        out["epilogue"] = epilogue_cost(dev, stream, max(args.steps, 100))

    # ---- LoRA MLP-block step: the 18 fp16 GEMMs of one forward + backward -------
    if not args.no_lora:
        out["lora_step"] = lora_step(dev, stream, max(args.steps, 20))
        out["lora_step_f32_out"] = lora_step(dev, stream, max(args.steps, 20), out="f32")
        out["lora_step_paired"] = lora_step_paired(dev, stream, max(args.steps, 20), not args.no_check)

    # ---- CPU baseline: the oracle on whole rows of the same problem -------------
    if not args.no_cpu:
        import oracle
        cores = oracle.default_threads()

        def oracle_rows(nrows):
            t = time.perf_counter()
            ref, ab = oracle.gemm(False, False, nrows, N, K, 1.0, a[:nrows], K, b, N, 0.0, None,
                                  N, nthreads=cores)
            return time.perf_counter() - t, ref, ab

        t_probe, _, _ = oracle_rows(cores)              # one row per thread
        nrows = cores * int(max(1, min(M // cores, args.cpu_seconds / max(t_probe, 1e-6))))
        t_cpu, ref, ab = oracle_rows(nrows)
        got = C[:nrows].cpu().numpy().astype(np.float64)
        worst, bad = oracle.compare("f32", got, ref, ab, 1.0, 0.0)
        flops = 2.0 * nrows * N * K
        out["cpu_baseline"] = {"value": round(flops / t_cpu / 1e12, 6), "unit": "TFLOP/s",
                               "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"rows 0..{nrows - 1} of C (all {N} columns, K={K}), "
                                         f"{t_cpu:.1f} s",
                               "sample_max_err_over_bound": round(worst, 4),
                               "sample_violations": bad}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
