"""Benchmark of the KDA forward scan on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload clip30s|clip5s|image4|packed8|tiny]
                [--no-backward] [--no-conv] [--no-shard] [--no-cpu-baseline] [--no-other-configs]
                [--no-state-step] [--copy-calib-mib M]

A step is one kda_forward call over the whole workload (every stage of the scan
runs inside it). The default workload is the 30-second clip: one sample of 189,272
tokens (512 text + a 121 x 30 x 52 latent grid), 16 heads, d_k = d_v = 128, bf16
data with fp32 states, the largest of the five configurations. Inputs are
generated once, copied to HBM, and the timed region holds exactly K back-to-back
steps between two device synchronisations. Inside the timed region the library
records HIP events on the launch stream around each of its kernels.

roofline: the scan must move 1,282 bytes per head-token (read q, k, v, log a and
beta once, write out once; bf16, d = 128) plus the fp32 final states. `achieved`
prices those bytes against the mean duration of the kernel with the largest time
per step; `path` prices them against the whole step. `traffic` is the kernel's
HBM bytes per launch from committed counter runs (profiles/), `traffic_ratio` that
over the algorithmic bytes.

The same line carries the other configurations' forward steps, the backward, the
short convolution and its backward, one GPU's share under a head or sequence
split, the step replayed from a HIP graph, single steps after a cache flush, the
serial state step of each scan kernel (state_step), the measured ceilings and the
oracle's CPU rate. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3
FP32_VECTOR_PEAK_TFLOPS = 157.3  # fp32 vector FMA, published (counts packed fp32 FMAs)
# fp32 vector FMA without packed ops (this build turns them off): 256 CUs x 4 SIMDs x 16 lanes
# x 2 flops x 2.4 GHz
FP32_VECTOR_UNPACKED_TFLOPS = 78.6
KERNEL_SOURCES = ["delta_rule_recurrent_kda_amd/csrc/kda_fused.hip",
                  "delta_rule_recurrent_kda_amd/csrc/kda_wy.hip",
                  "delta_rule_recurrent_kda_amd/csrc/kda_device.h",
                  "delta_rule_recurrent_kda_amd/csrc/kda_internal.h"]
BWD_SOURCES = ["delta_rule_recurrent_kda_amd/csrc/kda_bwd.hip",
               "delta_rule_recurrent_kda_amd/csrc/kda_device.h",
               "delta_rule_recurrent_kda_amd/csrc/kda_internal.h"]
CONV_SOURCES = ["delta_rule_recurrent_kda_amd/csrc/kda_conv.hip",
                "delta_rule_recurrent_kda_amd/csrc/kda_device.h",
                "delta_rule_recurrent_kda_amd/csrc/kda_internal.h"]
CONV_KERNELS = {"conv_plan": "kda_conv_plan_kernel", "conv": "kda_short_conv_kernel"}
CONV_BWD_KERNELS = {"conv_bwd_plan": "kda_conv_plan_kernel", "conv_dx": "kda_short_conv_kernel",
                    "conv_dw": "kda_short_conv_dw_kernel", "conv_dw_reduce": "kda_short_conv_dw_reduce_kernel"}
CONV_TAPS = (4, 3, 3, 3)        # text taps; visual frames x rows x columns
WORKLOADS = {"tiny": 0, "packed8": 1, "image4": 2, "clip5s": 3, "clip30s": 4}
CHUNK = 64
KERNEL_SYMBOL = {"fused": "kda_fused_kernel (output pass)", "fused_sum": "kda_fused_kernel (summary pass)",
                 "fused_combine": "kda_fused_combine_kernel", "plan": "kda_fused_plan_kernel",
                 "prep": "kda_wy_prep_kernel", "chain": "kda_wy_chain_kernel",
                 "segments": "kda_wy_chain_kernel", "scan": "kda_fwd"}
FUSED_C = 32                    # chunk of the fused scan (d_k = d_v = 128)


def kernel_sha(sources=None) -> str:
    """Hash of the sources a kernel is built from (the forward ones by default)."""
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES if sources is None else sources):
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(spec) -> int:
    """Bytes the scan must move: read q, k, v, log a, beta once, write out and final state."""
    es = 4 if spec.dtype == "f32" else 2
    T, H = spec.total_tokens, spec.heads
    return T * H * (3 * spec.dk + spec.dv) * es + T * H * es + T * H * spec.dv * es + \
        len(spec.seq_lens) * H * spec.dk * spec.dv * 4


def record_bytes(spec):
    """Per (64-token chunk, head) workspace record: (written by the prep, read by the chain).

    -W, Qh: 4 * d_k/32 fragments of 1 KB each; Kb^T: d_k/16 * 2 KB; P: 6 KB of used
    fragments; gamma: 4 d_k; U: d_v/16 * 2 KB. The chain reads the shared part once per
    (chunk, head) and U once in total over its value tiles.
    """
    dk, dv = spec.dk, spec.dv
    w = q = 4 * (dk // 32) * 1024
    kb = (dk // 16) * 2048
    return w + q + kb + 6 * 1024 + 4 * dk + (dv // 16) * 2048


def chunk_heads(spec) -> int:
    return sum((n + CHUNK - 1) // CHUNK for n in spec.seq_lens) * spec.heads


def split_plan(spec):
    """Sequence split of the library (same rule): chunks per segment (0 = none) and, over
    all samples, the chunks that lie in segments other than a sample's last one."""
    chunks = [(n + CHUNK - 1) // CHUNK for n in spec.seq_lens]
    bound = (spec.total_tokens + CHUNK - 1) // CHUNK
    lseg = 0
    if len(chunks) * spec.heads * (spec.dv // 64) <= 64:
        segs = max(1, 256 // (spec.heads * (spec.dv // 64)))
        cand = max(32, (bound + segs - 1) // segs)
        lseg = cand if cand < bound else 0
    if not lseg:
        return 0, 0, 0
    nsegs = [max(1, (c + lseg - 1) // lseg) for c in chunks]
    inner_segs = sum(s - 1 for s in nsegs)
    inner_chunks = sum(min(c, (s - 1) * lseg) for c, s in zip(chunks, nsegs))
    return lseg, inner_segs, inner_chunks


def fused_split(spec):
    """The fused scan's segment plan (the library's rule): chunks of 32 tokens per segment
    (0 = one segment per sample) and, over all samples, the chunks and the (segment, head)
    pairs of segments that are not their sample's last."""
    H = spec.heads
    chunks = (spec.total_tokens + FUSED_C - 1) // FUSED_C + len(spec.seq_lens)
    lseg = 0
    if len(spec.seq_lens) * H < 256:
        cand = max(16, (chunks * H + 255) // 256)
        lseg = cand if cand < chunks else 0
    if not lseg:
        return 0, 0, 0
    nch = [(n + FUSED_C - 1) // FUSED_C for n in spec.seq_lens]
    nsegs = [max(1, (c + lseg - 1) // lseg) for c in nch]
    inner_chunks = sum(min(c, (s - 1) * lseg) for c, s in zip(nch, nsegs))
    inner_segs = sum(s - 1 for s in nsegs)
    return lseg, inner_chunks, inner_segs


def fused_chunk_heads(spec, kernel: str) -> int:
    """(32-token chunk, head) steps one launch of a fused pass runs (0 for other kernels)."""
    if kernel == "fused":
        return sum((n + FUSED_C - 1) // FUSED_C for n in spec.seq_lens) * spec.heads
    if kernel == "fused_sum":
        return fused_split(spec)[1] * spec.heads
    return 0


def kernel_bytes(spec, kernel: str) -> int:
    """Algorithmic bytes of one launch of each kernel of the default bf16 scan."""
    es = 2
    T, H, N = spec.total_tokens, spec.heads, len(spec.seq_lens)
    dk, dv = spec.dk, spec.dv
    if kernel in ("fused", "fused_sum", "fused_combine"):
        _, inner_chunks, inner_segs = fused_split(spec)
        state = dk * dv * 4
        if kernel == "fused":       # every input once, out once, final states; entry states of segments
            return algorithmic_bytes(spec) + inner_segs * H * state
        inner_tok = min(T, inner_chunks * FUSED_C)
        if kernel == "fused_sum":   # k, v, log a, beta of inner segments; their local states and transitions
            return inner_tok * H * (2 * dk + dv + 1) * es + inner_segs * H * 2 * state
        return inner_segs * H * 3 * state       # combine: read S_loc and the transition, write S_in
    rec = chunk_heads(spec) * record_bytes(spec)
    _, inner_segs, inner_chunks = split_plan(spec)
    carry = inner_segs * H * (dk * dv + dk * dk) * 4       # S_loc and Phi of each inner segment
    if kernel == "prep":        # read q, k, v, log a, beta; write the records
        return T * H * (3 * dk + dv + 1) * es + rec
    if kernel == "chain":       # read the records (and the segment carries); write out and final state
        return rec + T * H * dv * es + N * H * dk * dv * 4 + carry
    if kernel == "segments":    # read the records of inner segments without Qh and P; write the carries
        used = record_bytes(spec) - 4 * (dk // 32) * 1024 - 6 * 1024
        return inner_chunks * H * used + carry
    if kernel == "plan":
        return 4 * (2 * N + 1)
    return algorithmic_bytes(spec)


BWD_C = 32
BWD_KERNELS = {"bwd_plan": "kda_bwd_plan_kernel", "bwd_prep": "kda_bwd_prep_kernel",
               "bwd_state_seg": "kda_bwd_state_kernel", "bwd_state": "kda_bwd_state_kernel",
               "bwd_dstate_seg": "kda_bwd_dstate_kernel", "bwd_dstate": "kda_bwd_dstate_kernel",
               "bwd_grad": "kda_bwd_grad_kernel"}


def bwd_split_chunks(spec) -> int:
    """Chunks (of 32 tokens) in samples that the backward chains split into several
    segments (the library's rule: at most 64 chain workgroups, segments of at least 64
    chunks); the first passes of the split walk exactly these."""
    chunks = [(n + BWD_C - 1) // BWD_C for n in spec.seq_lens]
    bound = (spec.total_tokens + BWD_C - 1) // BWD_C
    if len(chunks) * spec.heads * (spec.dv // 64) > 64:
        return 0
    segs = max(1, 256 // (spec.heads * (spec.dv // 64)))
    lseg = max(64, (bound + segs - 1) // segs)
    if lseg >= bound:
        return 0
    return sum(c for c in chunks if c > lseg)


def bwd_chunk_heads(spec) -> int:
    return sum((n + BWD_C - 1) // BWD_C for n in spec.seq_lens) * spec.heads


def bwd_kernel_macs(spec, kernel: str) -> int:
    """Multiply-adds of the matrix products of one launch (32-token chunks, fp32 MFMA)."""
    C, dk, dv = BWD_C, spec.dk, spec.dv
    per = {
        # X, dVn state term, dKbar, dQh and dKh state terms; Vn, dVn P term, dP, Z, dT and
        # the four chunk-internal products; dA (M and P come with the prep's record)
        "bwd_grad": 5 * C * dk * dv + 5 * C * C * dv + 4 * C * C * dk + 2 * C ** 3,
        "bwd_prep": 2 * C * C * dk,
        "bwd_state": 2 * C * dk * dv + C * C * dv,
        "bwd_dstate": 3 * C * dk * dv + 2 * C * C * dv,
    }.get(kernel, 0)
    if kernel == "bwd_state_seg":           # value tiles and the transition's d_k columns
        return (2 * C * dk + C * C) * (dv + dk) * bwd_split_chunks(spec) * spec.heads
    if kernel == "bwd_dstate_seg":
        return (3 * C * dk * dv + 2 * C * C * dv) * bwd_split_chunks(spec) * spec.heads
    return per * bwd_chunk_heads(spec)


def bwd_grad_mfma_floor_s(spec) -> float:
    """The least time the matrix cores need for one launch of the gradient kernel: on bf16
    data the five products with a state matrix (Kh S, Kc diag(gamma) dS', Vn dS'^T, dO S^T
    and dX S^T) and dO Vn^T, dVn X^T run on bf16 MFMA (three hi/lo terms, two where dO, exact
    as one bf16, is an operand), the products over tokens on fp32 MFMA; fp32 data runs every
    product on fp32 MFMA."""
    C, dk, dv = BWD_C, spec.dk, spec.dv
    ch = bwd_chunk_heads(spec)
    if spec.dtype != "bf16":
        return 2 * bwd_kernel_macs(spec, "bwd_grad") / (MFMA_F32_PEAK_TFLOPS * 1e12)
    f32_macs = (3 * C * C * dv + 4 * C * C * dk + 2 * C ** 3) * ch
    bf16_term_macs = ((3 + 3 + 3 + 2 + 3) * C * dk * dv + (2 + 3) * C * C * dv) * ch
    return 2 * f32_macs / (MFMA_F32_PEAK_TFLOPS * 1e12) + 2 * bf16_term_macs / (MFMA_BF16_PEAK_TFLOPS * 1e12)


def bwd_kernel_bytes(spec, kernel: str) -> int:
    """Algorithmic bytes of one launch of each backward kernel."""
    es = 4 if spec.dtype == "f32" else 2
    C, dk, dv, H, T = BWD_C, spec.dk, spec.dv, spec.heads, spec.total_tokens
    ch = bwd_chunk_heads(spec)
    state = ch * dk * dv * 4
    rec = ch * (3 * C * dk + 3 * C * C + dk + 3 * C) * 4     # Kh, Kc, Qh, T, P, M, gamma, b, 1/|q|, 1/|k|
    if kernel == "bwd_grad":    # the records, log a, v, dO; S and dS per chunk; five gradients
        return rec + T * H * (dk + 2 * dv) * es + 2 * state + T * H * (2 * dk + dk + dv + 1) * es
    if kernel == "bwd_prep":    # q, k, log a, beta; the records
        return T * H * (3 * dk + 1) * es + rec
    if kernel == "bwd_state":   # Kh, Kc, T, gamma, beta records and V; S per chunk
        return ch * (2 * C * dk + C * C + dk + C) * 4 + T * H * dv * es + state
    if kernel == "bwd_dstate":  # Kh, Kc, Qh, T, P, gamma, beta records and dO; dS per chunk
        return ch * (3 * C * dk + 2 * C * C + dk + C) * 4 + T * H * dv * es + state
    sc = bwd_split_chunks(spec) * H
    if kernel == "bwd_state_seg":   # Kh, Kc, T, gamma, beta records and V of split samples
        return sc * (2 * C * dk + C * C + dk + C) * 4 + sc * C * dv * es
    if kernel == "bwd_dstate_seg":  # all records and dO of split samples
        return sc * (3 * C * dk + 2 * C * C + dk + C) * 4 + sc * C * dv * es
    return 4 * (len(spec.seq_lens) + 1)


def chunk_flops(spec) -> int:
    """Dense chunk contractions per launch: 10*C*d + 6*d^2 per head-token (d = d_k = d_v)."""
    d = spec.dk
    return spec.head_tokens * (10 * CHUNK * d + 6 * d * d)


def traffic_for(workload: str, kernel: str, sha: str = None):
    """HBM bytes per launch of one kernel (by its timing name) from committed rocprofv3
    counter runs, if the kernel sources are unchanged since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha") != (kernel_sha() if sha is None else sha):
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """CPU model name and the number of processors the host reports."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count() or 1


def cpu_baseline(spec, a):
    """The fp64 oracle on the host cores over the whole workload (all samples, all heads): one
    thread per (sample, head) unit, at most 16 (the host share of one GPU)."""
    import oracle
    from delta_rule_recurrent_kda_amd import inputs
    model, nproc = host_cpu()
    units = len(spec.seq_lens) * spec.heads
    cores = max(1, min(16, units, nproc))
    f = {x: inputs.to_f64(a[x], spec.dtype) for x in ("q", "k", "v", "log_alpha", "beta")}
    oracle.build()
    t0 = time.perf_counter()
    oracle.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], a["cu_seqlens"], threads=cores)
    dt = time.perf_counter() - t0
    del f
    # one thread on one (sample, head) unit of the image workload, a rate that compares hosts
    s2 = inputs.config(WORKLOADS["image4"])
    a2 = inputs.generate(s2, heads=[0])
    L = s2.seq_lens[0]
    f2 = {x: inputs.to_f64(np.ascontiguousarray(a2[x][:L, :1]), s2.dtype) for x in ("q", "k", "v", "log_alpha", "beta")}
    t1 = time.perf_counter()
    oracle.forward(f2["q"], f2["k"], f2["v"], f2["log_alpha"], f2["beta"], np.array([0, L], np.int32), threads=1)
    d1 = time.perf_counter() - t1
    return {"value": spec.head_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "nproc": nproc, "cpu_model": model, "units": units,
            "sample": f"whole workload: {len(spec.seq_lens)} samples x {spec.heads} heads, "
                      f"{spec.head_tokens} head-tokens, fp64 token recurrence, {dt:.2f} s wall on {cores} threads",
            "single_thread": {"value": L / d1, "unit": "tokens/s", "cores": 1,
                              "sample": f"image workload, sample 0, head 0: {L} tokens, d = {s2.dk}, {d1:.3f} s"}}


def measured_ceilings(dev):
    """Rates this GPU reaches on plain work: 1 GiB device copies (read + write bytes), torch's and
    the probe library's grid-stride 16-byte copy at 4 and 8 workgroups per CU, the probe's
    read-only pass, and a 8192^3 bf16 matrix product (the vendor GEMM through torch, contiguous
    operands). bw_copy_GBs is the best copy."""
    import ctypes
    import torch
    from delta_rule_recurrent_kda_amd import build as kbuild
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    a = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    b = torch.randn((8192, 8192), device=dev).to(torch.bfloat16).contiguous()

    def timed(fn, reps):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    tc = timed(lambda: dst.copy_(src), 10)
    tg = timed(lambda: torch.matmul(a, b), 10)
    out = {"bw_torch_copy_GBs": 2 * n / tc / 1e9, "mfma_bf16_gemm_TFLOPs": 2 * 8192 ** 3 / tg / 1e12}
    probe = ctypes.CDLL(kbuild.PROBE_LIB)
    probe.kda_bw_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
    probe.kda_bw_probe.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev).cuda_stream
    for mode, key, factor in ((0, "bw_probe_copy_GBs", 2), (1, "bw_probe_read_GBs", 1)):
        best = 0.0
        for blocks in (1024, 2048):             # 4 and 8 workgroups per CU
            def run():
                if probe.kda_bw_probe(mode, src.data_ptr(), dst.data_ptr(), n, blocks, stream) != 0:
                    raise RuntimeError("bandwidth probe launch failed")
            best = max(best, factor * n / timed(run, 10) / 1e9)
        out[key] = best
    out["bw_copy_GBs"] = max(out["bw_torch_copy_GBs"], out["bw_probe_copy_GBs"])
    del src, dst, a, b
    return out


def graph_steps(step, n: int) -> float:
    """ms per step when the step is captured once in a HIP graph and replayed n times back to
    back (the same kernels without the host's launch work)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(n):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - w0) * 1e3 / n


def flushed_steps(step, stream, dev, n: int) -> float:
    """Median duration (ms) of single steps, each after a 512 MiB write that evicts the caches."""
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    times = []
    for _ in range(n):
        scratch.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(times))


def backward_bench(args, spec, t, cu, dev):
    """The gradient step (kda_backward) on the same workload: K timed steps after W warm-ups."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    d_out = torch.randn(t["v"].shape, device=dev, generator=g).to(t["v"].dtype)

    def step():
        kda.backward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], cu, d_out, with_initial_grad=False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for name in BWD_KERNELS:
        kda.timing_read(name)
    kda.timing_enable(True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kda.timing_enable(False)
    kernels = {}
    for name in BWD_KERNELS:
        n, ms = kda.timing_read(name)
        if n:
            macs, b = bwd_kernel_macs(spec, name), bwd_kernel_bytes(spec, name)
            sec = ms / n * 1e-3
            kernels[name] = {"launches": n, "ms_avg": ms / n, "flops": 2 * macs,
                             "achieved_TFLOPs": 2 * macs / sec / 1e12, "algorithmic_bytes": b,
                             "achieved_GBs": b / sec / 1e9}
    dom = max(kernels, key=lambda k: kernels[k]["ms_avg"])
    kd = kernels[dom]
    ms_step = wall * 1e3 / args.steps
    # the matrix cores' peak for the dominant kernel's mix of fp32 and bf16 products: its
    # algorithmic flops over the least time the mix needs
    peak = MFMA_F32_PEAK_TFLOPS
    peak_note = "fp32 MFMA peak"
    if dom == "bwd_grad":
        peak = kd["flops"] / bwd_grad_mfma_floor_s(spec) / 1e12
        if spec.dtype == "bf16":
            peak_note = ("the kernel's mix: algorithmic flops over (fp32-product flops / 157.3 TFLOP/s + bf16 "
                         "hi/lo term flops / 2,500 TFLOP/s), so frac = that floor time / the kernel's time")
    return {"metric": "KDA backward head-tokens/s (gradients of q, k, v, log a, beta)",
            "value": spec.head_tokens / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step,
            "dtype": "f32 arithmetic on " + spec.dtype + " data (fp32 MFMA; on bf16 data the two chains and the "
                     "gradient kernel's products with the state and over value columns take hi/lo bf16 MFMA "
                     "terms)",
            "roofline": {"bound": "mfma", "achieved": kd["achieved_TFLOPs"], "peak": peak,
                         "peak_note": peak_note,
                         "unit": "TFLOP/s", "frac": kd["achieved_TFLOPs"] / peak,
                         "traffic": traffic_for(args.workload, BWD_KERNELS[dom], kernel_sha(BWD_SOURCES)),
                         "kernel": BWD_KERNELS[dom], "kernel_ms_avg": kd["ms_avg"],
                         "flops": kd["flops"], "algorithmic_bytes": kd["algorithmic_bytes"],
                         "kernel_sha": kernel_sha(BWD_SOURCES)},
            "kernels": kernels}


def conv_bench(args, spec, dev):
    """The modality-aware short convolution over heads x d_k channels of one packed batch.

    The layout is the workload's (text prefix + latent grid per sample) when it has a grid,
    else the 5-second clip (512 text tokens + a 21 x 30 x 52 grid). A step is one
    kda_short_conv call; K timed steps after W warm-ups, HIP events around each kernel.
    """
    import torch
    from delta_rule_recurrent_kda_amd import inputs, kda
    cs = spec if spec.grid is not None else inputs.config(WORKLOADS["clip5s"])
    C = cs.heads * cs.dk
    n = len(cs.seq_lens)
    T = cs.total_tokens
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    x = torch.randn((T, C), device=dev, generator=g).to(torch.bfloat16)
    wt = torch.randn((CONV_TAPS[0], C), device=dev, generator=g) * 0.5
    wv = torch.randn((*CONV_TAPS[1:], C), device=dev, generator=g) * 0.3
    cu = torch.from_numpy(cs.cu_seqlens()).to(dev)
    tl = torch.tensor(list(cs.text_tokens), dtype=torch.int32, device=dev)
    gr = torch.tensor([list(cs.grid)] * n, dtype=torch.int32, device=dev)
    y = torch.empty_like(x)

    def step():
        kda.short_conv(x, wt, wv, cu, tl, gr, y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for name in CONV_KERNELS:
        kda.timing_read(name)
    kda.timing_enable(True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kda.timing_enable(False)
    kernels = {}
    for name in CONV_KERNELS:
        k, ms = kda.timing_read(name)
        if k:
            kernels[name] = {"launches": k, "ms_avg": ms / k}
    ms_step = wall * 1e3 / args.steps
    text = int(sum(cs.text_tokens))
    vis = T - text
    taps = CONV_TAPS[1] * CONV_TAPS[2] * CONV_TAPS[3]
    flops = 2 * C * (vis * taps + text * CONV_TAPS[0])     # one FMA per tap and output element
    nbytes = 2 * T * C * 2 + (CONV_TAPS[0] + taps) * C * 4  # read x, write y (bf16), weights
    kms = kernels["conv"]["ms_avg"]
    tflops = flops / (kms * 1e-3) / 1e12
    gbs = nbytes / (kms * 1e-3) / 1e9
    sha = kernel_sha(CONV_SOURCES)
    bwd = conv_backward_bench(args, x, wt, wv, cu, tl, gr, flops, nbytes, sha, cs.name.split("-")[0])
    return {"metric": "short convolution tokens/s (depthwise over heads x d_k channels)",
            "value": T / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step,
            "dtype": "f32 arithmetic on bf16 data",
            "config": {"workload": cs.name, "tokens": T, "channels": C, "text_taps": CONV_TAPS[0],
                       "visual_kernel": list(CONV_TAPS[1:])},
            "roofline": {"bound": "alu", "achieved": tflops, "peak": FP32_VECTOR_UNPACKED_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / FP32_VECTOR_UNPACKED_TFLOPS,
                         "peak_published": FP32_VECTOR_PEAK_TFLOPS, "frac_published": tflops / FP32_VECTOR_PEAK_TFLOPS,
                         "peak_note": "78.6 = 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz, fp32 FMA without "
                                      "packed ops (off in this build); 157.3 is the published figure with them",
                         "traffic": traffic_for(cs.name.split("-")[0], CONV_KERNELS["conv"], sha),
                         "kernel": CONV_KERNELS["conv"], "kernel_ms_avg": kms, "flops": flops,
                         "kernel_sha": sha},
            "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                    "algorithmic_bytes": nbytes},
            "kernels": kernels,
            "backward": bwd}


def conv_backward_bench(args, x, wt, wv, cu, tl, gr, fwd_flops, fwd_bytes, sha, workload):
    """kda_short_conv_backward on the same inputs (dy random bf16): dx and both weight gradients.

    dx is the forward's arithmetic on dy (same FLOPs and bytes); the weight gradients do the
    same FMAs again (one per tap and output element) reading x and dy, plus a small partial-sum
    buffer. The roofline entry is the dominant kernel against the fp32 vector peak."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    g = torch.Generator(device=x.device)
    g.manual_seed(8765)
    dy = torch.randn(x.shape, device=x.device, generator=g).to(x.dtype)
    dx = torch.empty_like(x)
    dwt = torch.empty_like(wt)
    dwv = torch.empty_like(wv)

    def step():
        kda.short_conv_backward(x, wt, wv, cu, tl, gr, dy, dx, dwt, dwv)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for name in CONV_BWD_KERNELS:
        kda.timing_read(name)
    kda.timing_enable(True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kda.timing_enable(False)
    work = {"conv_dx": (fwd_flops, fwd_bytes), "conv_dw": (fwd_flops, fwd_bytes)}
    kernels = {}
    for name in CONV_BWD_KERNELS:
        k, ms = kda.timing_read(name)
        if k:
            kernels[name] = {"launches": k, "ms_avg": ms / k}
            if name in work:
                f, b = work[name]
                sec = ms / k * 1e-3
                kernels[name].update({"flops": f, "achieved_TFLOPs": f / sec / 1e12, "algorithmic_bytes": b,
                                      "achieved_GBs": b / sec / 1e9})
    dom = max(work, key=lambda n: kernels[n]["ms_avg"])
    kd = kernels[dom]
    ms_step = wall * 1e3 / args.steps
    return {"metric": "short convolution backward tokens/s (dx, dw_text, dw_vis)",
            "value": x.shape[0] / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step,
            "dtype": "f32 arithmetic on bf16 data",
            "roofline": {"bound": "alu", "achieved": kd["achieved_TFLOPs"], "peak": FP32_VECTOR_UNPACKED_TFLOPS,
                         "unit": "TFLOP/s", "frac": kd["achieved_TFLOPs"] / FP32_VECTOR_UNPACKED_TFLOPS,
                         "peak_published": FP32_VECTOR_PEAK_TFLOPS,
                         "frac_published": kd["achieved_TFLOPs"] / FP32_VECTOR_PEAK_TFLOPS,
                         "traffic": traffic_for(workload, CONV_BWD_KERNELS[dom], sha),
                         "kernel": CONV_BWD_KERNELS[dom], "kernel_ms_avg": kd["ms_avg"], "flops": kd["flops"],
                         "kernel_sha": sha},
            "kernels": kernels}


def shard_bench(args, dev):
    """One GPU's share of the 30-second clip (config 4: 189,272 tokens, 16 heads, d = 128) under the
    two splits the scan allows across GPUs, timed at its real shape:
    - head split over 8 GPUs: the whole sequence with 2 of the 16 heads (no exchange);
    - sequence split over 8 GPUs: one eighth of the tokens (23,659) with all 16 heads, scanned from
      an initial state (kda_forward_from_state), as each GPU would after the all-gather of the
      segment summaries.
    Inputs are drawn on the device with the workload's distributions (q, k unit length, v ~ N(0,1),
    log a ~ -U(0.0005, 0.05), beta = sigmoid(N(0,1))); K timed steps after W warm-ups."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    g = torch.Generator(device=dev)
    g.manual_seed(2468)

    def draw(T, H, d=128):
        q = torch.nn.functional.normalize(torch.randn((T, H, d), device=dev, generator=g), dim=-1)
        k = torch.nn.functional.normalize(torch.randn((T, H, d), device=dev, generator=g), dim=-1)
        v = torch.randn((T, H, d), device=dev, generator=g)
        la = -(0.0005 + 0.0495 * torch.rand((T, H, d), device=dev, generator=g))
        b = torch.sigmoid(torch.randn((T, H), device=dev, generator=g))
        return [t.to(torch.bfloat16).contiguous() for t in (q, k, v, la, b)]

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - w0) * 1e3 / args.steps

    out = {}
    T = 512 + 121 * 30 * 52
    q, k, v, la, b = draw(T, 2)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    o = torch.empty_like(v)
    fs = torch.empty((1, 2, 128, 128), dtype=torch.float32, device=dev)
    ms = timed(lambda: kda.kda_forward(q, k, v, la, b, cu, o, fs))
    out["head_split_8"] = {"tokens": T, "heads": 2, "ms_per_step": ms, "value": T * 2 / (ms * 1e-3),
                           "unit": "tokens/s"}
    del q, k, v, la, b, o
    Ts = (T + 7) // 8
    q, k, v, la, b = draw(Ts, 16)
    cu = torch.tensor([0, Ts], dtype=torch.int32, device=dev)
    s0 = 0.05 * torch.randn((1, 16, 128, 128), device=dev, generator=g)
    o = torch.empty_like(v)
    fs = torch.empty((1, 16, 128, 128), dtype=torch.float32, device=dev)
    ms = timed(lambda: kda.kda_forward(q, k, v, la, b, cu, o, fs, initial_state=s0))
    out["sequence_split_8"] = {"tokens": Ts, "heads": 16, "ms_per_step": ms, "value": Ts * 16 / (ms * 1e-3),
                               "unit": "tokens/s", "initial_state": True}
    out["note"] = ("one GPU's share of config 4 (189,272 tokens x 16 heads) under an 8-way head or sequence split; "
                   "the sequence split also needs the all-gather of the segment summaries and their prefix, not timed")
    return out


def state_step(args, dev):
    """The serial state step of each scan kernel: packs of 256 samples x 1 head (one (sample,
    head) unit per CU, so no sequence split) at two sample lengths; a kernel's step is its
    mean launch time over the chunks one unit walks. Every CU runs a unit, so the step
    includes its share of HBM."""
    import torch
    from delta_rule_recurrent_kda_amd import inputs, kda
    lens = (2048, 8192)
    # (timing name, scan variant or "bwd", tokens per step)
    kinds = (("fused", None, 32), ("chain", "wy", 64), ("bwd_state", "bwd", 32), ("bwd_dstate", "bwd", 32))
    ms = {name: [] for name, _, _ in kinds}
    for L in lens:
        spec = inputs.custom([L] * 256, heads=1, d=128, seed=31)
        a = inputs.generate(spec)
        t = device_tensors(spec, a, dev)
        cu = torch.from_numpy(a["cu_seqlens"]).to(dev)
        for variant in (None, "wy"):
            if variant:
                os.environ["KDA_SCAN_VARIANT"] = variant
            try:
                _, kern, _ = forward_timing(spec, t, cu, dev, 5, 2)
            finally:
                os.environ.pop("KDA_SCAN_VARIANT", None)
            for name, var, _ in kinds:
                if var == variant and name in kern:
                    ms[name].append(kern[name]["ms_avg"])
        g = torch.Generator(device=dev)
        g.manual_seed(77)
        d_out = torch.randn(t["v"].shape, device=dev, generator=g).to(t["v"].dtype)
        for _ in range(2):
            kda.backward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], cu, d_out, with_initial_grad=False)
        torch.cuda.synchronize()
        for name in BWD_KERNELS:
            kda.timing_read(name)
        kda.timing_enable(True)
        for _ in range(3):
            kda.backward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], cu, d_out, with_initial_grad=False)
        torch.cuda.synchronize()
        kda.timing_enable(False)
        for name in ("bwd_state", "bwd_dstate"):
            n, tot = kda.timing_read(name)
            if n:
                ms[name].append(tot / n)
        del t, d_out
        torch.cuda.empty_cache()
    out = {}
    for name, _, tok in kinds:
        if len(ms[name]) != len(lens):
            continue
        out[name] = {"tokens_per_step": tok,
                     "us_per_step": {str(L): m * 1e3 / (L // tok) for L, m in zip(lens, ms[name])},
                     "launch_ms": {str(L): m for L, m in zip(lens, ms[name])}}
    out["note"] = ("256 samples x 1 head, d = 128, bf16, samples of 2,048 and 8,192 tokens (one unit per CU, no "
                   "sequence split); us_per_step = a kernel's mean launch time over the steps one unit walks, fill "
                   "and drain included. fused: the fused scan (32-token chunks, 8 waves per CU); chain: the WY "
                   "scan's chain (64-token chunks); bwd_state, bwd_dstate: the backward's two chains per 64-column "
                   "tile (32-token chunks), which run side by side on two streams and share the CUs")
    return out


def device_tensors(spec, a, dev):
    import torch
    t = {}
    for name in ("q", "k", "v", "log_alpha", "beta"):
        arr = a[name]
        t[name] = (torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16) if spec.dtype == "bf16"
                   else torch.from_numpy(arr)).to(dev)
    return t


def forward_timing(spec, t, cu, dev, steps, warmup):
    """W warm-ups, then K back-to-back forward steps between two synchronisations with the
    library's per-kernel HIP events on; returns (ms per step, per-kernel records, step fn)."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    out = torch.empty((spec.total_tokens, spec.heads, spec.dv), dtype=t["q"].dtype, device=dev)
    fs = torch.empty((len(spec.seq_lens), spec.heads, spec.dk, spec.dv), dtype=torch.float32, device=dev)

    def step():     # on torch's current stream: the default stream, or the capture stream of a graph
        kda.kda_forward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], cu, out, fs,
                        stream=torch.cuda.current_stream(dev))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    for name in KERNEL_SYMBOL:
        kda.timing_read(name)
    kda.timing_enable(True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kda.timing_enable(False)
    # a kernel may run several times per step: its launches share the step's bytes
    kernels = {}
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for name in KERNEL_SYMBOL:
        n, ms = kda.timing_read(name)
        if n:
            per_step = n / steps
            b = kernel_bytes(spec, name) / per_step
            kernels[name] = {"launches": n, "launches_per_step": per_step, "ms_avg": ms / n,
                             "ms_per_step": ms / steps, "algorithmic_bytes": b,
                             "achieved_GBs": b / (ms / n * 1e-3) / 1e9}
            ch = fused_chunk_heads(spec, name)
            if ch:
                # the serial state step as the pass runs it: one CU's time per 32-token chunk
                # (the launch's time spread over its chunk-heads, one workgroup per CU)
                kernels[name]["chunk_heads"] = ch
                kernels[name]["us_per_chunk_step"] = ms / n * 1e3 * cus / ch
    return wall * 1e3 / steps, kernels, step


def other_configs(args, dev):
    """Forward steps of the other bf16 configurations (parity cases of the same scan), each
    timed like the headline: K steps after W warm-ups."""
    import torch
    from delta_rule_recurrent_kda_amd import inputs
    res = {}
    for wl, cfg in WORKLOADS.items():
        if wl == args.workload or cfg == 0:
            continue
        spec = inputs.config(cfg)
        a = inputs.generate(spec)
        t = device_tensors(spec, a, dev)
        cu = torch.from_numpy(a["cu_seqlens"]).to(dev)
        ms, kernels, _ = forward_timing(spec, t, cu, dev, args.steps, args.warmup)
        b = algorithmic_bytes(spec)
        res[wl] = {"workload": spec.name, "head_tokens": spec.head_tokens, "ms_per_step": ms,
                   "value": spec.head_tokens / (ms * 1e-3), "unit": "tokens/s", "algorithmic_bytes": b,
                   "path_frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                   "kernels": {k: v["ms_avg"] for k, v in kernels.items()}}
        del t
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="clip30s", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-shard", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--no-state-step", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after timing, run 3 plain device copies of this many MiB (for scaling "
                         "HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the scan shards by (sample, head) with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    import torch
    from delta_rule_recurrent_kda_amd import inputs

    spec = inputs.config(WORKLOADS[args.workload])
    a = inputs.generate(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = device_tensors(spec, a, dev)
    cu = torch.from_numpy(a["cu_seqlens"]).to(dev)
    stream = torch.cuda.current_stream(dev)

    ms_per_step, kernels, step = forward_timing(spec, t, cu, dev, args.steps, args.warmup)
    flushed = flushed_steps(step, stream, dev, 20)
    graph_ms = graph_steps(step, args.steps)
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom_ms = kernels[dom]["ms_avg"]

    bytes_ = algorithmic_bytes(spec)
    flops = chunk_flops(spec)
    # the dominant kernel's own algorithmic bytes per launch (what its launch must read and
    # write at the least, from the same per-head-token figures) over its mean launch time
    dom_bytes = kernels[dom].get("algorithmic_bytes", bytes_ / kernels[dom]["launches_per_step"])
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    path_gbs = bytes_ / (ms_per_step * 1e-3) / 1e9
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if spec.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    traffic = traffic_for(args.workload, dom)

    rec = {
        "metric": "KDA fwd tokens/s (B·L·H) at dk=dv=128; % MFMA peak and % HBM BW, 1 MI355X",
        "value": spec.head_tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "samples": len(spec.seq_lens), "tokens": spec.total_tokens,
                   "heads": spec.heads, "d_k": spec.dk, "d_v": spec.dv, "head_tokens": spec.head_tokens},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_ratio": None if traffic is None else traffic / dom_bytes,
                     "kernel": KERNEL_SYMBOL[dom], "kernel_ms_avg": dom_ms, "algorithmic_bytes": dom_bytes,
                     "algorithmic_bytes_note": "the dominant kernel's own bytes: per head-token it covers, "
                                               "256 B each of q, k, v, log a read, 2 B of beta, 256 B of out "
                                               "written (those of its pass), plus its state traffic; the path "
                                               "as a whole is 1,282 B per head-token (see path)",
                     "kernel_sha": kernel_sha()},
        "kernels": kernels,
        "path": {"algorithmic_bytes": bytes_, "achieved_GBs": path_gbs, "frac_hbm": path_gbs / HBM_PEAK_GBS},
        "graph": {"ms_per_step": graph_ms, "value": spec.head_tokens / (graph_ms * 1e-3),
                  "note": "the same step captured once in a HIP graph and replayed K times back to back"},
        "flushed": {"ms_per_step_median": flushed, "value": spec.head_tokens / (flushed * 1e-3),
                    "note": "one step at a time after writing 512 MiB (evicts L2 and the 256 MB Infinity "
                            "Cache); HIP events on the launch stream around the step only"},
        "mfma": {"achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s", "frac": tflops / mfma_peak,
                 "flops_per_launch": flops},
    }
    ceil = measured_ceilings(dev)
    ceil.update({"roofline_frac_of_copy": achieved / ceil["bw_copy_GBs"],
                 "path_frac_of_copy": path_gbs / ceil["bw_copy_GBs"],
                 "mfma_frac_of_gemm": tflops / ceil["mfma_bf16_gemm_TFLOPs"]})
    rec["measured_ceilings"] = ceil
    if not args.no_backward:
        rec["backward"] = backward_bench(args, spec, t, cu, dev)
    if not args.no_other_configs:
        rec["other_configs"] = other_configs(args, dev)
    if not args.no_conv:
        rec["short_conv"] = conv_bench(args, spec, dev)
    if not args.no_shard:
        rec["shard"] = shard_bench(args, dev)
    if not args.no_state_step:
        rec["state_step"] = state_step(args, dev)
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calib_bytes"] = n
    if not args.no_cpu_baseline:
        del t
        torch.cuda.empty_cache()
        rec["cpu_baseline"] = cpu_baseline(spec, a)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
