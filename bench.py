#!/usr/bin/env python3
"""Benchmark of the grouped 4-bit expert GEMM on one MI355X.

Default workload (`--workload headline`): the Mixtral-8x7B configuration, the
largest single-GPU one, w1/w3 fused in NF4 (E=8 experts, K=4096, N=28672,
top-2 over 4096 tokens: M=8192 routed rows). One step = the prefill forward
GEMM, its input gradient (dgrad) on the same packed weights, and one decode
call of every configured token-decode case (OLMoE, Qwen3 gate_up and down,
gpt-oss gate_up and down at T=1; Qwen3 gate_up and down at T=64). Inputs are
seeded synthetic draws of the workloads' shapes and distributions, resident in
HBM before timing; every weight stack rotates over enough copies (>2.5 GB)
that no launch finds its weights in the 256 MB Infinity Cache.

Prints ONE JSON line:
  value      prefill TFLOP/s of the Mixtral w1/w3 forward call (2*M*N*K over
             routed rows / call time, HIP-graph timed); the dgrad leg beside it
  decode     packed-weight GB/s of each decode case (codes + scales of touched
             experts / call time) beside a plain device copy of the same bytes
  roofline   the dominant kernel of the step (the longer of the forward and the
             dgrad tiled kernels): algorithmic flops per launch over the kernel's
             own time from two HIP events the library records around it on the
             launch stream; beside it the profiler's mean of the same kernel, the
             clock it ran at and the peak at that clock, from profiles/kernels.json
             when that file matches the kernel sources
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same case

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]

Other workloads time one configuration's prefill and decode calls (olmoe,
qwen3, ...), the fused expert block (*_block), the adapter step (olmoe_lora),
the W4A8 variant (*_w4a8), or every decode path on the headline decode cases
(decode_paths: vector, narrow, skinny with K split 1, 2, 4 and 8 ways).
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

METRIC = "grouped 4-bit GEMM TFLOP/s (prefill) + packed-weight HBM GB/s (decode), 1 GPU"
PEAK_MFMA_TFLOPS = 256 * 2.4e9 * 4096 / 1e12     # dense fp16/bf16 MFMA, 2516.6
PEAK_FP8_TFLOPS = 2 * PEAK_MFMA_TFLOPS   # dense fp8 MFMA (fp8 x fp4 runs at the fp8 rate): 5.0 PFLOP/s published
PEAK_HBM_GBPS = 8000.0
ROTATE_BYTES = 2.5e9

WORKLOADS = {
    "olmoe": ("olmoe_gate_up_t2048", "olmoe_gate_up_t1"),
    "qwen3": ("qwen3_gate_up_t4096", "qwen3_gate_up_t1"),
    "qwen3_down": ("qwen3_down_t4096", "qwen3_down_t1"),
    "gptoss": ("gptoss_gate_up_t2048", "gptoss_gate_up_t1"),
    "gptoss_down": ("gptoss_down_t2048", "gptoss_down_t1"),
    "mixtral": ("mixtral_w13_t4096", None),
    "mixtral_w2": ("mixtral_w2_t4096", None),
    "mixtral_dgrad": ("mixtral_dgrad_w13", None),
    "mixtral_dgrad_w2": ("mixtral_dgrad_w2", None),
    "gptoss_dgrad": ("gptoss_dgrad_gate_up", None),
    # W4A8: activations quantised to MXFP8 on the device, block-scaled fp8 x fp4 MFMA
    "gptoss_w4a8": ("gptoss_gate_up_t2048", None),
    "gptoss_down_w4a8": ("gptoss_down_t2048", None),
    # decode-class only (no prefill leg): value is packed-weight GB/s
    "qwen3_t64": (None, "qwen3_gate_up_t64"),
    "qwen3_down_t64": (None, "qwen3_down_t64"),
}
# Fused expert block (gate_up -> SwiGLU -> down in one call): the gate_up and down
# cases of one model share their routing; (prefill gate_up, prefill down, decode
# gate_up, decode down).
W4A8_WORKLOADS = {"gptoss_w4a8", "gptoss_down_w4a8"}
# Low-rank adapter (rank, scale) on the grouped projection: forward with the delta
# fused into the tiled kernel's epilogue, backward with dgrad + adapter gradients.
LORA_WORKLOADS = {"olmoe_lora": ("olmoe_gate_up_t2048", 16, 2.0)}
BLOCK_WORKLOADS = {
    "qwen3_block": ("qwen3_gate_up_t4096", "qwen3_down_t4096", "qwen3_gate_up_t1", "qwen3_down_t1"),
    "gptoss_block": ("gptoss_gate_up_t2048", "gptoss_down_t2048", "gptoss_gate_up_t1", "gptoss_down_t1"),
}
KERNEL_SOURCES = ["geg_device.hpp", "geg_launch.hpp", "tile.hip", "skinny.hip", "vec.hip", "narrow.hip", "route.hip",
                  "w4a8.hip", "lora.hip", "util.hip",
                  "geg.cpp"]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "grouped_expert_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def make_inputs(c, seed, torch, geg, dev):
    """Activations, sizes and packed weights of one case on the device."""
    import synthetic
    a_bits, sizes = synthetic.rows_bf16(c, seed)
    a = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    sz = torch.from_numpy(sizes).to(dev)
    codes = torch.empty((c.E, c.N, c.K // 2), dtype=torch.uint8, device=dev)
    if c.fmt == "nf4":
        scales = torch.empty((c.E, c.N, c.K // 64), dtype=torch.float32, device=dev)
        for e in range(c.E):
            w = torch.from_numpy(synthetic.nf4_weight_f32(c, seed, e)).to(dev)
            q, s = geg.gnf4_quantize(w)
            codes[e].copy_(q)
            scales[e].copy_(s)
            del w, q, s
    else:
        scales = torch.empty((c.E, c.N, c.K // 32), dtype=torch.uint8, device=dev)
        for e in range(c.E):
            q, s = synthetic.mxfp4_bytes(c, seed, e)
            codes[e].copy_(torch.from_numpy(q))
            scales[e].copy_(torch.from_numpy(s))
    return a, sz, sizes, codes, scales


def touched_weight_bytes(c, sizes) -> int:
    per = c.N * c.K // 2 + (c.N * (c.K // 64) * 4 if c.fmt == "nf4" else c.N * (c.K // 32))
    return int(np.count_nonzero(sizes)) * per


def time_calls(fn, copies, steps, warmup, torch, use_graph=True):
    """Per-call device time (ms) of fn(copy), measured with events on the launch
    stream. With use_graph, `steps` calls (rotating weight copies) are captured
    into one HIP graph and replayed, so host-side call overhead cannot leak into
    the timing; the result is (replay time / calls) per replay."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(copies[i % len(copies)])
    torch.cuda.synchronize()
    if use_graph:
        try:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for i in range(steps):
                        fn(copies[i % len(copies)])
            torch.cuda.synchronize()
            times = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1) / steps)
            return times, "hip graph of %d calls, 5 replays" % steps
        except Exception as ex:  # capture not possible: fall back to eager events
            print(f"bench.py: graph timing unavailable ({ex}); using eager events", file=sys.stderr)
            torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        fn(copies[(warmup + i) % len(copies)])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev], "eager events"


def time_kernel(fn, copies, steps, warmup, geg, torch, slot, force_path=0):
    """Average device time (ms) of one kernel of the call, from the two HIP events
    the library records on the launch stream right before and after that kernel
    (slot 0: tiled or dgrad kernel, slot 1: the decode kernels). The calls run back to
    back with one event pair each; all are read after a final synchronisation."""
    for i in range(warmup):
        fn(copies[i % len(copies)], None)
    torch.cuda.synchronize()
    timers = [geg.KernelTimer(force_path) for _ in range(steps)]
    for i in range(steps):
        fn(copies[i % len(copies)], timers[i].opts())
    torch.cuda.synchronize()
    ms = [t.elapsed_ms()[slot] for t in timers]
    ms = [m for m in ms if m is not None]
    return float(np.mean(ms)) if ms else None


def cpu_baseline(c, seed, budget_s=12.0, unit="TFLOP/s", w4a8=False, max_cols=4096):
    """The fp64 oracle (decode each expert to fp64, one matmul per expert) on as
    many of the case's routed experts as fit in about budget_s seconds (at least
    one), as TFLOP/s or, for decode-class cases, packed-weight GB/s. Experts are
    packed one at a time as needed (not timed); for a projection wider than
    max_cols output columns only the first max_cols weight rows of each expert
    enter the sample (the oracle's rate does not depend on the width). With w4a8,
    the oracle of that variant: each expert's rows quantised to MXFP8 first
    (timed with the matmul)."""
    import oracle
    import synthetic
    a_bits, sizes = synthetic.rows_bf16(c, seed)
    off = oracle.offsets(sizes)
    ncols = min(c.N, max_cols)
    # distinct experts in the sample: up to 32, fewer for large experts (about
    # 6e7 packed weights in all, a few seconds of the oracle's packer)
    distinct = max(1, min(32, int(6e7 // (ncols * c.K))))
    routed = [e for e in range(c.E) if sizes[e] > 0][:distinct]
    packed = {}

    def pack(e):                              # input preparation, not timed
        if e not in packed:
            if c.fmt == "nf4":
                packed[e] = oracle.quantize_pack_nf4(synthetic.nf4_weight_f32(c, seed, e, first_rows=ncols))
            else:
                q, sc = synthetic.mxfp4_bytes(c, seed, e)
                packed[e] = (q[:ncols], sc[:ncols])
        return packed[e]

    flops, wbytes, t_dq, t_mm, used = 0.0, 0, 0.0, 0.0, 0
    i = 0
    while True:
        e = routed[i % len(routed)]
        i += 1
        q, s = pack(e)
        t0 = time.perf_counter()
        W = oracle.dequant_nf4(q, s) if c.fmt == "nf4" else oracle.dequant_mxfp4(q, s)
        t1 = time.perf_counter()
        rows = a_bits[off[e]:off[e + 1]]
        if w4a8:
            out = oracle.w4a8_grouped_ref(rows, np.array([len(rows)], np.int32), lambda _e: W, ncols)
        else:
            out = oracle.grouped_ref(rows, np.array([len(rows)], np.int32), lambda _e: W, ncols)
        t2 = time.perf_counter()
        t_dq += t1 - t0
        t_mm += t2 - t1
        flops += 2.0 * len(rows) * ncols * c.K
        wbytes += ncols * c.K // 2 + (ncols * (c.K // 64) * 4 if c.fmt == "nf4" else ncols * (c.K // 32))
        used += 1
        del W, out
        if t_dq + t_mm > budget_s:
            break
    secs = t_dq + t_mm
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info()] or [0]) or os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    value = flops / secs / 1e12 if unit == "TFLOP/s" else wbytes / secs / 1e9
    width = f"the first {ncols} of {c.N} weight rows of each expert" if ncols < c.N else "whole experts"
    return {"value": value, "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{c.name}: {used} expert GEMMs ({width}; cycling over the first {len(packed)} of "
                      f"{int(np.count_nonzero(sizes))} routed experts, {int(flops / 2 / ncols / c.K)} rows), "
                      + ("MXFP8 activation quantisation + " if w4a8 else "") + "fp64 decode + numpy matmul",
            "seconds": secs, "dequant_s": t_dq, "matmul_s": t_mm,
            "host_cpus": os.cpu_count()}


def cpu_baseline_block(cg, cdn, seed, budget_s=12.0):
    """The fp64 oracle of the fused expert block on as many routed experts as fit
    in about budget_s seconds, as TFLOP/s (both projections' flops)."""
    import oracle
    import synthetic
    from oracle import cases as C
    a_bits, sizes = synthetic.rows_bf16(cg, seed)
    off = oracle.offsets(sizes)
    experts = [e for e in range(cg.E) if sizes[e]][:16]
    H, I = cg.K, cg.N // 2
    flops, secs, used = 0.0, 0.0, 0
    t_start = time.perf_counter()
    i = 0
    while True:
        e = experts[i % len(experts)]
        i += 1
        if cg.fmt == "nf4":
            p13, p2 = C.nf4_expert(cg, seed, e), C.nf4_expert(cdn, seed, e)
            dq = oracle.dequant_nf4
        else:
            p13, p2 = synthetic.mxfp4_bytes(cg, seed, e), synthetic.mxfp4_bytes(cdn, seed, e)
            dq = oracle.dequant_mxfp4
        t0 = time.perf_counter()
        W13, W2 = dq(*p13), dq(*p2)
        rows = a_bits[off[e]:off[e + 1]]
        oracle.expert_block_ref(rows, np.array([len(rows)], np.int32), lambda _e: W13, lambda _e: W2, H, I)
        secs += time.perf_counter() - t0
        flops += 2.0 * len(rows) * 3 * H * I
        used += 1
        if time.perf_counter() - t_start > budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info()] or [0]) or os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{cg.name} block: {used} expert blocks (cycling over {len(experts)} routed experts), "
                      "fp64 decode + numpy matmuls + SwiGLU", "seconds": secs, "host_cpus": os.cpu_count()}


def cpu_baseline_lora(c, seed, r, s, budget_s=12.0):
    """The adapter oracle (fp64 forward and backward of the frozen projection plus
    the low-rank delta) on as many routed experts as fit in about budget_s
    seconds, as TFLOP/s of the whole step's flops."""
    import oracle
    import synthetic
    from oracle import cases as C
    from oracle import lora as L
    a_bits, sizes = synthetic.rows_bf16(c, seed)
    dy = synthetic.dgrad_dy_bf16(c, seed)
    off = oracle.offsets(sizes)
    rng = np.random.default_rng([seed, 9])
    experts = [e for e in range(c.E) if sizes[e]][:16]
    flops, secs, used = 0.0, 0.0, 0
    t_start = time.perf_counter()
    i = 0
    while True:
        e = experts[i % len(experts)]
        i += 1
        q, sc = C.nf4_expert(c, seed, e)
        A = (rng.standard_normal((1, r, c.K)) / np.sqrt(c.K)).astype(np.float32)
        B = (rng.standard_normal((1, c.N, r)) * 0.01).astype(np.float32)
        rows = slice(int(off[e]), int(off[e + 1]))
        n = int(off[e + 1] - off[e])
        t0 = time.perf_counter()
        W = oracle.dequant_nf4(q, sc)
        one = np.array([n], np.int32)
        L.lora_forward_ref(a_bits[rows], one, lambda _e: W, A, B, s, c.N)
        L.lora_backward_ref(a_bits[rows], dy[rows], one, lambda _e: W, A, B, s, c.K)
        secs += time.perf_counter() - t0
        flops += lora_step_flops(n, c.N, c.K, r)
        used += 1
        if time.perf_counter() - t_start > budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info()] or [0]) or os.cpu_count()
    except Exception:
        threads = os.cpu_count()
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{c.name} with a rank-{r} adapter: {used} expert forward + backward steps (cycling over "
                      f"{len(experts)} routed experts), fp64 decode + numpy matmuls", "seconds": secs,
            "host_cpus": os.cpu_count()}


def lora_step_flops(M, N, K, r):
    """Forward (projection + adapter) and backward (dgrad + adapter input gradient
    + both adapter gradients) of the adapted grouped projection."""
    return 2.0 * M * N * K * 2 + 2.0 * M * r * (K + N) + 2.0 * M * r * (N + K) + 2.0 * M * r * (N + K)


def main_lora(args, torch, geg, synthetic):
    name, r, s = LORA_WORKLOADS[args.workload]
    c = synthetic.case(name)
    dev = torch.device("cuda", 0)
    a, sz, sizes, codes, scales = make_inputs(c, args.seed, torch, geg, dev)
    rng = np.random.default_rng([args.seed, 9])
    A = torch.from_numpy((rng.standard_normal((c.E, r, c.K)) / np.sqrt(c.K)).astype(np.float32)).to(dev)
    B = torch.from_numpy((rng.standard_normal((c.E, c.N, r)) * 0.01).astype(np.float32)).to(dev)
    dy = torch.from_numpy(synthetic.dgrad_dy_bf16(c, args.seed).view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
    u = torch.empty((c.M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((c.M, c.K), dtype=torch.bfloat16, device=dev)
    ga = torch.empty((c.E, r, c.K), dtype=torch.float32, device=dev)
    gb = torch.empty((c.E, c.N, r), dtype=torch.float32, device=dev)
    ws = geg.Workspace(max(geg.lib().geg_lora_workspace_bytes(geg.GEG_OP_NF4_FWD, c.M, c.N, c.K, c.E, r),
                           geg.lib().geg_lora_workspace_bytes(geg.GEG_OP_NF4_DGRAD, c.M, c.N, c.K, c.E, r)))
    wc = [(codes, scales)]

    def fwd(w, opts=None):
        geg.gnf4_grouped_gemm_lora(a, sz, w[0], w[1], A, B, s, out=out, u=u, workspace=ws, opts=opts)

    def bwd(w, opts=None):
        geg.gnf4_grouped_dgrad_lora(dy, sz, w[0], w[1], a, A, B, u, s, dx=dx, grad_a=ga, grad_b=gb, workspace=ws,
                                    opts=opts)

    def fwd_plain(w, opts=None):
        geg.gnf4_grouped_gemm(a, sz, w[0], w[1], out=out, workspace=ws, opts=geg.Opts(2, 0))

    def bwd_plain(w, opts=None):
        geg.gnf4_grouped_dgrad(dy, sz, w[0], w[1], dx=dx, workspace=ws)

    fwd(wc[0])
    bwd(wc[0])
    torch.cuda.synchronize()
    assert ws.read_error() == 0, "device error word set"
    for i in range(args.warmup):
        fwd(wc[0]); bwd(wc[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fwd(wc[0]); bwd(wc[0])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    f_ms = float(np.mean(time_calls(fwd, wc, args.steps, args.warmup, torch)[0]))
    b_ms = float(np.mean(time_calls(bwd, wc, args.steps, args.warmup, torch)[0]))
    fp_ms = float(np.mean(time_calls(fwd_plain, wc, args.steps, args.warmup, torch)[0]))
    bp_ms = float(np.mean(time_calls(bwd_plain, wc, args.steps, args.warmup, torch)[0]))
    kern_ms = time_kernel(fwd, wc, args.steps, args.warmup, geg, torch, 0)
    flops = lora_step_flops(c.M, c.N, c.K, r)
    kflops = 2.0 * c.M * c.N * c.K + 2.0 * c.M * r * c.N   # the tiled kernel: projection + adapter delta
    result = {
        "metric": METRIC, "value": round(flops / ((f_ms + b_ms) * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": f"{name} with a rank-{r} adapter (forward + backward)", "format": c.fmt, "E": c.E,
                   "K": c.K, "N": c.N, "rows": c.M, "rank": r, "scale": s},
        "lora": {"forward_ms": round(f_ms, 5), "backward_ms": round(b_ms, 5), "plain_forward_ms": round(fp_ms, 5),
                 "plain_dgrad_ms": round(bp_ms, 5),
                 "adapter_overhead": round((f_ms + b_ms) / (fp_ms + bp_ms) - 1.0, 4)},
        "roofline": {"bound": "mfma", "achieved": round(kflops / (kern_ms * 1e-3) / 1e12, 2),
                     "peak": round(PEAK_MFMA_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(kflops / (kern_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                     "kernel": f"tiled kernel with the adapter epilogue (nf4), {name}",
                     "per_launch_gflop": round(kflops / 1e9, 3), "kernel_ms": round(kern_ms, 5), "traffic": None},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_lora(c, args.seed, r, s, args.cpu_budget)
    result["kernel_sha"] = kernel_sha()
    print(json.dumps(result), flush=True)


def main_block(args, torch, geg, synthetic):
    """Fused expert block workloads: prefill and decode calls of gnf4/gmxfp4_expert_block."""
    dev = torch.device("cuda", 0)
    pg, pdn, dg, ddn = (synthetic.case(n) for n in BLOCK_WORKLOADS[args.workload])
    blk = geg.gnf4_expert_block if pg.fmt == "nf4" else geg.gmxfp4_expert_block
    gemm = geg.gnf4_grouped_gemm if pg.fmt == "nf4" else geg.gmxfp4_grouped_gemm
    a, sz, sizes, c13, s13 = make_inputs(pg, args.seed, torch, geg, dev)
    _, _, sizes2, c2, s2 = make_inputs(pdn, args.seed, torch, geg, dev)
    assert (sizes == sizes2).all(), "gate_up and down cases must share their routing"
    H, I = pg.K, pg.N // 2
    assert pdn.K == I and pdn.N == H
    stack = sum(t.numel() * t.element_size() for t in (c13, s13, c2, s2))
    ncopies = max(1, int(np.ceil(ROTATE_BYTES / stack)))
    wcopies = [(c13, s13, c2, s2)] + [tuple(t.clone() for t in (c13, s13, c2, s2)) for _ in range(ncopies - 1)]
    ws = geg.Workspace(geg.geg_workspace_bytes(3 if pg.fmt == "nf4" else 4, pg.M, H, I, pg.E))
    out = torch.empty((pg.M, H), dtype=torch.bfloat16, device=dev)
    h = torch.empty((pg.M, 2 * I), dtype=torch.bfloat16, device=dev)
    act = torch.zeros((pg.M, I), dtype=torch.bfloat16, device=dev)

    def prefill(wc, opts=None):
        blk(a, sz, wc[0], wc[1], wc[2], wc[3], out=out, workspace=ws, opts=opts)

    def unfused(wc, opts=None):
        # the two plain GEMMs of the same shapes (timing only: the down GEMM reads
        # a zero intermediate; an unfused block would also need a SwiGLU pass)
        gemm(a, sz, wc[0], wc[1], out=h, workspace=ws)
        gemm(act, sz, wc[2], wc[3], out=out, workspace=ws)

    da_bits, dsizes = synthetic.rows_bf16(dg, args.seed)
    da = torch.from_numpy(da_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    dsz = torch.from_numpy(dsizes).to(dev)
    dout = torch.empty((dg.M, H), dtype=torch.bfloat16, device=dev)
    dws = geg.Workspace(geg.geg_workspace_bytes(3 if pg.fmt == "nf4" else 4, dg.M, H, I, dg.E))

    def decode(wc, opts=None):
        blk(da, dsz, wc[0], wc[1], wc[2], wc[3], out=dout, workspace=dws, opts=opts)

    # A whole MoE layer around the block: the router's top-k ids -> device sort and
    # row gather -> fused block -> weighted combine back to token order.
    ids = torch.from_numpy(synthetic.topk_ids(pg, args.seed).astype(np.int32)).to(dev)
    xtok = torch.from_numpy(synthetic.activations_bf16(pg, args.seed).view(np.int16)).view(torch.bfloat16).to(dev)
    wr = torch.full((pg.T, pg.top_k), 1.0 / pg.top_k, dtype=torch.float32, device=dev)
    rws = geg.Workspace(geg.lib().geg_route_workspace_bytes(pg.T, pg.top_k, pg.E))
    lsz, lro, lso, lxs = geg.route_sort(ids, pg.E, x=xtok, workspace=rws)
    torch.cuda.synchronize()
    assert (lsz.cpu().numpy() == sizes).all(), "device routing sort disagrees with the workload's sizes"
    assert torch.equal(lxs.view(torch.int16), a.view(torch.int16)), "device gather disagrees with the grouped rows"
    ly = torch.empty((pg.M, H), dtype=torch.bfloat16, device=dev)
    lout = torch.empty((pg.T, H), dtype=torch.bfloat16, device=dev)

    def route(wc, opts=None):
        geg.route_sort(ids, pg.E, x=xtok, workspace=rws)

    def combine(wc, opts=None):
        geg.route_combine(ly, lro, wr, pg.top_k, out=lout)

    def layer(wc, opts=None):
        s_, ro_, so_, xs_ = geg.route_sort(ids, pg.E, x=xtok, workspace=rws)
        blk(xs_, s_, wc[0], wc[1], wc[2], wc[3], out=ly, workspace=ws)
        geg.route_combine(ly, ro_, wr, pg.top_k, out=lout)

    prefill(wcopies[0])
    decode(wcopies[0])
    layer(wcopies[0])
    torch.cuda.synchronize()
    assert ws.read_error() == 0 and dws.read_error() == 0 and rws.read_error() == 0, "device error word set"
    for i in range(args.warmup):
        prefill(wcopies[i % ncopies]); decode(wcopies[i % ncopies])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        prefill(wcopies[i % ncopies]); decode(wcopies[i % ncopies])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    flops = 2.0 * pg.M * 3 * H * I
    pre_ms, pre_how = time_calls(prefill, wcopies, args.steps, args.warmup, torch)
    pre_avg = float(np.mean(pre_ms))
    un_ms, _ = time_calls(unfused, wcopies, args.steps, args.warmup, torch)
    blk_ms = time_kernel(prefill, wcopies, args.steps, args.warmup, geg, torch, 0)
    tflops = flops / (pre_avg * 1e-3) / 1e12
    ktflops = flops / (blk_ms * 1e-3) / 1e12
    route_ms, _ = time_calls(route, wcopies, args.steps, args.warmup, torch)
    comb_ms, _ = time_calls(combine, wcopies, args.steps, args.warmup, torch)
    layer_ms, _ = time_calls(layer, wcopies, args.steps, args.warmup, torch)
    dbytes = touched_weight_bytes(dg, dsizes) + touched_weight_bytes(ddn, dsizes)
    dec_ms, dec_how = time_calls(decode, wcopies, max(args.steps, 50), args.warmup, torch)
    dec_avg = float(np.mean(dec_ms))
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16" if pg.fmt == "nf4" else "bf16", "data": "synthetic",
        "config": {"workload": f"{pg.name} + {pdn.name} fused block, {dg.name} + {ddn.name} fused block",
                   "format": pg.fmt, "E": pg.E, "H": H, "I": I, "prefill_rows": pg.M,
                   "decode_rows": dg.M, "top_k": pg.top_k, "weight_copies_rotated": ncopies},
        "prefill": {"ms": round(pre_avg, 5), "gflop": flops / 1e9, "tflops": round(tflops, 2),
                    "timing": pre_how, "two_plain_gemms_ms": round(float(np.mean(un_ms)), 5),
                    "block_events_ms": round(blk_ms, 5)},
        "moe_layer": {"tokens": pg.T, "route_sort_gather_ms": round(float(np.mean(route_ms)), 5),
                      "combine_ms": round(float(np.mean(comb_ms)), 5),
                      "layer_ms": round(float(np.mean(layer_ms)), 5),
                      "timing": "hip graphs; sort + gather, block, combine on the device"},
        "decode": {"value": round(dbytes / (dec_avg * 1e-3) / 1e9, 1), "unit": "GB/s",
                   "ms": round(dec_avg, 5), "weight_bytes": dbytes, "timing": dec_how},
        "roofline": {"bound": "mfma", "achieved": round(ktflops, 2), "peak": round(PEAK_MFMA_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(ktflops / PEAK_MFMA_TFLOPS, 4),
                     "kernel": f"fused expert block ({pg.fmt}): both projections' kernels, {pg.name}",
                     "per_launch_gflop": round(flops / 1e9, 3), "kernel_ms": round(blk_ms, 5),
                     "traffic": None},
        "kernel_sha": kernel_sha(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_block(pg, pdn, args.seed, args.cpu_budget)
    print(json.dumps(result), flush=True)


HEADLINE_PREFILL = "mixtral_w13_t4096"
HEADLINE_DGRAD = "mixtral_dgrad_w13"
HEADLINE_DECODE = ["olmoe_gate_up_t1", "qwen3_gate_up_t1", "qwen3_down_t1", "gptoss_gate_up_t1",
                   "gptoss_down_t1", "qwen3_gate_up_t64", "qwen3_down_t64"]
PROFILE_FILE = os.path.join(ROOT, "profiles", "kernels.json")


def make_weights(c, seed, torch, geg, dev, experts):
    """Packed weight stack [E, N, K/2] + scales of case c with the listed experts
    filled (the kernels read only experts with routed rows; the rest stay zero)."""
    import synthetic
    codes = torch.zeros((c.E, c.N, c.K // 2), dtype=torch.uint8, device=dev)
    if c.fmt == "nf4":
        scales = torch.zeros((c.E, c.N, c.K // 64), dtype=torch.float32, device=dev)
    else:
        scales = torch.zeros((c.E, c.N, c.K // 32), dtype=torch.uint8, device=dev)
    for e in experts:
        e = int(e)
        if c.fmt == "nf4":
            w = torch.from_numpy(synthetic.nf4_weight_f32(c, seed, e)).to(dev)
            q, sc = geg.gnf4_quantize(w)
            del w
        else:
            qn, sn = synthetic.mxfp4_bytes(c, seed, e)
            q, sc = torch.from_numpy(qn).to(dev), torch.from_numpy(sn).to(dev)
        codes[e].copy_(q)
        scales[e].copy_(sc)
    return codes, scales


def rotated_copies(tensors):
    """The stack plus as many clones as make the copies exceed ROTATE_BYTES."""
    nbytes = sum(t.numel() * t.element_size() for t in tensors)
    n = max(1, int(np.ceil(ROTATE_BYTES / nbytes)))
    return [tuple(tensors)] + [tuple(t.clone() for t in tensors) for _ in range(n - 1)]


def host_info():
    """CPU model, logical CPUs and the BLAS numpy runs the oracle's matmuls on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                break
    except Exception:
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas": blas}


def profile_record(workload, kernel):
    """The profiler's figures for (workload, kernel) from profiles/kernels.json, if
    they were taken with the current kernel sources."""
    try:
        rec = json.load(open(PROFILE_FILE)).get(f"{workload}:{kernel}")
    except Exception:
        return None
    if rec and rec.get("kernel_sha") == kernel_sha():
        return rec
    return None


def traffic_record(name):
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(tfile)).get(name)
    except Exception:
        return None
    if rec and rec.get("kernel_sha") == kernel_sha():
        return rec["hbm_bytes"]
    return None


def copy_floor_ms(nbytes, steps, warmup, torch, dev):
    """Per-call time of one plain device copy of nbytes (read nbytes, write
    nbytes), sources rotated like the weight stacks, HIP-graph timed."""
    n = max(16, (int(nbytes) + 15) // 16 * 16)
    k = max(2, int(np.ceil(ROTATE_BYTES / n)))
    srcs = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(k)]
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    ms, _ = time_calls(lambda src: dst.copy_(src), srcs, steps, warmup, torch)
    del srcs, dst
    return float(np.mean(ms))


def main_headline(args, torch, geg, synthetic):
    dev = torch.device("cuda", 0)
    cp, cg = synthetic.case(HEADLINE_PREFILL), synthetic.case(HEADLINE_DGRAD)
    assert (cp.E, cp.K, cp.N, cp.T) == (cg.E, cg.K, cg.N, cg.T), "the dgrad runs on the forward's weights"
    a_bits, sizes = synthetic.rows_bf16(cp, args.seed)
    a = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    sz = torch.from_numpy(sizes).to(dev)
    codes, scales = make_weights(cp, args.seed, torch, geg, dev, np.nonzero(sizes)[0])
    wcopies = rotated_copies((codes, scales))
    out = torch.empty((cp.M, cp.N), dtype=torch.bfloat16, device=dev)
    ws = geg.Workspace(geg.geg_workspace_bytes(geg.GEG_OP_NF4_FWD, cp.M, cp.N, cp.K, cp.E))
    dy = torch.from_numpy(synthetic.dgrad_dy_bf16(cg, args.seed).view(np.int16)).view(torch.bfloat16).to(dev)
    dx = torch.empty((cg.M, cg.K), dtype=torch.bfloat16, device=dev)
    dws = geg.Workspace(geg.geg_workspace_bytes(geg.GEG_OP_NF4_DGRAD, cg.M, cg.N, cg.K, cg.E))

    def fwd(wc, opts=None):
        geg.gnf4_grouped_gemm(a, sz, wc[0], wc[1], out=out, workspace=ws, opts=opts)

    def dgrad(wc, opts=None):
        geg.gnf4_grouped_dgrad(dy, sz, wc[0], wc[1], dx=dx, workspace=dws, opts=opts)

    # decode cases: weights of the same model shared across token counts
    decs = []
    stacks = {}
    for name in HEADLINE_DECODE:
        c = synthetic.case(name)
        key = (c.fmt, c.E, c.K, c.N)
        dbits, dsizes = synthetic.rows_bf16(c, args.seed)
        touched = set(np.nonzero(dsizes)[0].tolist())
        for other in HEADLINE_DECODE:          # every case of this stack
            oc = synthetic.case(other)
            if (oc.fmt, oc.E, oc.K, oc.N) == key:
                touched |= set(np.nonzero(synthetic.rows_bf16(oc, args.seed)[1])[0].tolist())
        if key not in stacks:
            stacks[key] = rotated_copies(make_weights(c, args.seed, torch, geg, dev, sorted(touched)))
        da = torch.from_numpy(dbits.view(np.int16)).view(torch.bfloat16).to(dev)
        dsz = torch.from_numpy(dsizes).to(dev)
        dout = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
        dws_c = geg.Workspace(geg.geg_workspace_bytes(0 if c.fmt == "nf4" else 1, c.M, c.N, c.K, c.E))
        fn = geg.gnf4_grouped_gemm if c.fmt == "nf4" else geg.gmxfp4_grouped_gemm

        def dec(wc, opts=None, fn=fn, da=da, dsz=dsz, dout=dout, w=dws_c):
            fn(da, dsz, wc[0], wc[1], out=dout, workspace=w, opts=opts)
        decs.append((c, dsizes, dec, stacks[key], dws_c))

    # correctness gate before timing: device error words clean
    fwd(wcopies[0])
    dgrad(wcopies[0])
    for c, _, dec, cps, w in decs:
        dec(cps[0])
    torch.cuda.synchronize()
    assert ws.read_error() == 0 and dws.read_error() == 0, "device error word set"
    for c, _, _, _, w in decs:
        assert w.read_error() == 0, f"device error word set ({c.name})"

    # ---- timed region: K steps (forward, dgrad, every decode case), wall clock
    def step(i):
        fwd(wcopies[i % len(wcopies)])
        dgrad(wcopies[i % len(wcopies)])
        for c, _, dec, cps, _ in decs:
            dec(cps[i % len(cps)])
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    flops = 2.0 * cp.M * cp.N * cp.K
    # forward call, timed twice (self-pair: the run-to-run noise beside every ratio)
    f1, how = time_calls(fwd, wcopies, args.steps, args.warmup, torch)
    f2, _ = time_calls(fwd, wcopies, args.steps, args.warmup, torch)
    f_ms, f2_ms = float(np.mean(f1)), float(np.mean(f2))
    fk_ms = time_kernel(fwd, wcopies, args.steps, args.warmup, geg, torch, 0)
    g1, _ = time_calls(dgrad, wcopies, args.steps, args.warmup, torch)
    g_ms = float(np.mean(g1))
    gk_ms = time_kernel(dgrad, wcopies, args.steps, args.warmup, geg, torch, 0)

    def kroof(name, kernel, kms, gflop):
        ach = gflop * 1e9 / (kms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 2), "peak": round(PEAK_MFMA_TFLOPS, 1), "unit": "TFLOP/s",
             "frac": round(ach / PEAK_MFMA_TFLOPS, 4), "kernel": f"{kernel} (nf4), {name}",
             "per_launch_gflop": round(gflop, 3), "kernel_ms": round(kms, 5),
             "timing": f"HIP events around the kernel on its launch stream, mean of {args.steps} back-to-back "
                       "launches"}
        prof = profile_record(name, kernel)
        if prof:
            pms = prof["mean_us"] * 1e-3
            r["profile"] = {"kernel_ms": round(pms, 5), "frac": round(gflop * 1e9 / (pms * 1e-3) / 1e12
                                                                        / PEAK_MFMA_TFLOPS, 4),
                            "events_over_profile": round(kms / pms, 4), "launches": prof.get("launches"),
                            "source": prof.get("source")}
            if prof.get("clock_ghz"):
                peak_clk = 256 * 4096 * prof["clock_ghz"] * 1e9 / 1e12
                r["measured_clock"] = {"ghz": prof["clock_ghz"], "peak_at_clock": round(peak_clk, 1),
                                       "frac_at_clock": round(ach / peak_clk, 4), "source": prof.get("source")}
            if prof.get("mfma_busy") is not None:
                r["mfma_busy"] = prof["mfma_busy"]
        r["traffic"] = traffic_record(name)
        return r

    rf = kroof(cp.name, "tile_kernel", fk_ms, flops / 1e9)
    rg = kroof(cg.name, "tile_kernel_dgrad", gk_ms, flops / 1e9)

    # decode legs: each call (HIP graph), its kernels (events), a copy of the same bytes
    dsteps = max(args.steps, 50)
    dec_res = {}
    tot_b, tot_ms = 0, 0.0
    for c, dsizes, dec, cps, _ in decs:
        dms, dhow = time_calls(dec, cps, dsteps, args.warmup, torch)
        d_ms = float(np.mean(dms))
        kms = time_kernel(dec, cps, dsteps, args.warmup, geg, torch, 1)
        dbytes = touched_weight_bytes(c, dsizes)
        cms = copy_floor_ms(dbytes, dsteps, args.warmup, torch, dev)
        dec_res[c.name] = {"gbps": round(dbytes / (d_ms * 1e-3) / 1e9, 1), "ms": round(d_ms, 5),
                           "weight_bytes": dbytes, "frac_of_hbm_peak": round(dbytes / (d_ms * 1e-3) / 1e9
                                                                             / PEAK_HBM_GBPS, 4),
                           "kernels_ms": round(kms, 5),
                           "copy_of_same_bytes_ms": round(cms, 5),
                           "frac_of_copy_time": round(cms / d_ms, 4)}
        if c.T == 1:
            tot_b += dbytes
            tot_ms += d_ms
    dec_gbps = tot_b / (tot_ms * 1e-3) / 1e9

    roof = max((rf, rg), key=lambda r: r["kernel_ms"])
    result = {
        "metric": METRIC, "value": round(flops / (f_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": f"{cp.name} (forward + dgrad) + decode " + ", ".join(HEADLINE_DECODE),
                   "format": cp.fmt, "E": cp.E, "K": cp.K, "N": cp.N, "prefill_rows": cp.M, "top_k": cp.top_k,
                   "weight_copies_rotated": len(wcopies)},
        "prefill": {"ms": round(f_ms, 5), "gflop": flops / 1e9, "tflops": round(flops / (f_ms * 1e-3) / 1e12, 2),
                    "timing": how, "self_pair_ms": [round(f_ms, 5), round(f2_ms, 5)],
                    "self_pair_ratio": round(f2_ms / f_ms, 4),
                    "kernel_ms": round(fk_ms, 5), "kernel_tflops": rf["achieved"],
                    "frac_of_mfma_peak": round(flops / (f_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)},
        "dgrad": {"workload": cg.name, "ms": round(g_ms, 5), "tflops": round(flops / (g_ms * 1e-3) / 1e12, 2),
                  "kernel_ms": round(gk_ms, 5), "kernel_tflops": rg["achieved"]},
        "decode": {"value": round(dec_gbps, 1), "unit": "GB/s",
                   "what": "packed-weight bytes of the five T=1 cases over their summed call times",
                   "frac_of_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4), "timing": "hip graph of "
                   f"{dsteps} calls, 5 replays; copies: torch device copy of the same byte count",
                   "cases": dec_res},
        "roofline": roof,
        "roofline_other": rg if roof is rf else rf,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cp, args.seed, args.cpu_budget, "TFLOP/s")
        cb.update(host_info())
        result["cpu_baseline"] = cb
    result["kernel_sha"] = kernel_sha()
    print(json.dumps(result), flush=True)


DECODE_PATHS = [("auto", 0, 0), ("vector", 3, 0), ("narrow", 4, 0), ("skinny_s1", 1, 1), ("skinny_s2", 1, 2),
                ("skinny_s4", 1, 4), ("skinny_s8", 1, 8)]


def main_decode_paths(args, torch, geg, synthetic):
    """Every decode path on every headline decode case: the automatic choice, the
    vector and narrow kernels, and the skinny kernel with K split S = 1, 2, 4, 8
    ways (S > 1 adds the fixed-order reduce launch), beside a copy of the same
    bytes; per-call time from a HIP graph of back-to-back calls."""
    dev = torch.device("cuda", 0)
    steps = max(args.steps, 50)
    cases = {}
    for name in HEADLINE_DECODE:
        c = synthetic.case(name)
        a_bits, sizes = synthetic.rows_bf16(c, args.seed)
        a = torch.from_numpy(a_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        sz = torch.from_numpy(sizes).to(dev)
        cps = rotated_copies(make_weights(c, args.seed, torch, geg, dev, np.nonzero(sizes)[0]))
        out = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
        ws = geg.Workspace(64 << 20)
        fn = geg.gnf4_grouped_gemm if c.fmt == "nf4" else geg.gmxfp4_grouped_gemm
        nbytes = touched_weight_bytes(c, sizes)
        res = {"weight_bytes": nbytes, "max_rows": int(sizes.max())}
        for vname, fp, sk in DECODE_PATHS:
            if vname == "vector" and int(sizes.max()) > 8:
                continue   # the vector kernel takes experts of at most 8 rows
            o = geg.Opts(force_path=fp, split_k=sk, kernel_events=None, cu_limit=0)

            def call(wc, opts=None, o=o):
                fn(a, sz, wc[0], wc[1], out=out, workspace=ws, opts=o)
            call(cps[0])
            torch.cuda.synchronize()
            assert ws.read_error() == 0, f"device error word set ({name}, {vname})"
            ms, _ = time_calls(call, cps, steps, args.warmup, torch)
            res[vname] = {"us": round(float(np.mean(ms)) * 1e3, 3),
                          "gbps": round(nbytes / (float(np.mean(ms)) * 1e-3) / 1e9, 1)}
        res["copy_of_same_bytes_us"] = round(copy_floor_ms(nbytes, steps, args.warmup, torch, dev) * 1e3, 3)
        cases[name] = res
        print(f"bench.py: {name} " + json.dumps(res), file=sys.stderr, flush=True)
        del cps
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "decode call time per path (us)", "value": None, "unit": "us", "n_gpus": 1,
                      "steps": steps, "warmup": args.warmup, "higher_is_better": False, "data": "synthetic",
                      "timing": f"hip graph of {steps} calls, 5 replays", "cases": cases,
                      "kernel_sha": kernel_sha()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "decode_paths"] + sorted(WORKLOADS) + sorted(BLOCK_WORKLOADS)
                    + sorted(LORA_WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 times): the "
                         "reference kernel that scales the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the grouped GEMM's multi-GPU sharding is a design note, not a measured path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4,
                          "copy_calibration_bytes_written": dst.numel() * 4}), flush=True)
        return
    import grouped_expert_gemm_amd as geg
    import synthetic

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.workload == "headline":
        main_headline(args, torch, geg, synthetic)
        return
    if args.workload == "decode_paths":
        main_decode_paths(args, torch, geg, synthetic)
        return
    if args.workload in BLOCK_WORKLOADS:
        main_block(args, torch, geg, synthetic)
        return
    if args.workload in LORA_WORKLOADS:
        main_lora(args, torch, geg, synthetic)
        return
    pre_name, dec_name = WORKLOADS[args.workload]
    cp = synthetic.case(pre_name or dec_name)
    w4a8 = args.workload in W4A8_WORKLOADS
    fn = geg.gnf4_grouped_gemm if cp.fmt == "nf4" else geg.gmxfp4_grouped_gemm
    if w4a8:
        fn = geg.gmxfp4_w4a8_grouped_gemm

    # The weight stack of the workload (the decode leg uses the same experts).
    a, sz, sizes, codes, scales = make_inputs(cp, args.seed, torch, geg, dev)
    stack_bytes = codes.numel() + scales.numel() * scales.element_size()
    ncopies = max(1, int(np.ceil(ROTATE_BYTES / stack_bytes)))
    wcopies = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(ncopies - 1)]

    prefill = None
    if pre_name:
        ws = geg.Workspace(1 << 20)
        if cp.op == "dgrad":
            dy = torch.from_numpy(synthetic.dgrad_dy_bf16(cp, args.seed).view(np.int16)).view(torch.bfloat16).to(dev)
            dx = torch.empty((cp.M, cp.K), dtype=torch.bfloat16, device=dev)

            dfn = geg.gnf4_grouped_dgrad if cp.fmt == "nf4" else geg.gmxfp4_grouped_dgrad

            def prefill(wc, opts=None):
                dfn(dy, sz, wc[0], wc[1], dx=dx, workspace=ws, opts=opts)
        else:
            out = torch.empty((cp.M, cp.N), dtype=torch.bfloat16, device=dev)

            def prefill(wc, opts=None):
                fn(a, sz, wc[0], wc[1], out=out, workspace=ws, opts=opts)

    dec = None
    if dec_name:
        cd = synthetic.case(dec_name)
        da_bits, dsizes = synthetic.rows_bf16(cd, args.seed)
        da = torch.from_numpy(da_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        dsz = torch.from_numpy(dsizes).to(dev)
        dout = torch.empty((cd.M, cd.N), dtype=torch.bfloat16, device=dev)
        dws = geg.Workspace(geg.geg_workspace_bytes(0 if cd.fmt == "nf4" else 1, cd.M, cd.N, cd.K, cd.E))

        def decode(wc, opts=None):
            fn(da, dsz, wc[0], wc[1], out=dout, workspace=dws, opts=opts)
        dec = (cd, dsizes, decode)

    # correctness gate before timing: device error words clean
    if prefill:
        prefill(wcopies[0])
    if dec:
        dec[2](wcopies[0])
    torch.cuda.synchronize()
    if prefill:
        assert ws.read_error() == 0, "device error word set"
    if dec:
        assert dws.read_error() == 0, "device error word set (decode)"

    # ---- timed region: K steps of (prefill + decode), whole-step wall clock
    def step(i):
        if prefill:
            prefill(wcopies[i % ncopies])
        if dec:
            dec[2](wcopies[i % ncopies])
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    result = {
        "metric": METRIC, "value": None, "unit": None, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8xfp4" if w4a8 else ("fp16" if cp.fmt == "nf4" else "bf16"), "data": "synthetic",
        "config": {"workload": " + ".join(x for x in (pre_name, dec_name) if x),
                   "format": cp.fmt, "E": cp.E, "K": cp.K, "N": cp.N,
                   "prefill_rows": cp.M if pre_name else 0,
                   "decode_rows": dec[0].M if dec else 0, "top_k": cp.top_k,
                   "weight_copies_rotated": ncopies},
    }
    roof = None
    # ---- prefill: per-call time (HIP graph of back-to-back calls) and the tiled
    # kernel's own time (events around it)
    if prefill:
        pre_ms, pre_how = time_calls(prefill, wcopies, args.steps, args.warmup, torch)
        flops = 2.0 * cp.M * cp.N * cp.K
        pre_avg = float(np.mean(pre_ms))
        tflops = flops / (pre_avg * 1e-3) / 1e12
        kern_ms = time_kernel(prefill, wcopies, args.steps, args.warmup, geg, torch, 0)
        ktflops = flops / (kern_ms * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if w4a8 else PEAK_MFMA_TFLOPS
        result["value"], result["unit"] = round(tflops, 2), "TFLOP/s"
        result["prefill"] = {"ms": round(pre_avg, 5), "ms_min": round(float(np.min(pre_ms)), 5),
                             "gflop": flops / 1e9, "tflops": round(tflops, 2), "timing": pre_how,
                             "kernel_ms": round(kern_ms, 5), "kernel_tflops": round(ktflops, 2),
                             "frac_of_mfma_peak": round(tflops / peak, 4)}
        kname = ("W4A8 kernel (block-scaled fp8 x fp4 MFMA)" if w4a8
                 else "dgrad (tiled) kernel" if cp.op == "dgrad" else "tiled kernel")
        roof = {"bound": "mfma", "achieved": round(ktflops, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(ktflops / peak, 4),
                "kernel": kname + f" ({cp.fmt}), {cp.name}",
                "per_launch_gflop": round(flops / 1e9, 3), "kernel_ms": round(kern_ms, 5)}
    if dec:
        cd, dsizes, decode = dec
        dsteps = max(args.steps, 50)
        dec_ms, dec_how = time_calls(decode, wcopies, dsteps, args.warmup, torch)
        dbytes = touched_weight_bytes(cd, dsizes)
        dec_avg = float(np.mean(dec_ms))
        gbps = dbytes / (dec_avg * 1e-3) / 1e9
        kern_ms = time_kernel(decode, wcopies, dsteps, args.warmup, geg, torch, 1)
        kgbps = dbytes / (kern_ms * 1e-3) / 1e9
        result["decode"] = {"value": round(gbps, 1), "unit": "GB/s", "ms": round(dec_avg, 5),
                            "ms_min": round(float(np.min(dec_ms)), 5), "weight_bytes": dbytes,
                            "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "timing": dec_how,
                            "decode_kernels_ms": round(kern_ms, 5), "decode_kernels_gbps": round(kgbps, 1)}
        if not prefill:
            result["value"], result["unit"] = round(gbps, 1), "GB/s"
            roof = {"bound": "hbm", "achieved": round(kgbps, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(kgbps / PEAK_HBM_GBPS, 4),
                    "kernel": f"decode kernels ({cd.fmt}), {cd.name}",
                    "per_launch_bytes": dbytes, "kernel_ms": round(kern_ms, 5)}
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    tname = (pre_name or dec_name) + (":w4a8" if w4a8 else "")
    if os.path.exists(tfile):
        try:
            rec = json.load(open(tfile)).get(tname)
            if rec and rec.get("kernel_sha") == kernel_sha():
                traffic = rec["hbm_bytes"]
        except Exception:
            traffic = None
    roof["traffic"] = traffic
    result["roofline"] = roof
    if not args.no_cpu_baseline and cp.op == "fwd":
        result["cpu_baseline"] = cpu_baseline(cp, args.seed, args.cpu_budget, result["unit"], w4a8=w4a8)
        result["cpu_baseline"].update(host_info())
    result["kernel_sha"] = kernel_sha()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
