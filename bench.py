#!/usr/bin/env python3
"""Throughput of the MI355X WKV-6 forward (tokens/s = B*T per second).

One step = one wkv6_fwd call (the whole hot path: load, decay transform,
in-chunk scans, MFMA contractions, state carries in both directions, merge and
store) over one batch of synthetic input already resident in HBM.  Inputs and
outputs rotate over enough copies that no step finds its data in the 256 MB
Infinity Cache left by the previous steps.

Prints ONE JSON line (rank 0) with, besides the throughput:
  roofline      achieved HBM bandwidth of the call from HIP events on the launch
                stream: algorithmic bytes per call / mean call time (the call is
                the sweep kernel, for bf16 inputs the fast-path sweep plus a
                fix-up kernel that finds no work unless a chunk needed the slow
                path, plus the segment summary kernels when a sequence is
                split); traffic = bytes the
                committed rocprofv3 counter runs measured for the same sources
  mfma          executed matrix-core work per call and its rate vs the bf16 peak
  cpu_baseline  the float64 CPU oracle timed on the host on a bounded sample

--op selects another entry point of the library on the same workload shapes
(default wkv6_fwd, the headline):
  wkv6_bwd   the backward (gradients of sum(y * dy)): on long bf16 sequences
             the chunked MFMA kernels, reported against the HBM roofline;
             otherwise token-serial float32 vector arithmetic, whose roofline
             is the fp32 vector peak over the algorithmic flops (12 N^2 per
             token, head and direction)
  wkv6_fwd_gn  the forward with the per-head group normalisation, affine and
             gate fused into its output (bf16 out; y never written)
  wkv6_fwd_then_gn  the same result in the unfused order: wkv6_fwd, then
             wkv6_group_norm_gate on its y (same algorithmic bytes as the
             fused op, so the two lines compare call times directly)
  wkv5_fwd   RWKV-5: the forward with one decay per channel for every token
  wkv4_fwd   RWKV-4: the normalised per-channel operator (always causal)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_rnn_amd import inputs as I  # noqa: E402

HEADLINE = "text-long-causal-bf16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak, published
OPS = ("wkv6_fwd", "wkv6_bwd", "wkv6_fwd_gn", "wkv6_fwd_then_gn", "wkv5_fwd", "wkv4_fwd")
MALL_BYTES = 256 << 20
MFMA_FLOPS = 2 * 16 * 16 * 32  # one v_mfma_f32_16x16x32_bf16
METRIC = "WKV6 fwd tokens/s (B·T/s) + % HBM roofline & MFMA util at N=64, 1 GPU"


# The sources the forward kernels are compiled from.
FWD_SOURCES = ("wkv6_device.h", "wkv6_internal.h", "wkv6_kernels.hip")


def kernel_source_hash() -> str:
    """Hash of the forward kernels' sources (their .hip file and the headers
    it includes) with comments and blank lines stripped, so that a recorded
    counter run stays matched to the kernels it measured; host-only code and
    the other entry points' kernels are left out."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_rnn_amd", "csrc")
    for name in FWD_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(name.encode() + code.encode())
    return h.hexdigest()[:16]


def plan_segments(w: I.Workload) -> tuple[int, int]:
    """(segments per sequence, chunks per segment) as the library picks them."""
    nc = math.ceil(w.T / 64)
    bh = w.B * w.H
    env = os.environ.get("WKV6_SEGMENTS")
    if env:
        g = int(env)
    else:
        target = 256 * (3 if w.dtype == "bf16" else 2)
        g = math.ceil(target / bh) if bh < target else 1
        if w.dtype == "bf16" and bh < target:
            # the library prefers a grid with as many workgroups on every CU
            for per in (3, 2):
                want = 256 * per
                if want % bh == 0 and want // bh <= nc and math.ceil(nc / math.ceil(nc / (want // bh))) == want // bh:
                    g = want // bh
                    break
    g = max(1, min(g, nc))
    segc = math.ceil(nc / g)
    return math.ceil(nc / segc), segc


def mfma_count(w: I.Workload) -> int:
    """v_mfma_f32_16x16x32_bf16 instructions one call issues on the fast path
    (mirrors the kernels' loop structure: per chunk and wave, the score tiles
    up to the wave's own block, the score x value products, the product with
    the carried state, and the state update)."""
    sp, sv = (2, 1) if w.dtype == "bf16" else (3, 3)

    def prods(sa, sb):
        m = max(sa, sb)
        return sum(1 for d in range(m) for i in range(d + 1) if i < sa and d - i < sb)

    def sweep(n, out, have_s):
        nch, tot = math.ceil(n / 64), 0
        for ch in range(nch):
            lv = min(64, n - 64 * ch)
            if out:
                for J in range(4):
                    if 16 * J >= lv:
                        continue
                    tot += (J + 1) * 2 * prods(sp, sp)
                    tot += (J // 2 + 1) * 4 * prods(sv, sp)
                    if ch > 0 or have_s:
                        tot += 2 * 4 * prods(sp, sp)
            if not (out and ch == nch - 1):
                tot += 4 * (2 if lv > 32 else 1) * 4 * prods(sp, sv)
        return tot

    g, segc = plan_segments(w)
    bidir = w.mode == "bidirectional"
    per_bh = 0
    for seg in range(g):
        n = min(w.T, (seg + 1) * segc * 64) - seg * segc * 64
        per_bh += sweep(n, True, seg > 0)
        if bidir:
            per_bh += sweep(n, True, seg < g - 1)
        if g > 1:
            if seg < g - 1:
                per_bh += sweep(n, False, False)
            if bidir and seg > 0:
                per_bh += sweep(n, False, False)
    return per_bh * w.B * w.H


def bwd_path(w: I.Workload) -> str:
    """Which kernels the library's backward planner picks for this workload:
    the chunked MFMA kernels take bf16 calls of at least 64 tokens that run
    unsegmented (at least 256 (batch, head) pairs, or fewer than 128
    tokens)."""
    unsegmented = w.B * w.H >= 256 or w.T < 128
    return "chunked" if w.dtype == "bf16" and w.T >= 64 and unsegmented else "token-serial"


def traffic_record(workload: str):
    """HBM bytes per call from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(w: I.Workload, x: dict, budget_s: float = 20.0, op: str = "wkv6_fwd") -> dict:
    """Time the float64 oracle of the op on whole batch items of the same
    workload until about `budget_s` seconds of CPU work, single-threaded."""
    from threadpoolctl import threadpool_limits

    import oracle

    def run(nb):
        if op == "wkv6_fwd":
            oracle.wkv6_ref(x["r"][:nb], x["k"][:nb], x["v"][:nb], x["w_raw"][:nb], x["u"], w.H, w.mode)
        elif op == "wkv6_bwd":
            oracle.wkv6_ref_backward(x["r"][:nb], x["k"][:nb], x["v"][:nb], x["w_raw"][:nb], x["u"],
                                     x["dy"][:nb], w.H, w.mode)
        elif op in ("wkv6_fwd_gn", "wkv6_fwd_then_gn"):
            oracle.wkv6_gn_ref(x["r"][:nb], x["k"][:nb], x["v"][:nb], x["w_raw"][:nb], x["u"], x["g"][:nb],
                               x["gamma"], x["beta"], 64e-5, w.H, w.mode)
        elif op == "wkv5_fwd":
            oracle.wkv5_ref(x["r"][:nb], x["k"][:nb], x["v"][:nb], x["w_raw"], x["u"], w.H, w.mode)
        else:
            oracle.wkv4_ref(x["k"][:nb], x["v"][:nb], x["w"], x["u"])

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        run(1)
        t1 = time.perf_counter() - t0
        nb = max(1, min(w.B, int(budget_s / max(t1, 1e-3))))
        if nb > 1:
            t0 = time.perf_counter()
            run(nb)
            el = time.perf_counter() - t0
        else:
            el = t1
    mode = "causal" if op == "wkv4_fwd" else w.mode
    return {"value": nb * w.T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{nb} of {w.B} batch items (T={w.T}, C={w.C}, H={w.H}, {mode}, {op} oracle, "
                      f"float64 numpy recurrence, BLAS limited to 1 thread), {el:.1f} s"}


def copy_calibration(torch, mib: int, steps: int, warmup: int) -> int:
    """Copy mib MiB between two device buffers, steps times after warmup
    copies: a kernel whose HBM bytes are known exactly (mib MiB read and mib
    MiB written per launch), so rocprofv3's FETCH_SIZE / WRITE_SIZE readings
    for it give the factor that turns those counters into bytes."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": steps + warmup, "ms_per_copy": ms,
                      "copy_GBps": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=[x.name for x in I.WORKLOADS])
    ap.add_argument("--op", default="wkv6_fwd", choices=OPS,
                    help="library entry point to time (default: the headline forward)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-rotate", action="store_true",
                    help="reuse one input set (warm Infinity Cache; not the headline number)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="instead of the operator, time a plain device-to-device copy of MIB "
                         "MiB (reference kernel for scaling rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library and this benchmark run on one GPU only (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        return copy_calibration(torch, args.copy_calibration, args.steps, args.warmup)

    from linear_attention_rnn_amd import wkv6

    def dev(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(I.bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    w = I.workload(args.workload)
    op = args.op
    isz = 2 if w.dtype == "bf16" else 4
    E = w.elements
    mode = "causal" if op == "wkv4_fwd" else w.mode
    if op == "wkv6_fwd":
        x = I.make_inputs(w)
        per_copy = w.algorithmic_bytes()
    elif op == "wkv6_bwd":
        x = I.make_inputs(w)
        x["dy"] = np.random.default_rng(w.seed + 1000).normal(0.0, 0.5, size=(w.B, w.T, w.C)).astype(np.float32)
        # read r, k, v, w_raw, dy and u; write dr, dk, dv, dw_raw and du
        per_copy = E * (4 * isz + 4 + 16) + 2 * w.C * 4
    elif op in ("wkv6_fwd_gn", "wkv6_fwd_then_gn"):
        x = I.make_inputs(w)
        rng = np.random.default_rng(w.seed + 2000)
        x["g"] = rng.normal(size=(w.B, w.T, w.C)).astype(np.float32)
        if w.dtype == "bf16":
            x["g"] = I.round_to_bf16(x["g"])
        x["gamma"] = rng.uniform(0.5, 1.5, size=w.C).astype(np.float32)
        x["beta"] = rng.normal(0.0, 0.3, size=w.C).astype(np.float32)
        # read r, k, v, w_raw, g and u, gamma, beta; write the bf16 output
        per_copy = E * (5 * isz + 2) + 3 * w.C * 4
    elif op == "wkv5_fwd":
        x = I.random_inputs_wkv5(w.B, w.T, w.C, seed=w.seed, dtype=w.dtype, wraw_lo=w.wraw_lo, wraw_hi=w.wraw_hi)
        per_copy = E * (3 * isz + 4) + w.C * (isz + 4)
    else:
        x = I.random_inputs_wkv4(w.B, w.T, w.C, seed=w.seed, dtype=w.dtype)
        per_copy = E * (2 * isz + 4) + 2 * w.C * 4
    ncopy = 1 if args.no_rotate else max(2, math.ceil(2 * MALL_BYTES / per_copy) + 1)
    sets = []
    for _ in range(ncopy):
        if op == "wkv4_fwd":
            d = [dev(x["k"], w.dtype), dev(x["v"], w.dtype), f32(x["w"]), f32(x["u"])]
        else:
            d = [dev(x[key], w.dtype) for key in ("r", "k", "v", "w_raw")] + [f32(x["u"])]
        if op == "wkv6_bwd":
            d.append(f32(x["dy"]))
        if op in ("wkv6_fwd_gn", "wkv6_fwd_then_gn"):
            d += [dev(x["g"], w.dtype), f32(x["gamma"]), f32(x["beta"])]
        y = torch.empty((w.B, w.T, w.C), dtype=torch.bfloat16 if op in ("wkv6_fwd_gn", "wkv6_fwd_then_gn")
                        else torch.float32, device="cuda") if op != "wkv6_bwd" else None
        if op == "wkv6_fwd_then_gn":   # the forward's y between the two passes
            d.append(torch.empty((w.B, w.T, w.C), dtype=torch.float32, device="cuda"))
        sets.append((d, y))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(i):
        d, y = sets[i % ncopy]
        if op == "wkv6_fwd":
            wkv6.fwd(*d, w.H, w.mode, out=y, stream=stream)
        elif op == "wkv6_bwd":
            wkv6.bwd(*d, w.H, w.mode, stream=stream)
        elif op == "wkv6_fwd_gn":
            wkv6.fwd_gn(*d, w.H, w.mode, out=y, stream=stream)
        elif op == "wkv6_fwd_then_gn":
            r_, k_, v_, w_, u_, g_, ga_, be_, ybuf = d
            wkv6.fwd(r_, k_, v_, w_, u_, w.H, w.mode, out=ybuf, stream=stream)
            wkv6.group_norm_gate(ybuf, g_, ga_, be_, w.H, eps=64e-5, out=y, stream=stream)
        elif op == "wkv5_fwd":
            wkv6.fwd5(*d, w.H, w.mode, out=y, stream=stream)
        else:
            wkv6.fwd4(*d, out=y, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(args.warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    mean_ms = float(np.mean(per_call_ms))
    ms_per_step = 1e3 * wall / args.steps

    alg_bytes = per_copy
    achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
    forward6 = op in ("wkv6_fwd", "wkv6_fwd_gn", "wkv6_fwd_then_gn", "wkv5_fwd")   # the chunked MFMA kernels
    n_mfma = mfma_count(w) if forward6 else 0
    mfma_tflops = n_mfma * MFMA_FLOPS / (mean_ms * 1e-3) / 1e12
    traffic = traffic_record(w.name) if op == "wkv6_fwd" else None
    if op == "wkv6_bwd":
        # algorithmic fp32 work: per token, head and direction the state and
        # adjoint updates (3 N^2 each: a product and a fused multiply-add per
        # entry) and the dr, dk, dv contractions (2 N^2 each)
        flops = 12 * w.N * w.N * w.B * w.T * w.H * (2 if w.mode == "bidirectional" else 1)
        tflops = flops / (mean_ms * 1e-3) / 1e12
        if bwd_path(w) == "chunked":
            # matrix-core kernels: bounded by the HBM bytes
            roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                        "kernel": "wkv6_bwd call: chunked MFMA kernels (chunk states, gradients) + u reduction",
                        "mean_call_ms": mean_ms, "algorithmic_bytes": alg_bytes,
                        "algorithmic_flops": flops, "fp32_tflops": tflops}
        else:
            roofline = {"bound": "alu", "achieved": tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tflops / FP32_VECTOR_PEAK_TFLOPS, "traffic": None,
                        "kernel": "wkv6_bwd call: token-serial backward sweeps + u reduction",
                        "mean_call_ms": mean_ms, "algorithmic_flops": flops,
                        "hbm_achieved_GBps": achieved, "algorithmic_bytes": alg_bytes}
    else:
        # bf16 sweeps run the fast path and leave slow chunks to a fix-up
        # launch; float32 sweeps carry the general sweeps themselves
        sweep = "fast-path sweep kernel" if w.dtype == "bf16" else "sweep kernel"
        fix = " + fix-up kernel" if w.dtype == "bf16" else ""
        kern = {"wkv6_fwd": f"wkv6_fwd call: {sweep}{fix}",
                "wkv6_fwd_gn": f"wkv6_fwd_gn call: {sweep} with the fused epilogue{fix}",
                "wkv6_fwd_then_gn": "wkv6_fwd call, then wkv6_group_norm_gate on its y (the unfused order)",
                "wkv5_fwd": f"wkv5_fwd call: {sweep}{fix}",
                "wkv4_fwd": "wkv4_fwd call: per-channel recurrence kernels"}[op]
        if forward6 and plan_segments(w)[0] > 1:
            kern += " + segment summary kernels"
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kern,
                    "mean_call_ms": mean_ms, "algorithmic_bytes": alg_bytes}
    metric = METRIC if op == "wkv6_fwd" else METRIC.replace("WKV6 fwd", op.upper().replace("_", " "))

    out = {
        "metric": metric,
        "value": w.tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if (w.dtype == "bf16" and forward6) else "f32",
        "data": "synthetic (seeded numpy draws, recipe in linear_attention_rnn_amd/inputs.py)",
        "config": {"workload": w.name, "op": op, "mode": mode, "B": w.B, "T": w.T, "C": w.C, "H": w.H,
                   "N": w.N, "inputs": w.dtype,
                   "state_and_output": "f32 state, bf16 output" if op in ("wkv6_fwd_gn", "wkv6_fwd_then_gn") else "f32",
                   "rotating_copies": ncopy, "parallelism": "single GPU"},
        "roofline": roofline,
    }
    if forward6:
        out["mfma"] = {"instructions": n_mfma, "executed_tflops": mfma_tflops,
                       "util": mfma_tflops / MFMA_BF16_PEAK_TFLOPS, "peak_tflops": MFMA_BF16_PEAK_TFLOPS}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget, op)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
