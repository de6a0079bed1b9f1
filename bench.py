#!/usr/bin/env python3
"""Benchmark of the strided-layout GEMM on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-vendor]

A step is one call of sl_gemm over the workload's operands, already resident
in HBM.  W untimed steps (without --warmup: at least 10 steps and at least
one second of them, so that the timed region runs at the clock the chip
sustains under this load -- from idle it takes a fraction of a second to
get there, and 10 warm-up steps of the 8192^3 default left the next 50
3-4% slow), then K steps timed between two device synchronisations; HIP events on the launch stream give the kernel's
average duration for the roofline object (for the HBM-bound workloads, the
median of launches timed after a 512 MiB read, so that the inputs come from
HBM rather than the Infinity Cache).  Prints one JSON line.

Default workload: fp16 TN GEMM M = N = K = 8192 with C (normal(0,1) inputs,
seed 1) -- the large square case the fp16 throughput target is stated on.
Other workloads (for measurement only): fp16_4096 (the same recipe at 4096),
ragged (4000x3000x2056), skinny (8192x128x8192), batched_nn / batched_nt
(64 x 512^3, A M-contiguous), batched_tn / batched_tt (A K-contiguous),
mxfp8 (8192^3 MXFP8), nvfp4_8192 / mxfp4_8192 (8192^3 NVFP4 / MXFP4),
bf16_8192 (the default recipe in bf16).

The CPU baseline is the oracle (plain fp64 triple loop, all host cores) on a
bounded sample of output points of the same workload, scaled to TFLOP/s.
For context (not a baseline), the single fp16 and MXFP8 products are also
timed through PyTorch's calls into the vendor library on the same operands
("vendor_library" in the JSON line; --no-vendor skips it).
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

METRIC = "TFLOP/s and % of dense MFMA peak, fp16 TN GEMM 4096^3/8192^3 on 1 MI355X"
PEAK_F16 = 2516.6   # TFLOP/s: 256 CUs x 2.4 GHz x 4096 dense fp16 FLOP/clk/CU
PEAK_F8 = 5033.2    # TFLOP/s: 256 CUs x 2.4 GHz x 8192 dense MX-fp8 FLOP/clk/CU
PEAK_F4 = 10066.3   # TFLOP/s: 256 CUs x 2.4 GHz x 16384 dense MX-fp4 FLOP/clk/CU
PEAK_HBM = 8000.0   # GB/s


def workloads():
    from stride_layouts_lds_amd import inputs as I
    return {
        "fp16_8192": ("fp16 TN GEMM M=N=K=8192, A/B/C normal(0,1) fp16, seed 1", lambda: I.config2(8192)),
        "fp16_4096": ("fp16 TN GEMM M=N=K=4096, A/B/C normal(0,1) fp16, seed 1", lambda: I.config2(4096)),
        "ragged": ("fp16 TN GEMM 4000x3000x2056, uniform[-1,1], C=0, seed 2", lambda: I.config3()[0]),
        "skinny": ("fp16 TN GEMM 8192x128x8192, uniform[-1,1], C=0, seed 2", lambda: I.config3()[1]),
        "batched_nn": ("fp16 batched 64x512^3, A M-contiguous, B K-contiguous, seed 3", lambda: I.config4("NN")),
        "batched_nt": ("fp16 batched 64x512^3, A M-contiguous, B N-contiguous, seed 3", lambda: I.config4("NT")),
        "batched_tn": ("fp16 batched 64x512^3, A and B K-contiguous, seed 3", lambda: I.config4("TN")),
        "batched_tt": ("fp16 batched 64x512^3, A K-contiguous, B N-contiguous, seed 3", lambda: I.config4("TT")),
        "mxfp8": ("MXFP8 GEMM M=N=K=8192, E4M3 data, E8M0 scale per 32 K, C=0, seed 4", lambda: I.config5(8192)),
        "nvfp4_8192": ("NVFP4 GEMM M=N=K=8192, E2M1 codes uniform, E4M3 scale per 16 K (2^[-4,0] x any mantissa), "
                       "C=0, seed 6", lambda: I.nvfp4_workload("nvfp4_8192", 8192, 8192, 8192, seed=6)),
        "mxfp4_8192": ("MXFP4 GEMM M=N=K=8192, E2M1 codes uniform, E8M0 scale per 32 K (2^[-4,0]), C=0, seed 7",
                       lambda: I.mxfp4_workload("mxfp4_8192", 8192, 8192, 8192, seed=7)),
        "mxfp6_8192": ("MXFP6 GEMM M=N=K=8192, FP6 E2M3 codes uniform, E8M0 scale per 32 K (2^[-4,0]), C=0, "
                       "seed 8", lambda: I.mxfp6_workload("mxfp6_8192", 8192, 8192, 8192, seed=8)),
        "bf16_8192": ("bf16 TN GEMM M=N=K=8192, A/B/C normal(0,1) bf16, seed 1",
                      lambda: I.gemm_workload("bf16_tn_8192_c", 8192, 8192, 8192, seed=1, dist="normal",
                                              with_c=True, bf16=True)),
    }


def algorithmic_bytes(w) -> int:
    """A, B (and scales) read once, C read once if present, D written once."""
    es = 0.5 if w.fp4 else 0.75 if w.fp6 else 1 if w.mx else 2
    b = int(w.batch * (w.M * w.K + w.N * w.K) * es) + w.batch * w.M * w.N * 2
    if w.c is not None:
        b += w.batch * w.M * w.N * 2
    if w.mx:
        b += w.sfa.storage.size + w.sfb.storage.size
    return b


def source_hash() -> str:
    """Hash of the sources that decide what runs on the GPU (kernels, device
    headers, the planner); the host-only layout algebra and plan trace are
    left out."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "stride_layouts_lds_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.startswith(("layout_algebra.", "describe.")):
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, target_s: float = 12.0):
    """The oracle, as it stands, on a bounded sample of output points."""
    import numpy as np
    from oracle import gemm as OG
    threads = max(1, len(os.sched_getaffinity(0)))
    rng = np.random.default_rng(123)

    def ora(op, code=None):
        if op is None:
            return None
        if code is not None:  # raw storage with element strides (packed E2M1 / 6-bit, NVFP4 scales)
            return OG.packed(op.storage, op.shape, op.strides, code)
        return op.view
    if w.nvfp4:
        ops = (ora(w.a, OG.E2M1), ora(w.b, OG.E2M1), ora(w.c), ora(w.sfa, OG.E4M3), ora(w.sfb, OG.E4M3))
    elif w.mxfp4:
        ops = (ora(w.a, OG.E2M1), ora(w.b, OG.E2M1), ora(w.c), ora(w.sfa), ora(w.sfb))
    elif w.fp6:
        code = OG.E2M3 if w.a.kind == "e2m3" else OG.E3M2
        ops = (ora(w.a, code), ora(w.b, code), ora(w.c), ora(w.sfa), ora(w.sfb))
    else:
        ops = (ora(w.a), ora(w.b), ora(w.c), ora(w.sfa), ora(w.sfb))

    def run(n, nthreads):
        pts = np.stack([rng.integers(0, w.batch, n), rng.integers(0, w.M, n), rng.integers(0, w.N, n)], 1)
        t0 = time.perf_counter()
        OG.gemm_points(*ops, points=pts, block_k=w.block_k, nthreads=nthreads, bf16=w.bf16)
        return time.perf_counter() - t0

    def timed(nthreads, seconds):
        n = max(nthreads * 4, 64)
        dt = run(n, nthreads)
        while dt < 0.5:
            n *= 4
            dt = run(n, nthreads)
        n = max(n, int(n * seconds / dt))
        return n, run(n, nthreads)

    n, dt = timed(threads, target_s)
    flop = 2.0 * w.K * n
    # the same oracle on one thread, on a smaller sample
    n1, dt1 = timed(1, target_s / 4)
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} output elements of the same workload (each a {w.K}-term fp64 dot product), "
                      f"{dt:.1f} s on {threads} threads",
            "single_thread": {"value": round(2.0 * w.K * n1 / dt1 / 1e12, 6), "unit": "TFLOP/s",
                              "sample": f"{n1} output elements, {dt1:.1f} s on 1 thread"}}


def vendor_timing(w, a, b, c, sfa, sfb, out, stream, reps: int = 20):
    """The vendor library through PyTorch on the same device operands, for
    context (not a baseline): torch.addmm / torch.mm for the single fp16
    products with K-contiguous A and B (C + A B^T), torch._scaled_mm with
    E8M0 block scales for MXFP8.  Average launch time over `reps` launches
    between HIP events on the launch stream after at least a second of
    back-to-back warm-up calls, and the relative Frobenius
    difference of its D from the library's (`out`, which holds the
    library's result).  None for the other workloads."""
    import torch
    if w.mx and (w.fp4 or w.fp6 or w.nvfp4) or (not w.mx and w.bf16):
        return None  # packed formats, and bf16 (kept off the vendor's bf16 path here)
    if not isinstance(a, torch.Tensor) or not isinstance(b, torch.Tensor):
        return None
    if w.batch != 1 or a.dim() != 2 or b.dim() != 2 or a.stride(1) != 1 or b.stride(1) != 1:
        return None
    if w.mx and w.block_k == 32 and w.c is None:
        name = "torch._scaled_mm (E4M3 data, E8M0 scale per 32 K)"
        sa, sb = sfa.view(torch.float8_e8m0fnu), sfb.view(torch.float8_e8m0fnu)
        a8, b8 = a.view(torch.float8_e4m3fn), b.view(torch.float8_e4m3fn)

        def fn():
            return torch._scaled_mm(a8, b8.t(), scale_a=sa, scale_b=sb, out_dtype=torch.float16)
    elif not w.mx and not w.bf16:
        name = "torch.addmm(C, A, B^T)" if c is not None else "torch.mm(A, B^T)"

        def fn():
            return torch.addmm(c, a, b.t()) if c is not None else torch.mm(a, b.t())
    else:
        return None
    try:
        r = fn()
        torch.cuda.synchronize()
    except Exception as e:  # this PyTorch build has no such path
        return {"call": name, "error": f"{type(e).__name__}: {str(e)[:200]}"}
    ref = out.float()
    diff = ((r.float() - ref).norm() / ref.norm().clamp_min(1e-30)).item()
    del r
    # the same warm-up as the library's default: at least one second of
    # back-to-back calls, so that both are timed at the sustained clock
    n, t_w = 0, time.perf_counter()
    while n < 10 or time.perf_counter() - t_w < 1.0:
        for _ in range(10):
            fn()
        n += 10
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"call": name, "launches": reps, "us_per_launch": round(us, 1),
            "tflops": round(w.flops / (us * 1e-6) / 1e12, 1), "rel_diff_from_library": float(f"{diff:.3e}")}


def per_launch_timing(api, margs, sid, stream, reps: int) -> dict:
    """Per-launch event timings, median and best: back to back ("warm": the
    inputs may sit in the 256 MB Infinity Cache from the previous launch) and
    "cold", after reading a 512 MiB buffer before each launch so that the
    inputs come from HBM.  The flush reads rather than writes: a written
    buffer would leave the cache full of dirty lines whose write-back then
    lands inside the timed launch."""
    import torch
    flush = torch.ones((512 << 20) // 4, dtype=torch.float32, device="cuda")
    out = {}
    for kind in ("warm", "cold"):
        ts = []
        for r in range(reps):
            if kind == "cold":
                flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            api.sl_gemm(margs, sid)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        out[kind + "_median_us"] = round(ts[len(ts) // 2], 2)
        out[kind + "_best_us"] = round(ts[0], 2)
    out["reps"] = reps
    out["flush_bytes"] = flush.numel() * 4
    del flush
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed region (default: at least 10 and at least 1 s of them)")
    ap.add_argument("--workload", default="fp16_8192")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip timing the vendor library (through PyTorch) on the same operands")
    ap.add_argument("--per-launch", type=int, default=30,
                    help="launches for the per-launch warm and cold timings after the timed region (0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 times), the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 1 << 30
        x = torch.empty(n // 2, dtype=torch.float16, device="cuda").normal_()
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    from stride_layouts_lds_amd import api
    api.lib()

    desc, make = workloads()[args.workload]
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    w = make()
    from stride_layouts_lds_amd.inputs import to_device
    a, b, c = to_device(w.a), to_device(w.b), to_device(w.c)
    sfa, sfb = to_device(w.sfa), to_device(w.sfb)
    out = torch.empty(w.d_shape, dtype=torch.bfloat16 if w.bf16 else torch.float16, device="cuda")
    margs = api.make_args(a, b, c, out, sfa, sfb, w.block_k)
    ws = api.workspace_for(margs)  # a split-K plan's fp32 partial sums (caller-owned)
    api.set_workspace(margs, ws)
    plan = api.sl_gemm_plan(margs)
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream

    print(f"[bench] plan {plan}", file=sys.stderr, flush=True)
    if args.warmup is None:
        warmup, t_w = 0, time.perf_counter()
        while warmup < 10 or time.perf_counter() - t_w < 1.0:
            for _ in range(10):
                api.sl_gemm(margs, sid)
            warmup += 10
            torch.cuda.synchronize()
    else:
        warmup = args.warmup
        for _ in range(warmup):
            api.sl_gemm(margs, sid)
    torch.cuda.synchronize()
    print(f"[bench] {warmup} warm-up steps", file=sys.stderr, flush=True)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        api.sl_gemm(margs, sid)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {args.steps} steps in {wall:.4f} s; {kern_ms * 1e3:.1f} us per launch (events)",
          file=sys.stderr, flush=True)

    flop = w.flops
    peak = PEAK_F4 if (w.mxfp4 or w.fp6) else PEAK_F8 if (w.mx and not w.nvfp4) else PEAK_F16
    mfma_bound = flop / algorithmic_bytes(w) >= peak * 1e12 / (PEAK_HBM * 1e9)
    # an HBM-bound workload's roofline is taken from cold launches (inputs
    # read from HBM, not from the Infinity Cache), so those are always timed
    reps = args.per_launch if mfma_bound else max(args.per_launch, 30)
    timing = per_launch_timing(api, margs, sid, stream, reps=reps) if reps > 0 else None
    vendor = None if args.no_vendor else vendor_timing(w, a, b, c, sfa, sfb, out, stream)

    value = flop * args.steps / wall / 1e12
    # NVFP4 is decoded to fp16 and multiplied on the fp16 matrix cores;
    # MXFP4 runs on the scaled MFMAs at the fp4 rate
    # MXFP6 runs at the fp4 rate too (dense fp6 and fp4: 10.1 PFLOP/s)
    # The roofline that bounds the workload: MFMA when its arithmetic
    # intensity (algorithmic FLOP per algorithmic byte) is above the ridge
    # point peak / HBM bandwidth, HBM below it.
    if mfma_bound:
        achieved = flop / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    else:
        # cold launches: the median launch after a 512 MiB read, so that the
        # inputs come from HBM; the back-to-back rate is reported as "warm"
        cold_us = timing["cold_median_us"]
        achieved = algorithmic_bytes(w) / (cold_us * 1e-6) / 1e9
        warm = algorithmic_bytes(w) / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM, 4), "timing": "cold median launch",
                "warm": {"achieved": round(warm, 1), "frac": round(warm / PEAK_HBM, 4),
                         "timing": "timed-region average, inputs may sit in the Infinity Cache"}}
    roof["traffic"] = measured_traffic(args.workload)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f4e2m1" if w.fp4 else ("f6" + w.a.kind[1:]) if w.fp6 else "f8e4m3" if w.mx
                  else "bf16" if w.bf16 else "f16"),
        "data": "synthetic",
        "config": {"workload": desc, "M": w.M, "N": w.N, "K": w.K, "batch": w.batch,
                   "tile": f"{plan['tile_m']}x{plan['tile_n']}x{plan['tile_k']}",
                   "workgroups": plan["workgroups"], "peak_frac": round(value / peak, 4)},
        "roofline": roof,
        "timing": timing,
    }
    if vendor is not None:
        res["vendor_library"] = vendor
    if rank == 0 and not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w)
    if rank == 0:
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
