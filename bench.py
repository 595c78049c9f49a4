#!/usr/bin/env python3
"""Q4_0 linear-layer benchmark on one MI355X.

Headline: batched-decode GEMV weight GB/s on the 5120 x 5120 attention
projection (M = 1, 4, 10, 16 per step, fp16 activations, fp16 output), with
the packed weights rotated over >= 1 GiB of distinct copies so every launch
streams from HBM rather than the 256 MB last-level cache.  One step = one
GEMV launch per batch size, each on its own weight copy.

The same JSON line carries:
  roofline      -- the dominant GEMV launch: weight bytes / mean launch time
                   (HIP events on the launch stream) against 8 TB/s HBM;
  gemm          -- prefill GEMM on the 2048 x 17408 x 5120 workload, whole
                   batch and 8 chunks of 256 rows, TFLOP/s against fp16 MFMA;
  quantize      -- the quantiser on the same 5120 x 5120 fp32 weight;
  cpu_baseline  -- the CPU oracle timed on a bounded sample of the step.

Run: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "Q4_0 GEMV weight GB/s + GEMM TFLOPS, as % of MI355X HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 matrix peak
BLOCK_BYTES, QK = 18, 32


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted((ROOT / "bit_block_quantized_q4_amd" / "csrc").glob("*")):
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernels changed since the counters were taken."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        data = json.loads(f.read_text())
    except ValueError:
        return None
    if data.get("source_hash") != kernel_source_hash():
        return None
    return data.get("kernels", {}).get(kernel_key)


def events_elapsed_ms(pairs):
    return [s.elapsed_time(e) for s, e in pairs]


def bench_gemv(q4, torch, dev, steps, warmup, rotate_bytes):
    import synth
    wl = synth.WORKLOADS[2]
    lin = wl.linears[0]
    n, k = lin.n, lin.k
    wbytes = n * (k // QK) * BLOCK_BYTES
    w = synth.workload_weights(wl, lin)
    wd = torch.from_numpy(w).to(dev)
    ncopies = max(4, -(-rotate_bytes // wbytes))
    packed = [q4.q4_quantize(wd) for _ in range(ncopies)]
    ms = list(wl.ms)
    x = torch.from_numpy(synth.workload_activations(wl, k, max(ms))).to(dev)
    ys = {m: torch.empty((m, n), dtype=torch.float16, device=dev) for m in ms}
    torch.cuda.synchronize()

    launch = [0]

    def step(record=None):
        for m in ms:
            p = packed[launch[0] % ncopies]
            launch[0] += 1
            if record is not None:
                s = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                s.record()
            q4.q4_gemv(x[:m], p, y=ys[m])
            if record is not None:
                e.record()
                record[m].append((s, e))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    rec = {m: [] for m in ms}
    t0 = time.perf_counter()
    for _ in range(steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_m = []
    for m in ms:
        d = np.array(events_elapsed_ms(rec[m]))
        avg_s = float(d.mean()) * 1e-3
        per_m.append({
            "m": m, "mean_us": avg_s * 1e6, "p10_us": float(np.percentile(d, 10)) * 1e3,
            "p90_us": float(np.percentile(d, 90)) * 1e3,
            "weight_gbs": wbytes / avg_s / 1e9,
            "total_gbs": (wbytes + m * k * 2 + m * n * 2) / avg_s / 1e9,
            "frac_hbm": wbytes / avg_s / 1e9 / HBM_PEAK_GBS,
        })
    step_s = wall / steps
    return {
        "wl": wl, "n": n, "k": k, "ms": ms, "wbytes": wbytes, "ncopies": ncopies,
        "step_s": step_s, "value_gbs": wbytes * len(ms) / step_s / 1e9, "per_m": per_m,
        "w_host": w, "packed0": packed[0],
    }


def bench_quantize(q4, torch, dev, w_host, reps, rotate_bytes):
    n, k = w_host.shape
    in_bytes = n * k * 4
    copies = max(2, -(-rotate_bytes // in_bytes))
    ws = [torch.from_numpy(w_host).to(dev) for _ in range(copies)]
    out = torch.empty((n, (k // QK) * BLOCK_BYTES), dtype=torch.uint8, device=dev)
    for i in range(3):
        q4.q4_quantize(ws[i % copies], packed=out)
    torch.cuda.synchronize()
    pairs = []
    for i in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        q4.q4_quantize(ws[i % copies], packed=out)
        e.record()
        pairs.append((s, e))
    torch.cuda.synchronize()
    avg_s = float(np.mean(events_elapsed_ms(pairs))) * 1e-3
    alg = n * k * 4 + n * (k // QK) * BLOCK_BYTES
    gbs = alg / avg_s / 1e9
    return {"workload": "quantize_fp32_5120x5120", "mean_us": avg_s * 1e6,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("quantize_fp32_5120x5120")}}


def bench_gemm(q4, torch, dev, reps):
    import synth
    wl = synth.WORKLOADS[4]
    lin = wl.linears[0]
    n, k, m = lin.n, lin.k, 2048
    w = synth.workload_weights(wl, lin)
    packed = q4.q4_quantize(torch.from_numpy(w).to(dev))
    del w
    x = torch.from_numpy(synth.workload_activations(wl, k, m)).to(dev)
    y = torch.empty((m, n), dtype=torch.float16, device=dev)
    ws = q4.q4_gemm_workspace_size(m, n, k)
    wsc = q4.q4_gemm_workspace_size(256, n, k)
    work = torch.empty(max(ws, wsc, 1), dtype=torch.uint8, device=dev)

    def whole():
        q4.q4_gemm(x, packed, y=y, workspace=work)

    def chunks():
        for c in range(8):
            q4.q4_gemm(x[c * 256:(c + 1) * 256], packed, y=y[c * 256:(c + 1) * 256], workspace=work)

    res = {}
    for name, fn, calls in (("whole_2048", whole, 1), ("chunked_8x256", chunks, 8)):
        fn()
        torch.cuda.synchronize()
        pairs = []
        for _ in range(reps):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            pairs.append((s, e))
        torch.cuda.synchronize()
        avg_s = float(np.mean(events_elapsed_ms(pairs))) * 1e-3
        tf = 2.0 * m * n * k / avg_s / 1e12
        res[name] = {"mean_us": avg_s * 1e6, "launches": calls, "tflops": tf,
                     "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS}
    best = res["whole_2048"]["tflops"]
    return {
        "workload": "prefill_chunked_2048x17408x5120", "m": m, "n": n, "k": k,
        **res,
        "roofline": {"bound": "mfma", "achieved": best, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": best / MFMA_F16_PEAK_TFLOPS,
                     "traffic": load_traffic("gemm_2048x17408x5120")},
    }


def cpu_baseline(w_host, n, k, ms, budget_s=12.0):
    """The oracle, untuned, on the decode step (all four batch sizes)."""
    import oracle
    import synth
    wl = synth.WORKLOADS[2]
    packed = oracle.quantize(w_host)
    xs = {m: synth.workload_activations(wl, k, m) for m in ms}
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    t0 = time.perf_counter()
    steps = 0
    while True:
        for m in ms:
            oracle.matmul_ref(xs[m], packed, n, k)
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = (time.perf_counter() - t0) / steps
    wbytes = n * (k // QK) * BLOCK_BYTES
    return {"value": wbytes * len(ms) / el / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} full decode steps (M={ms}) of the 5120x5120 workload, "
                      f"{el:.2f} s per step"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-mib", type=int, default=1024)
    ap.add_argument("--gemm-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "gemv", "gemm", "quantize"], default="all")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Q4_0 path has no multi-GPU leg "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_block_quantized_q4_amd as q4
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    q4.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    rotate = args.rotate_mib << 20

    out = {"metric": METRIC}
    g = bench_gemv(q4, torch, dev, args.steps, args.warmup, rotate)
    dom = max(g["per_m"], key=lambda r: r["mean_us"])
    out.update({
        "value": g["value_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": g["step_s"] * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": g["wl"].name, "n": g["n"], "k": g["k"], "ms": g["ms"],
                   "x_dtype": "f16", "y_dtype": "f16",
                   "weight_copies_rotated": g["ncopies"],
                   "weight_bytes_per_launch": g["wbytes"]},
        "roofline": {"bound": "hbm", "achieved": dom["weight_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dom["weight_gbs"] / HBM_PEAK_GBS,
                     "traffic": load_traffic(f"gemv_5120x5120_m{dom['m']}"),
                     "kernel": f"q4_gemv m={dom['m']}"},
        "per_m": g["per_m"],
    })
    if args.only in ("all", "quantize"):
        out["quantize"] = bench_quantize(q4, torch, dev, g["w_host"], 20, rotate)
    if args.only in ("all", "gemm"):
        out["gemm"] = bench_gemm(q4, torch, dev, args.gemm_reps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(g["w_host"], g["n"], g["k"], g["ms"])
    out["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
