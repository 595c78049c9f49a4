#!/usr/bin/env python3
"""Q4_0 linear-layer benchmark on one MI355X.

Headline: batched-decode GEMV weight GB/s on the 5120 x 5120 attention
projection (M = 1, 4, 10, 16 per step, fp16 activations, fp16 output), with
the packed weights rotated over >= 1 GiB of distinct copies so every launch
streams from HBM rather than the 256 MB last-level cache.  One step = one
GEMV launch per batch size, each on its own weight copy.  The W warm-up steps
and the K timed steps are each recorded into a HIP graph and replayed, so the
HIP events around the replay time GPU work, not Python's launch latency.

The same JSON line carries:
  roofline      -- the step's dominant GEMV launch (K launches of that batch
                   size back to back): algorithmic bytes (packed weights + x +
                   y) / mean launch time, against 8 TB/s HBM; `traffic` is the
                   HBM bytes per launch from the committed counter passes;
  gemm          -- prefill GEMM on the 2048 x 17408 x 5120 workload, whole
                   batch and 8 chunks of 256 rows, TFLOP/s against fp16 MFMA,
                   plus the chunk-size sweep (128, 256 and 512 rows);
  quantize      -- the quantiser on the same 5120 x 5120 fp32 weight;
  layer_decode  -- one 27B-class layer's seven decode linears at M = 1 and 10,
                   as seven launches and as four (q/k/v and gate/up each one
                   launch on their concatenated packed rows);
  layer_prefill -- the same layer's GEMMs at M = 256 and 4096, seven launches
                   and four;
  other_configs -- the 512 x 512 fp32 linear (latency: quantise, GEMV) and the
                   17408 x 5120 gate/up weight with outlier blocks, m = 1, 10, 32;
  bf16          -- bf16 activations on the headline GEMV and the prefill GEMM;
  host_twin     -- the host-CPU twin (libq4host) on the same packed bytes,
                   on the host cores (a second backend, not a GPU figure);
  cpu_baseline  -- the CPU oracle timed on a bounded sample of the step.

Counter passes (HBM traffic): run `bench.py --traffic` once under
`rocprofv3 --pmc FETCH_SIZE` and once under `--pmc WRITE_SIZE`, then
`bench.py --traffic-summary FETCH.csv WRITE.csv` writes profiles/traffic.json.
Matrix-core pass: `bench.py --mfma` under `rocprofv3 --pmc MfmaUtil MfmaFlopsF16`,
then `bench.py --mfma-summary PMC.csv` writes profiles/mfma.json.
Wave-state pass: `bench.py --traffic` under `rocprofv3 --pmc` with the SQ
counters of SQ_COUNTERS (and GRBM_GUI_ACTIVE), then `bench.py --sq-summary
PMC.csv` writes profiles/sq.json.

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
CHUNK_ROWS = (128, 256, 512)     # prefill chunk-size sweep over the 2048-row batch


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted((ROOT / "bit_block_quantized_q4_amd" / "csrc").glob("*")):
        if p.suffix not in (".hip", ".hpp", ".h"):
            continue  # sources only (not compiler by-products left beside them)
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


def load_mfma_util(kernel_key: str):
    """Matrix-core busy percentage of a GEMM kernel from the committed counter
    summary, or None when the kernels changed since it was taken."""
    f = ROOT / "profiles" / "mfma.json"
    if not f.exists():
        return None
    try:
        data = json.loads(f.read_text())
    except ValueError:
        return None
    if data.get("source_hash") != kernel_source_hash():
        return None
    k = data.get("kernels", {}).get(kernel_key)
    return None if k is None else k.get("MfmaUtil")


def capture(torch, fn):
    """fn's launches recorded into a HIP graph (one eager call first warms them)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_seconds(torch, g):
    """GPU time of one replay, from HIP events on the replay stream."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e-3


def gemv_setup(q4, torch, dev, rotate_bytes):
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
    del wd
    torch.cuda.synchronize()
    return {"wl": wl, "n": n, "k": k, "wbytes": wbytes, "w_host": w, "ncopies": ncopies,
            "packed": packed, "ms": ms, "x": x, "ys": ys}


def gemv_launches(q4, s, nsteps, ms, first):
    """nsteps steps of one launch per batch size in ms, each launch on the next
    weight copy (so no launch finds its weights in the last-level cache)."""
    def fn():
        i = first
        for _ in range(nsteps):
            for m in ms:
                q4.q4_gemv(s["x"][:m], s["packed"][i % s["ncopies"]], y=s["ys"][m])
                i += 1
    return fn


def gemv_alg_bytes(m, n, k):
    """Bytes a launch must move at least once: packed weights, x (fp16), y (fp16)."""
    return n * (k // QK) * BLOCK_BYTES + 2 * m * k + 2 * m * n


def bench_gemv(q4, torch, dev, steps, warmup, rotate_bytes):
    s = gemv_setup(q4, torch, dev, rotate_bytes)
    n, k, ms, wbytes = s["n"], s["k"], s["ms"], s["wbytes"]
    # The whole step (all batch sizes), K steps in one graph after W warm-up steps.
    gw = capture(torch, gemv_launches(q4, s, max(warmup, 1), ms, 0))
    gt = capture(torch, gemv_launches(q4, s, steps, ms, max(warmup, 1) * len(ms)))
    gw.replay()
    step_s = replay_seconds(torch, gt) / steps
    del gw, gt
    # Per batch size: K launches back to back, mean launch time.
    per_m = []
    for m in ms:
        g = capture(torch, gemv_launches(q4, s, steps, [m], 0))
        g.replay()
        avg_s = replay_seconds(torch, g) / steps
        del g
        alg = gemv_alg_bytes(m, n, k)
        per_m.append({
            "m": m, "mean_us": avg_s * 1e6, "weight_gbs": wbytes / avg_s / 1e9,
            "alg_bytes": alg, "alg_gbs": alg / avg_s / 1e9,
            "frac_hbm": alg / avg_s / 1e9 / HBM_PEAK_GBS,
        })
    return {
        "wl": s["wl"], "n": n, "k": k, "ms": ms, "wbytes": wbytes, "ncopies": s["ncopies"],
        "step_s": step_s, "value_gbs": wbytes * len(ms) / step_s / 1e9, "per_m": per_m,
        "w_host": s["w_host"], "packed0": s["packed"][0], "setup": s,
    }


def bench_gemv_dense_library(torch, dev, s, per_m, steps, rotate_bytes):
    """Context, not the metric: the same decode products through the fp16
    library GEMM (torch.mm) on the unquantised weights rounded to fp16, as a
    contiguous [k, n] operand, rotated over >= rotate_bytes like the packed
    copies; and the Q4_0 launches' speed relative to it."""
    n, k, ms = s["n"], s["k"], s["ms"]
    wt0 = torch.from_numpy(s["w_host"]).to(dev).half().t().contiguous()
    dbytes = n * k * 2
    copies = max(4, -(-rotate_bytes // dbytes))
    wts = [wt0] + [wt0.clone() for _ in range(copies - 1)]
    q4_us = {r["m"]: r["mean_us"] for r in per_m}
    rows = []
    for m in ms:
        x, y = s["x"][:m], s["ys"][m]

        def fn():
            for i in range(steps):
                torch.mm(x, wts[i % copies], out=y)
        g = capture(torch, fn)
        g.replay()
        avg_s = replay_seconds(torch, g) / steps
        del g
        rows.append({"m": m, "mean_us": avg_s * 1e6, "weight_gbs": dbytes / avg_s / 1e9,
                     "q4_speed_vs_library": avg_s * 1e6 / q4_us[m]})
    del wts, wt0
    torch.cuda.empty_cache()
    return {"op": "torch.mm, fp16 x and fp16 weights [k, n] contiguous", "weight_bytes": dbytes,
            "copies_rotated": copies, "per_m": rows}


def bench_quantize(q4, torch, dev, w_host, reps, rotate_bytes):
    n, k = w_host.shape
    in_bytes = n * k * 4
    copies = max(2, -(-rotate_bytes // in_bytes))
    ws = [torch.from_numpy(w_host).to(dev) for _ in range(copies)]
    out = torch.empty((n, (k // QK) * BLOCK_BYTES), dtype=torch.uint8, device=dev)

    def fn():
        for i in range(reps):
            q4.q4_quantize(ws[i % copies], packed=out)

    g = capture(torch, fn)
    g.replay()
    avg_s = replay_seconds(torch, g) / reps
    alg = n * k * 4 + n * (k // QK) * BLOCK_BYTES
    gbs = alg / avg_s / 1e9
    return {"workload": "quantize_fp32_5120x5120", "mean_us": avg_s * 1e6, "alg_bytes": alg,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("quantize_fp32_5120x5120")}}


def gemm_setup(q4, torch, dev, x_dtype=None, dense=False):
    """The prefill workload's launches.  With dense=True also returns
    dense(cs): the same product in cs-row launches of the fp16 library GEMM
    (torch.mm) on the unquantised weights rounded to fp16, a same-box
    reference for the matrix-core kernels."""
    import synth
    wl = synth.WORKLOADS[4]
    lin = wl.linears[0]
    n, k, m = lin.n, lin.k, 2048
    w = synth.workload_weights(wl, lin)
    wd = torch.from_numpy(w).to(dev)
    packed = q4.q4_quantize(wd)
    wt = wd.half().t().contiguous() if dense else None  # [k, n] fp16, contiguous
    del w, wd
    x = torch.from_numpy(synth.workload_activations(wl, k, m)).to(dev)
    if x_dtype is not None:
        x = x.to(x_dtype)
    y = torch.empty((m, n), dtype=torch.float16, device=dev)
    xcode = q4._dtype_code(x)
    ws = max([q4.q4_gemm_workspace_size_dt(c, n, k, xcode) for c in (m,) + CHUNK_ROWS] + [1])
    work = torch.empty(ws, dtype=torch.uint8, device=dev)

    def whole():
        q4.q4_gemm(x, packed, y=y, workspace=work)

    def chunked(cs):
        def fn():
            for c in range(m // cs):
                q4.q4_gemm(x[c * cs:(c + 1) * cs], packed, y=y[c * cs:(c + 1) * cs], workspace=work)
        return fn

    if not dense:
        return m, n, k, whole, chunked

    def dense_chunked(cs):
        def fn():
            for c in range(m // cs):
                torch.mm(x[c * cs:(c + 1) * cs], wt, out=y[c * cs:(c + 1) * cs])
        return fn

    return m, n, k, whole, chunked, dense_chunked


def time_gemm_calls(torch, fn, reps):
    """Mean GPU seconds of one fn() (its launches replayed from a HIP graph)."""
    def rep():
        for _ in range(reps):
            fn()
    g = capture(torch, rep)
    g.replay()
    t = replay_seconds(torch, g) / reps
    del g
    return t


def bench_gemm(q4, torch, dev, reps):
    """The 2048-row prefill of a 17408 x 5120 weight as one launch, as eight
    256-row chunks (the serving page's chunk size), and the chunk-size sweep:
    smaller chunks bound the activation memory a step holds, at the cost of
    streaming the packed weight once per chunk and of fewer output tiles per
    launch."""
    m, n, k, whole, chunked, dense = gemm_setup(q4, torch, dev, dense=True)
    flop = 2.0 * m * n * k
    res = {}
    for name, fn, calls in (("whole_2048", whole, 1), ("chunked_8x256", chunked(256), 8)):
        avg_s = time_gemm_calls(torch, fn, reps)
        tf = flop / avg_s / 1e12
        res[name] = {"mean_us": avg_s * 1e6, "launches": calls, "tflops": tf,
                     "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS}
    # the fp16 library GEMM of the same shapes on the same box (context, not
    # the metric): speed of the Q4_0 launches relative to it
    lib = {}
    for name, cs in (("whole_2048", m), ("chunked_8x256", 256)):
        avg_s = time_gemm_calls(torch, dense(cs), reps)
        lib[name] = {"mean_us": avg_s * 1e6, "frac_mfma": flop / avg_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
                     "q4_speed_vs_library": avg_s * 1e6 / res[name]["mean_us"]}
    res["dense_fp16_library"] = {"op": "torch.mm, fp16 x and fp16 weights [k, n] contiguous", **lib}
    sweep = []
    for cs in CHUNK_ROWS:
        avg_s = time_gemm_calls(torch, chunked(cs), reps)
        tf = flop / avg_s / 1e12
        sweep.append({"chunk_rows": cs, "launches": m // cs, "mean_us": avg_s * 1e6,
                      "us_per_chunk": avg_s * 1e6 / (m // cs), "tflops": tf,
                      "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS})
    best = res["whole_2048"]["tflops"]
    return {
        "workload": "prefill_chunked_2048x17408x5120", "m": m, "n": n, "k": k,
        **res, "chunk_sweep": sweep,
        "roofline": {"bound": "mfma", "achieved": best, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": best / MFMA_F16_PEAK_TFLOPS,
                     "traffic": load_traffic("gemm_2048x17408x5120"),
                     "mfma_util_pct": load_mfma_util("gemm_mfma_256x256_f16_out")},
    }


def bench_layer_decode(q4, torch, dev, steps, rotate_bytes, ms=(1, 10)):
    """Decode through one 27B-class layer's seven linears (q, k, v, o, gate,
    up, down) at M = 1 and 10: seven launches, against four where q/k/v and
    gate/up run as one launch each on their packed rows concatenated (packed
    rows are independent, so a concatenated buffer is simply a taller weight).
    Each linear's packed copy is a row slice of its group's buffer, so both
    variants stream the same bytes; layer copies are rotated over >= 1 GiB."""
    import synth
    lins = {l.name: l for l in synth.WORKLOADS[5].linears}
    k_model = lins["q"].k
    groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gateup", ["gate", "up"]), ("down", ["down"])]
    layer_bytes = sum(l.n * (l.k // QK) * BLOCK_BYTES for l in lins.values())
    copies = max(2, -(-rotate_bytes // layer_bytes))
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    layers = []
    for _ in range(copies):
        bufs, views = {}, {}
        for gname, names in groups:
            kk = lins[names[0]].k
            rows = sum(lins[nm].n for nm in names)
            buf = torch.empty((rows, (kk // QK) * BLOCK_BYTES), dtype=torch.uint8, device=dev)
            r = 0
            for nm in names:
                n = lins[nm].n
                w = torch.randn((n, kk), device=dev, generator=gen) * 0.02
                views[nm] = buf[r:r + n]
                q4.q4_quantize(w, packed=views[nm])
                r += n
            bufs[gname] = buf
        layers.append((bufs, views))
    torch.cuda.synchronize()
    res = {}
    for m in ms:
        x = torch.randn((m, k_model), device=dev, generator=gen).half()
        xd = torch.randn((m, lins["down"].k), device=dev, generator=gen).half()
        ysep = {nm: torch.empty((m, l.n), dtype=torch.float16, device=dev) for nm, l in lins.items()}
        ygrp = {g: torch.empty((m, sum(lins[nm].n for nm in names)), dtype=torch.float16, device=dev)
                for g, names in groups}

        def separate():
            for i in range(steps):
                _, views = layers[i % copies]
                for nm in ("q", "k", "v", "o", "gate", "up"):
                    q4.q4_gemv(x, views[nm], y=ysep[nm])
                q4.q4_gemv(xd, views["down"], y=ysep["down"])

        def fused():
            for i in range(steps):
                bufs, _ = layers[i % copies]
                for g in ("qkv", "o", "gateup"):
                    q4.q4_gemv(x, bufs[g], y=ygrp[g])
                q4.q4_gemv(xd, bufs["down"], y=ygrp["down"])

        row = {}
        for name, fn, launches in (("separate", separate, 7), ("fused", fused, 4)):
            g = capture(torch, fn)
            g.replay()
            t = replay_seconds(torch, g) / steps
            del g
            row[name] = {"launches": launches, "us_per_layer": t * 1e6,
                         "weight_gbs": layer_bytes / t / 1e9,
                         "frac_hbm": layer_bytes / t / 1e9 / HBM_PEAK_GBS}
        res[f"m{m}"] = row
    return {"workload": "decode_layer_27b_dense (q,k,v,o,gate,up,down)", "weight_bytes": layer_bytes,
            "layer_copies_rotated": copies, **res}


def bench_layer_prefill(q4, torch, dev, reps, ms=(256, 4096)):
    """Prefill through one 27B-class layer's seven linears at M = 256 (one
    chunk) and 4096 rows: seven launches, and four with q/k/v and gate/up
    each run on their concatenated packed rows.  The GEMM is bound by the
    matrix cores, so one copy of the layer's weights serves every call."""
    import synth
    lins = {l.name: l for l in synth.WORKLOADS[5].linears}
    groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gateup", ["gate", "up"]), ("down", ["down"])]
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    bufs, views = {}, {}
    for gname, names in groups:
        kk = lins[names[0]].k
        rows = sum(lins[nm].n for nm in names)
        buf = torch.empty((rows, (kk // QK) * BLOCK_BYTES), dtype=torch.uint8, device=dev)
        r = 0
        for nm in names:
            nn = lins[nm].n
            views[nm] = buf[r:r + nn]
            q4.q4_quantize(torch.randn((nn, kk), device=dev, generator=gen) * 0.02, packed=views[nm])
            r += nn
        bufs[gname] = buf
    flop_per_row = 2.0 * sum(l.n * l.k for l in lins.values())
    res = {}
    for m in ms:
        x = torch.randn((m, lins["q"].k), device=dev, generator=gen).half()
        xd = torch.randn((m, lins["down"].k), device=dev, generator=gen).half()
        ysep = {nm: torch.empty((m, l.n), dtype=torch.float16, device=dev) for nm, l in lins.items()}
        ygrp = {g: torch.empty((m, sum(lins[nm].n for nm in names)), dtype=torch.float16, device=dev)
                for g, names in groups}
        wsz = max([q4.q4_gemm_workspace_size(m, b.shape[0], lins[names[0]].k)
                   for (g, names), b in zip(groups, bufs.values())] +
                  [q4.q4_gemm_workspace_size(m, l.n, l.k) for l in lins.values()] + [1])
        work = torch.empty(wsz, dtype=torch.uint8, device=dev)

        def separate():
            for nm in ("q", "k", "v", "o", "gate", "up"):
                q4.q4_gemm(x, views[nm], y=ysep[nm], workspace=work)
            q4.q4_gemm(xd, views["down"], y=ysep["down"], workspace=work)

        def fused():
            for g in ("qkv", "o", "gateup"):
                q4.q4_gemm(x, bufs[g], y=ygrp[g], workspace=work)
            q4.q4_gemm(xd, bufs["down"], y=ygrp["down"], workspace=work)

        row = {}
        for name, fn, launches in (("separate", separate, 7), ("fused", fused, 4)):
            t = time_gemm_calls(torch, fn, reps)
            tf = flop_per_row * m / t / 1e12
            row[name] = {"launches": launches, "us_per_layer": t * 1e6, "tflops": tf,
                         "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS}
        res[f"m{m}"] = row
        del x, xd, ysep, ygrp, work
    return {"workload": "prefill_layer_27b_dense (q,k,v,o,gate,up,down)",
            "gflop_per_row": flop_per_row / 1e9, **res}


def bench_host_twin(q4, torch, packed_dev, n, k, ms, budget_s=1.0):
    """The host-CPU twin (libq4host) on the same packed bytes as the headline
    GEMV, copied once to host memory: each batch size repeated for about
    budget_s seconds on the default thread count.  A second backend's rate on
    the host cores, not a GPU figure."""
    import numpy as np
    import synth
    from bit_block_quantized_q4_amd.host import q4_host_default_threads, q4_host_gemv
    packed = packed_dev.cpu().numpy()
    wl = synth.WORKLOADS[2]
    xs = synth.workload_activations(wl, k, max(ms))
    wbytes = packed.nbytes
    threads = q4_host_default_threads()
    per_m, step = [], 0.0
    for m in ms:
        x = np.ascontiguousarray(xs[:m])
        y = np.empty((m, n), np.float16)
        q4_host_gemv(x, packed, y=y)
        reps, t0 = 0, time.perf_counter()
        while True:
            q4_host_gemv(x, packed, y=y)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        avg = el / reps
        step += avg
        per_m.append({"m": m, "mean_ms": avg * 1e3, "weight_gbs": wbytes / avg / 1e9})
    return {"workload": f"decode_attn_proj_{n}x{k} (host memory)", "threads": threads,
            "value": wbytes * len(ms) / step / 1e9, "unit": "GB/s", "per_m": per_m}


def bench_bf16(q4, torch, dev, s, steps, gemm_reps):
    """bf16 activations: the headline GEMV on the same rotated weights (the
    kernels convert x to fp16 in LDS or in registers), and the 2048-row
    prefill, whole and in 256-row chunks (x staged as fp16 in the workspace
    by a pre-pass, which is inside the timed launches)."""
    n, k, wbytes = s["n"], s["k"], s["wbytes"]
    sb = dict(s, x=s["x"].to(torch.bfloat16))
    per_m = []
    for m in s["ms"]:
        g = capture(torch, gemv_launches(q4, sb, steps, [m], 0))
        g.replay()
        avg_s = replay_seconds(torch, g) / steps
        del g
        alg = gemv_alg_bytes(m, n, k)
        per_m.append({"m": m, "mean_us": avg_s * 1e6, "alg_gbs": alg / avg_s / 1e9,
                      "frac_hbm": alg / avg_s / 1e9 / HBM_PEAK_GBS})
    m, n2, k2, whole, chunked = gemm_setup(q4, torch, dev, torch.bfloat16)
    flop = 2.0 * m * n2 * k2
    gemm = {}
    for name, fn, calls in (("whole_2048", whole, 1), ("chunked_8x256", chunked(256), 8)):
        t = time_gemm_calls(torch, fn, gemm_reps)
        tf = flop / t / 1e12
        gemm[name] = {"mean_us": t * 1e6, "launches": calls, "tflops": tf,
                      "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS}
    return {"gemv_workload": f"decode_attn_proj_{n}x{k}, bf16 x, fp16 y", "gemv_per_m": per_m,
            "gemm_workload": f"prefill_{m}x{n2}x{k2}, bf16 x, fp16 y", "gemm": gemm}


def bench_other_configs(q4, torch, dev, steps, rotate_bytes):
    """The two other single-linear configurations: the 512 x 512 linear with
    fp32 activations and output (a latency figure: its 147 KB of packed
    weights stay in L2, so one copy is reused), quantise and GEMV; and the
    17408 x 5120 gate/up weight with 0.1% outlier blocks at m = 1, 10 and 32
    (weights rotated over >= 1 GiB, weight GB/s against 8 TB/s)."""
    import synth
    out = {}
    wl = synth.WORKLOADS[1]
    lin = wl.linears[0]
    w = torch.from_numpy(synth.workload_weights(wl, lin)).to(dev)
    packed = q4.q4_quantize(w)
    x = torch.from_numpy(synth.workload_activations(wl, lin.k, 1)).to(dev)
    y = torch.empty((1, lin.n), dtype=torch.float32, device=dev)

    def quant():
        for _ in range(steps):
            q4.q4_quantize(w, packed=packed)

    def gemv():
        for _ in range(steps):
            q4.q4_gemv(x, packed, y=y)

    row = {}
    for name, fn in (("quantize_us", quant), ("gemv_us", gemv)):
        g = capture(torch, fn)
        g.replay()
        row[name] = replay_seconds(torch, g) / steps * 1e6
        del g
    out[wl.name] = {"n": lin.n, "k": lin.k, "m": 1, "x_dtype": "f32", "y_dtype": "f32", **row}

    wl = synth.WORKLOADS[3]
    lin = wl.linears[0]
    n, k = lin.n, lin.k
    wbytes = n * (k // QK) * BLOCK_BYTES
    wd = torch.from_numpy(synth.workload_weights(wl, lin)).to(dev)
    ncopies = max(2, -(-rotate_bytes // wbytes))
    copies = [q4.q4_quantize(wd) for _ in range(ncopies)]
    del wd
    xs = torch.from_numpy(synth.workload_activations(wl, k, max(wl.ms))).to(dev)
    per_m = []
    for m in wl.ms:
        y = torch.empty((m, n), dtype=torch.float16, device=dev)
        reps = min(steps, 100)

        def fn(m=m, y=y, reps=reps):
            for i in range(reps):
                q4.q4_gemv(xs[:m], copies[i % ncopies], y=y)

        g = capture(torch, fn)
        g.replay()
        t = replay_seconds(torch, g) / reps
        del g
        alg = gemv_alg_bytes(m, n, k)
        per_m.append({"m": m, "mean_us": t * 1e6, "alg_gbs": alg / t / 1e9,
                      "frac_hbm": alg / t / 1e9 / HBM_PEAK_GBS})
    out[wl.name] = {"n": n, "k": k, "weight_copies_rotated": ncopies, "per_m": per_m}
    del copies
    return out


# ------------------------------------------------------------ HBM traffic

TRAFFIC_CALIB_BYTES = 512 << 20


def traffic_run(q4, torch, dev, rotate_bytes, launches=20):
    """The launches the two counter passes (FETCH_SIZE, then WRITE_SIZE) read:
    a plain device copy of known size (torch's negation kernel: reads and writes
    TRAFFIC_CALIB_BYTES once), then the GEMV at every batch size, the
    quantiser and the whole-batch GEMM, each repeated."""
    src = torch.ones(TRAFFIC_CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    del src, dst
    s = gemv_setup(q4, torch, dev, rotate_bytes)
    for m in s["ms"]:
        gemv_launches(q4, s, launches, [m], 0)()
    torch.cuda.synchronize()
    ws = [torch.from_numpy(s["w_host"]).to(dev) for _ in range(2)]
    for i in range(launches):
        q4.q4_quantize(ws[i % 2], packed=s["packed"][0])
    del s, ws
    torch.cuda.synchronize()
    _, _, _, whole, _ = gemm_setup(q4, torch, dev)
    for _ in range(3):
        whole()
    torch.cuda.synchronize()
    print("traffic launches done", flush=True)


def mfma_run(q4, torch, dev, reps=3):
    """The launches the matrix-core counter pass (MfmaUtil, MfmaFlopsF16) reads:
    the 2048 x 17408 x 5120 prefill as one launch and as 8 chunks of 256 rows."""
    _, _, _, whole, chunked = gemm_setup(q4, torch, dev)
    for _ in range(reps):
        whole()
    for _ in range(reps):
        chunked(256)()
    torch.cuda.synchronize()
    print("mfma launches done", flush=True)


def mfma_summary(csv_path, out_path):
    """profiles/mfma.json from the counter pass over mfma_run: per GEMM kernel,
    the median per dispatch of MfmaUtil (matrix-core busy cycles over the
    dispatch's active cycles, all SIMDs) and of MfmaFlopsF16 (fp16 matrix
    flops issued), with the algorithmic flops of the dispatch's share."""
    import re
    by = {}
    for did, name, cnt, val in _pmc_rows(csv_path):
        if "gemm_" not in name and "splitk_reduce" not in name:
            continue
        if "gemm_mfma_kernel" in name:
            key = "gemm_mfma_256x256" if ("ILi256" in name or "<256" in name) else "gemm_mfma_128x128"
        elif "gemm_slicek_kernel" in name:
            key = "gemm_slicek_128x128"
        elif "splitk_reduce" in name:
            key = "splitk_reduce"
        else:
            key = "other_gemm"
        # the output type is the kernels' last template argument: fp16 y, or
        # fp32 split-K partials (the tail)
        if re.search(r"kernelI(?:Li\d+E)*fE", name) or "float>" in name:
            key += "_f32_partials"
        else:
            key += "_f16_out"
        by.setdefault(key, {}).setdefault(cnt, []).append(val)
    kernels = {}
    for key, cnts in sorted(by.items()):
        kernels[key] = {c: float(np.median(v)) for c, v in cnts.items()}
        kernels[key]["dispatches"] = max(len(v) for v in cnts.values())
    data = {"source_hash": kernel_source_hash(),
            "workload": "prefill_2048x17408x5120, whole launch and 8 x 256-row chunks",
            "peak_mfma_f16_tflops": MFMA_F16_PEAK_TFLOPS, "kernels": kernels}
    Path(out_path).write_text(json.dumps(data, indent=1) + "\n")
    return data


def _pmc_rows(csv_path):
    """(dispatch id, kernel name, counter, value) rows of a rocprofv3 counter CSV."""
    import csv
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            cnt = r.get("Counter_Name") or r.get("Counter-Name") or ""
            val = float(r.get("Counter_Value") or r.get("Counter-Value") or 0.0)
            did = int(r.get("Dispatch_Id") or r.get("Dispatch-Id") or len(rows))
            rows.append((did, name, cnt, val))
    rows.sort()
    return rows


def _traffic_key(name):
    """Workload of a dispatch in the traffic_run launches (None: not counted)."""
    if "neg_kernel" in name:
        return "calib_copy"
    if "gemv_" in name and "_kernel" in name:
        return "gemv"
    if "quantize_kernel" in name:
        return "quantize_fp32_5120x5120"
    if "gemm_mfma_kernelILi256" in name or "gemm_mfma_kernel<256" in name:
        return "gemm_2048x17408x5120"
    return None


def _traffic_groups(csv_path, counter):
    """Per workload, the per-dispatch values of one counter of a traffic_run
    pass.  GEMV dispatches are attributed to batch sizes by launch order
    (traffic_run launches them in WORKLOADS[2].ms order)."""
    import synth
    ms = list(synth.WORKLOADS[2].ms)
    by, gemv = {}, []
    for did, name, cnt, val in _pmc_rows(csv_path):
        if cnt != counter:
            continue
        key = _traffic_key(name)
        if key == "gemv":
            gemv.append(val)
        elif key:
            by.setdefault(key, []).append(val)
    if gemv:
        per = len(gemv) // len(ms)
        for i, m in enumerate(ms):
            by[f"gemv_5120x5120_m{m}"] = gemv[i * per:(i + 1) * per]
    return by


SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
               "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT")


def sq_summary(csv_path, out_path):
    """profiles/sq.json from one counter pass of SQ_COUNTERS over traffic_run:
    per workload, the median per dispatch of each counter, and the ratios read
    from them (waiting cycles per wave cycle; LDS bank-conflict cycles per
    cycle of LDS instruction activity)."""
    kernels = {}
    for c in SQ_COUNTERS:
        for key, vals in _traffic_groups(csv_path, c).items():
            if key == "calib_copy":
                continue
            kernels.setdefault(key, {})[c] = float(np.median(vals))
            kernels[key]["dispatches"] = len(vals)
    for v in kernels.values():
        wc = v.get("SQ_WAVE_CYCLES") or 0.0
        lds = v.get("SQ_ACTIVE_INST_LDS") or 0.0
        v["wait_any_per_wave_cycle"] = v.get("SQ_WAIT_ANY", 0.0) / wc if wc else None
        v["wait_inst_per_wave_cycle"] = v.get("SQ_WAIT_INST_ANY", 0.0) / wc if wc else None
        v["lds_conflict_per_lds_active"] = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds else None
    data = {"source_hash": kernel_source_hash(), "counters": list(SQ_COUNTERS), "kernels": kernels}
    Path(out_path).write_text(json.dumps(data, indent=1) + "\n")
    return data


def traffic_summary(fetch_csv, write_csv, out_path):
    """profiles/traffic.json from the two counter passes: per kernel, the median
    FETCH_SIZE and WRITE_SIZE per dispatch (KiB), each scaled by known bytes /
    counted bytes of the plain copy.  GEMV dispatches are attributed to batch
    sizes by launch order (traffic_run launches them in WORKLOADS[2].ms order)."""
    def medians(path, counter):
        by = _traffic_groups(path, counter)
        return {k: float(np.median(v)) for k, v in by.items()}, {k: len(v) for k, v in by.items()}

    fetch, nf = medians(fetch_csv, "FETCH_SIZE")
    write, nw = medians(write_csv, "WRITE_SIZE")
    f_scale = TRAFFIC_CALIB_BYTES / (fetch["calib_copy"] * 1024.0)
    w_scale = TRAFFIC_CALIB_BYTES / (write["calib_copy"] * 1024.0)
    kernels = {}
    for key in sorted(set(fetch) & set(write)):
        if key == "calib_copy":
            continue
        fb = fetch[key] * 1024.0 * f_scale
        wb = write[key] * 1024.0 * w_scale
        kernels[key] = {"fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb,
                        "fetch_kib_raw": fetch[key], "write_kib_raw": write[key],
                        "dispatches": min(nf[key], nw[key])}
    data = {"source_hash": kernel_source_hash(),
            "calibration": {"bytes": TRAFFIC_CALIB_BYTES, "fetch_kib": fetch["calib_copy"],
                            "write_kib": write["calib_copy"], "fetch_scale": f_scale,
                            "write_scale": w_scale},
            "kernels": kernels}
    Path(out_path).write_text(json.dumps(data, indent=1) + "\n")
    return data


def trace_summary(trace_csv, steps, warmup):
    """Per batch size, the mean duration of the GEMV dispatches that bench_gemv
    times, from a rocprofv3 kernel-trace CSV of a run with the same steps and
    warmup.  bench_gemv is the run's first GEMV work: (2 max(warmup, 1) +
    2 steps) len(ms) dispatches for the whole-step graphs (eager capture runs,
    then the replays), then per batch size in WORKLOADS[2].ms order `steps`
    eager launches (capture), `steps` in the warm replay and `steps` in the
    timed replay.  Later legs (layer decode, bf16) launch more GEMVs after
    these."""
    import csv
    import synth
    ms = list(synth.WORKLOADS[2].ms)
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            # this library's kernels (demangled when launched directly, mangled
            # when replayed from a graph)
            ours = "q4::" in name or name.startswith("_ZN2q4")
            if ours and "gemv_" in name and "_kernel" in name:
                start = int(r.get("Start_Timestamp") or r.get("Start-Timestamp"))
                end = int(r.get("End_Timestamp") or r.get("End-Timestamp"))
                rows.append((start, end - start, name))
    rows.sort()
    first = (2 * max(warmup, 1) + 2 * steps) * len(ms)
    tail = rows[first:first + 3 * steps * len(ms)]
    out = []
    for i, m in enumerate(ms):
        rep = tail[(3 * i + 2) * steps:(3 * i + 3) * steps]
        names = sorted({r[2] for r in rep})
        out.append({"m": m, "dispatches": len(rep), "mean_us": float(np.mean([r[1] for r in rep])) / 1e3,
                    "kernels": names})
    return out


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
    ap.add_argument("--only", choices=["all", "gemv", "gemm", "quantize", "layer", "host", "bf16",
                                       "other"],
                    default="all")
    ap.add_argument("--traffic", action="store_true",
                    help="run the launches the FETCH_SIZE / WRITE_SIZE counter passes read")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from the two counter passes")
    ap.add_argument("--mfma", action="store_true",
                    help="run the launches the MfmaUtil / MfmaFlopsF16 counter pass reads")
    ap.add_argument("--mfma-summary", metavar="PMC_CSV",
                    help="write profiles/mfma.json from that counter pass")
    ap.add_argument("--sq-summary", metavar="PMC_CSV",
                    help="write profiles/sq.json from an SQ counter pass over --traffic")
    ap.add_argument("--trace-summary", metavar="TRACE_CSV",
                    help="print per-batch-size GEMV durations from a kernel-trace CSV of a default run")
    args = ap.parse_args()

    if args.trace_summary:
        for r in trace_summary(args.trace_summary, args.steps, args.warmup):
            print(json.dumps(r))
        return
    if args.traffic_summary:
        d = traffic_summary(args.traffic_summary[0], args.traffic_summary[1],
                            ROOT / "profiles" / "traffic.json")
        print(json.dumps(d, indent=1))
        return
    if args.mfma_summary:
        print(json.dumps(mfma_summary(args.mfma_summary, ROOT / "profiles" / "mfma.json"), indent=1))
        return
    if args.sq_summary:
        print(json.dumps(sq_summary(args.sq_summary, ROOT / "profiles" / "sq.json"), indent=1))
        return

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
    if args.traffic:
        traffic_run(q4, torch, dev, rotate)
        return
    if args.mfma:
        mfma_run(q4, torch, dev)
        return

    out = {"metric": METRIC}
    g = bench_gemv(q4, torch, dev, args.steps, args.warmup, rotate)
    dom = max(g["per_m"], key=lambda r: r["mean_us"])  # the step's dominant launch
    out.update({
        "value": g["value_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": g["step_s"] * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": g["wl"].name, "n": g["n"], "k": g["k"], "ms": g["ms"],
                   "x_dtype": "f16", "y_dtype": "f16",
                   "weight_copies_rotated": g["ncopies"],
                   "weight_bytes_per_launch": g["wbytes"]},
        "roofline": {"bound": "hbm", "achieved": dom["alg_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dom["alg_gbs"] / HBM_PEAK_GBS,
                     "traffic": load_traffic(f"gemv_5120x5120_m{dom['m']}"),
                     "kernel": f"q4_gemv m={dom['m']}", "mean_us": dom["mean_us"],
                     "alg_bytes_per_launch": dom["alg_bytes"]},
        "per_m": g["per_m"],
    })
    out["gemv_dense_fp16_library"] = bench_gemv_dense_library(
        torch, dev, g["setup"], g["per_m"], args.steps, rotate)
    if args.only in ("all", "quantize"):
        out["quantize"] = bench_quantize(q4, torch, dev, g["w_host"], 20, rotate)
    if args.only in ("all", "gemm"):
        out["gemm"] = bench_gemm(q4, torch, dev, args.gemm_reps)
    if args.only in ("all", "layer"):
        out["layer_decode"] = bench_layer_decode(q4, torch, dev, min(args.steps, 50), rotate)
        out["layer_prefill"] = bench_layer_prefill(q4, torch, dev, 3)
    if args.only in ("all", "other"):
        out["other_configs"] = bench_other_configs(q4, torch, dev, args.steps, rotate)
    if args.only in ("all", "bf16"):
        out["bf16"] = bench_bf16(q4, torch, dev, g["setup"], args.steps, args.gemm_reps)
    if args.only in ("all", "host"):
        out["host_twin"] = bench_host_twin(q4, torch, g["packed0"], g["n"], g["k"], g["ms"])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(g["w_host"], g["n"], g["k"], g["ms"])
    out["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
