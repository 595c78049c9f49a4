#!/usr/bin/env python3
"""Q4_0 linear-layer benchmark on one MI355X.

Headline: one 27B-class dense decoder layer's linears (q/k/v, o, gate/up,
down; K = 5120 or 17408; Student-t(3) x 0.02 weights, fp16 activations, fp16
outputs) in batched decode at M = 1 and M = 10.  q/k/v and gate/up each run as
one launch over their packed rows stacked, so a step is eight q4_gemv launches
(four per batch size) streaming 2 x 185.8 MB of packed weights; layer copies
are rotated over >= 1 GiB so every launch reads HBM rather than the 256 MB
last-level cache.  `value` is the step's packed-weight GB/s; `roofline` is the
step's dominant launch (algorithmic bytes: packed weights + x + y) against
8 TB/s.  The W warm-up steps and the K timed steps are recorded into HIP
graphs and replayed, so the HIP events around a replay time GPU work, not
Python's launch latency.  Before a timed replay the same graph is replayed,
untimed, for a fixed wall time (0.5 s before the step, 0.1 s before every
other timed replay; Q4_BENCH_SETTLE_S sets the first, the rest scale with it):
the shader clock follows the load with a delay, and a launch timed right
after different work runs at whatever clock that work left (the decode
launches measured up to 15 % slower that way).

The GEMM half (`gemm`): the same layer's prefill at M = 4096 (four launches),
TFLOP/s against the fp16 matrix-core peak, with its own roofline object on the
dominant launch and the shader clock sampled during the leg; `mfma_ceiling`
times libq4floor's matrix-core kernel (the GEMM tile's fragment reads and
products, nothing else) under the same kind of load, and the roofline object
gives the dominant launch's fraction of that sustained rate too.

The same JSON line carries:
  read_floor     -- libq4floor's plain streaming read of the same rotated
                    packed buffers, launch by launch: what streaming these bytes
                    costs without any Q4_0 work;
  layer_decode   -- the layer as seven launches against four, M = 1 and 10;
  layer_prefill  -- the layer's GEMMs at M = 256 and 4096, seven and four;
  attn_proj      -- the 5120 x 5120 projection at M = 1, 4, 10, 16;
  gemm           -- also the 2048 x 17408 x 5120 prefill, whole and as 8 chunks
                    of 256 rows, and the chunk-size sweep (128, 256, 512);
  quantize       -- the quantiser on the 5120 x 5120 fp32 weight;
  other_configs  -- the 512 x 512 fp32 linear (latency) and the 17408 x 5120
                    weight with outlier blocks, m = 1, 10, 32;
  bf16           -- bf16 activations on the attention projection and prefill;
  host_twin      -- the host-CPU twin (libq4host) on the same packed bytes;
  cpu_baseline   -- the CPU oracle per configuration (quantise + matmul) on
                    bounded samples, on the host cores of this process.

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
SETTLE_S = float(os.environ.get("Q4_BENCH_SETTLE_S", "0.5"))  # untimed clock settle before timing
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 matrix peak
BLOCK_BYTES, QK = 18, 32
CHUNK_ROWS = (128, 256, 512)     # prefill chunk-size sweep over the 2048-row batch


def kernel_hash() -> str:
    """Hash of the built libq4.so: committed counter summaries describe that
    exact binary, and are reported only while it is the one that runs."""
    p = ROOT / "bit_block_quantized_q4_amd" / "libq4.so"
    if not p.exists():
        return "unbuilt"
    return hashlib.sha256(p.read_bytes()).hexdigest()[:16]


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
    if data.get("kernel_hash") != kernel_hash():
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
    if data.get("kernel_hash") != kernel_hash():
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


def settle(torch, g, seconds):
    """Replay g (untimed) until `seconds` of wall time have passed, so the GPU
    clock reaches its steady state under this load before anything is timed."""
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def replay_seconds(torch, g, settle_s=None, mark=None):
    """GPU time of one replay, from HIP events on the replay stream, after
    untimed replays that settle the clock (settle_s of wall time, by default
    SETTLE_S / 5).  mark(), if given, launches a marker kernel just before and
    just after the timed replay (outside the events) for trace attribution."""
    settle(torch, g, SETTLE_S / 5 if settle_s is None else settle_s)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if mark:
        mark()
    s.record()
    g.replay()
    e.record()
    if mark:
        mark()
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


def gemm_setup(q4, torch, dev, x_dtype=None):
    """The 2048-row prefill workload's launches: whole() and chunked(cs)."""
    import synth
    wl = synth.WORKLOADS[4]
    lin = wl.linears[0]
    n, k, m = lin.n, lin.k, 2048
    w = synth.workload_weights(wl, lin)
    wd = torch.from_numpy(w).to(dev)
    packed = q4.q4_quantize(wd)
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

    return m, n, k, whole, chunked


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
    m, n, k, whole, chunked = gemm_setup(q4, torch, dev)
    flop = 2.0 * m * n * k
    res = {}
    for name, fn, calls in (("whole_2048", whole, 1), ("chunked_8x256", chunked(256), 8)):
        avg_s = time_gemm_calls(torch, fn, reps)
        tf = flop / avg_s / 1e12
        res[name] = {"mean_us": avg_s * 1e6, "launches": calls, "tflops": tf,
                     "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS}
    sweep = []
    for cs in CHUNK_ROWS:
        avg_s = time_gemm_calls(torch, chunked(cs), reps)
        tf = flop / avg_s / 1e12
        sweep.append({"chunk_rows": cs, "launches": m // cs, "mean_us": avg_s * 1e6,
                      "us_per_chunk": avg_s * 1e6 / (m // cs), "tflops": tf,
                      "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS})
    return {"workload": "prefill_chunked_2048x17408x5120", "m": m, "n": n, "k": k,
            **res, "chunk_sweep": sweep}


# ------------------------------------------------------------ the 27B-class layer

LAYER_GROUPS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")),
                ("down", ("down",)))


def layer_linears():
    import synth
    return {l.name: l for l in synth.WORKLOADS[5].linears}


def packed_bytes(rows, k):
    return rows * (k // QK) * BLOCK_BYTES


def student_t_device(torch, shape, gen, dev, sigma=0.02):
    """Student-t(3) x sigma drawn on the device from its definition:
    Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) with independent standard normals."""
    z = torch.randn(shape, device=dev, generator=gen)
    v = torch.zeros(shape, device=dev)
    for _ in range(3):
        e = torch.randn(shape, device=dev, generator=gen)
        v.addcmul_(e, e)
        del e
    return z.div_(v.div_(3.0).sqrt_()).mul_(sigma)


def layer_setup(q4, torch, dev, seed=5):
    """One layer's packed weights as the four launch groups: each group one
    buffer, each linear quantised into its row slice (Student-t(3) x 0.02)."""
    lins = layer_linears()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    bufs, views = {}, {}
    for g, names in LAYER_GROUPS:
        kk = lins[names[0]].k
        rows = sum(lins[nm].n for nm in names)
        buf = torch.empty((rows, (kk // QK) * BLOCK_BYTES), dtype=torch.uint8, device=dev)
        r = 0
        for nm in names:
            nn = lins[nm].n
            views[nm] = buf[r:r + nn]
            q4.q4_quantize(student_t_device(torch, (nn, kk), gen, dev), packed=views[nm])
            r += nn
        bufs[g] = buf
    torch.cuda.synchronize()
    return lins, bufs, views


def group_shape(lins, g):
    names = dict(LAYER_GROUPS)[g]
    return sum(lins[nm].n for nm in names), lins[names[0]].k


def rotated(torch, buf, rotate_bytes, minimum=2):
    """Distinct copies of buf totalling >= rotate_bytes (buf first)."""
    nb = buf.numel() * buf.element_size()
    count = max(minimum, -(-rotate_bytes // nb))
    return [buf] + [buf.clone() for _ in range(count - 1)]


def bench_headline_decode(q4, torch, dev, steps, warmup, rotate_bytes, ms=(1, 10)):
    """The headline step: the layer's four decode launches at each M in ms,
    layer copies rotated; then each launch on its own, K launches back to back
    over >= rotate_bytes of copies of its group buffer (so no launch finds its
    weights in the last-level cache)."""
    lins, bufs, _ = layer_setup(q4, torch, dev)
    layer_bytes = sum(packed_bytes(*group_shape(lins, g)) for g, _ in LAYER_GROUPS)
    ncopies = max(2, -(-rotate_bytes // layer_bytes))
    layers = [bufs] + [{g: b.clone() for g, b in bufs.items()} for _ in range(ncopies - 1)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    xs = {m: torch.randn((m, lins["q"].k), device=dev, generator=gen).half() for m in ms}
    xd = {m: torch.randn((m, lins["down"].k), device=dev, generator=gen).half() for m in ms}
    ys = {(m, g): torch.empty((m, group_shape(lins, g)[0]), dtype=torch.float16, device=dev)
          for m in ms for g, _ in LAYER_GROUPS}

    def launch(m, g, buf):
        q4.q4_gemv(xd[m] if g == "down" else xs[m], buf, y=ys[(m, g)])

    def step_fn(nsteps, first):
        def fn():
            i = first
            for _ in range(nsteps):
                for m in ms:  # every batch size reads the next layer copy
                    lay = layers[i % ncopies]
                    for g, _ in LAYER_GROUPS:
                        launch(m, g, lay[g])
                    i += 1
        return fn

    gw = capture(torch, step_fn(max(warmup, 1), 0))
    gt = capture(torch, step_fn(steps, max(warmup, 1) * len(ms)))
    gw.replay()
    step_s = replay_seconds(torch, gt, settle_s=SETTLE_S) / steps
    del gw, gt, layers
    sep = separator(torch, dev)
    per_launch = []
    for g, _ in LAYER_GROUPS:
        rows, k = group_shape(lins, g)
        copies = rotated(torch, bufs[g], rotate_bytes)
        for m in ms:
            def fn(m=m, g=g, copies=copies):
                for i in range(steps):
                    launch(m, g, copies[i % len(copies)])
            gr = capture(torch, fn)
            t = replay_seconds(torch, gr, mark=sep) / steps
            del gr
            wb = packed_bytes(rows, k)
            alg = wb + 2 * m * k + 2 * m * rows
            per_launch.append({"group": g, "m": m, "n": rows, "k": k, "mean_us": t * 1e6,
                               "weight_bytes": wb, "alg_bytes": alg,
                               "weight_gbs": wb / t / 1e9, "alg_gbs": alg / t / 1e9,
                               "frac_hbm": alg / t / 1e9 / HBM_PEAK_GBS,
                               "copies_rotated": len(copies)})
        del copies
    return {"lins": lins, "bufs": bufs, "layer_bytes": layer_bytes, "ncopies": ncopies,
            "ms": list(ms), "step_s": step_s,
            "value_gbs": layer_bytes * len(ms) / step_s / 1e9, "per_launch": per_launch}


def floor_lib():
    """libq4floor.so (the measurement kernels: the plain read of
    include/q4_read_floor.h and the matrix-core ceiling of
    include/q4_mfma_ceiling.h)."""
    import ctypes
    import torch  # noqa: F401  (its HIP runtime first, as for libq4)
    L = ctypes.CDLL(str(ROOT / "bit_block_quantized_q4_amd" / "libq4floor.so"))
    L.q4_read_floor.restype = ctypes.c_int
    L.q4_read_floor.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_void_p]
    L.q4_mfma_ceiling.restype = ctypes.c_int
    L.q4_mfma_ceiling.argtypes = [ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    return L


CEILING_WAVES, CEILING_PRODUCTS = 8, 8     # waves per workgroup, products per wave and step
CEILING_FLOP = 2.0 * 32 * 32 * 16          # one v_mfma_f32_32x32x16_f16


def ceiling_flop(workgroups, iters):
    """Flops of one q4_mfma_ceiling launch."""
    return float(workgroups) * CEILING_WAVES * iters * CEILING_PRODUCTS * CEILING_FLOP


def bench_mfma_ceiling(torch, dev, reps=4, iters=4096, seed=0x5EED):
    """The matrix cores' sustained rate under a long dense load: libq4floor's
    ceiling kernel (the GEMM tile's fragment reads and fp16 matrix products,
    nothing else) on one workgroup per compute unit, launches about as long
    as the layer's gate/up GEMM, replayed back to back after the clock
    settles; the shader clock is sampled meanwhile."""
    L = floor_lib()
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(cu * 64 * CEILING_WAVES, dtype=torch.float32, device=dev)

    def launch():
        rc = L.q4_mfma_ceiling(seed, iters, sink.data_ptr(), cu, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"q4_mfma_ceiling returned {rc}")
    t = time_gemm_calls(torch, launch, reps)
    g = capture(torch, launch)
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            for _ in range(20):
                g.replay()
            torch.cuda.synchronize()
    del g, sink
    tf = ceiling_flop(cu, iters) / t / 1e12
    return {"op": "libq4floor q4_mfma_ceiling: v_mfma_f32_32x32x16_f16 with fragment reads "
                  "from LDS, 8 waves per workgroup, one workgroup per compute unit",
            "workgroups": cu, "iters": iters, "mean_us": t * 1e6, "tflops": tf,
            "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS, "clock": clk.summary()}


FLOOR_GRIDS = (256, 512, 1024, 2048, 4096)


def bench_read_floor(torch, bufs, rotate_bytes, reps):
    """A plain read of the same bytes: libq4floor's streaming kernel over each
    group's packed buffer, >= rotate_bytes of rotated copies as the GEMV reads
    them, at several grid sizes (the best is reported).  It does no Q4_0
    work, so it shows what streaming these bytes in one launch costs here."""
    L = floor_lib()
    out = {}
    for g, buf in bufs.items():
        copies = rotated(torch, buf, rotate_bytes)
        nb = buf.numel()
        sink = torch.empty(max(FLOOR_GRIDS) * 256, dtype=torch.int32, device=buf.device)
        best = None
        for gi, wg in enumerate(FLOOR_GRIDS):
            def fn(wg=wg):
                st = torch.cuda.current_stream().cuda_stream
                for i in range(reps):
                    rc = L.q4_read_floor(copies[i % len(copies)].data_ptr(), nb, sink.data_ptr(), wg, st)
                    if rc != 0:
                        raise RuntimeError(f"q4_read_floor returned {rc}")
            gr = capture(torch, fn)
            gr.replay()
            # the clock is settled once per group (the grids are one load)
            t = replay_seconds(torch, gr, settle_s=None if gi == 0 else 0.0) / reps
            del gr
            if best is None or t < best[0]:
                best = (t, wg)
        del copies, sink
        t, wg = best
        out[g] = {"bytes": nb, "mean_us": t * 1e6, "gbs": nb / t / 1e9,
                  "frac_hbm": nb / t / 1e9 / HBM_PEAK_GBS, "workgroups": wg}
    return out


class ClockSampler:
    """Samples the GPU's shader clock (amdsmi, MHz) on a host thread while a
    leg runs; reports None where amdsmi cannot read it."""

    def __init__(self, period_s=0.005):
        self.period, self.samples, self.error = period_s, [], None
        self._stop, self._thread, self._h = None, None, None

    def __enter__(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read = lambda: amdsmi.amdsmi_get_clock_info(self._h, amdsmi.AmdSmiClkType.GFX)["clk"]
            self._read()
        except Exception as e:  # noqa: BLE001 - any failure leaves the clock unreported
            self.error = f"{type(e).__name__}: {e}"[:200]
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    self.samples.append(float(self._read()))
                except Exception:  # noqa: BLE001
                    pass
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        try:
            import amdsmi
            amdsmi.amdsmi_shut_down()
        except Exception:  # noqa: BLE001
            pass
        return False

    def summary(self):
        if not self.samples:
            return {"sclk_mhz": None, "error": self.error or "no samples"}
        v = np.array(self.samples)
        return {"sclk_mhz_median": float(np.median(v)), "sclk_mhz_min": float(v.min()),
                "sclk_mhz_max": float(v.max()), "samples": int(v.size), "peak_sclk_mhz": 2400.0}


def bench_headline_prefill(q4, torch, dev, lins, bufs, reps, m=4096):
    """The layer's prefill at M = m: the four launches as a step, and each on
    its own (one weight copy: the GEMM is bound by the matrix cores), with
    the shader clock sampled meanwhile."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    x = torch.randn((m, lins["q"].k), device=dev, generator=gen).half()
    xd = torch.randn((m, lins["down"].k), device=dev, generator=gen).half()
    ys = {g: torch.empty((m, group_shape(lins, g)[0]), dtype=torch.float16, device=dev)
          for g, _ in LAYER_GROUPS}
    wsz = max([q4.q4_gemm_workspace_size(m, *group_shape(lins, g)) for g, _ in LAYER_GROUPS] + [1])
    work = torch.empty(wsz, dtype=torch.uint8, device=dev)

    def launch(g):
        q4.q4_gemm(xd if g == "down" else x, bufs[g], y=ys[g], workspace=work)

    def step():
        for g, _ in LAYER_GROUPS:
            launch(g)

    flop_step = sum(2.0 * m * group_shape(lins, g)[0] * group_shape(lins, g)[1] for g, _ in LAYER_GROUPS)
    t_step = time_gemm_calls(torch, step, reps)
    per_launch = []
    for g, _ in LAYER_GROUPS:
        rows, k = group_shape(lins, g)
        t = time_gemm_calls(torch, lambda g=g: launch(g), reps)
        fl = 2.0 * m * rows * k
        per_launch.append({"group": g, "m": m, "n": rows, "k": k, "mean_us": t * 1e6,
                           "flop": fl, "tflops": fl / t / 1e12,
                           "frac_mfma": fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS})
    # The shader clock under this load: the step replayed back to back for
    # about a second while a host thread samples it.
    gsoak = capture(torch, step)
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            for _ in range(20):
                gsoak.replay()
            torch.cuda.synchronize()
    del gsoak
    tf = flop_step / t_step / 1e12
    dom = max(per_launch, key=lambda r: r["mean_us"])
    return {"workload": f"layer_27b_dense prefill, M = {m}, 4 launches (q/k/v and gate/up fused)",
            "m": m, "us_per_layer": t_step * 1e6, "tflops": tf, "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS,
            "per_launch": per_launch, "clock": clk.summary(),
            "roofline": {"bound": "mfma", "achieved": dom["tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": dom["frac_mfma"],
                         "traffic": load_traffic(f"gemm_layer_{dom['group']}_m{m}"),
                         "kernel": f"q4_gemm {dom['group']} {m}x{dom['n']}x{dom['k']}",
                         "mean_us": dom["mean_us"], "alg_flop_per_launch": dom["flop"],
                         "mfma_util_pct": load_mfma_util(f"gemm_layer_{dom['group']}_m{m}")}}


def group_views(lins, bufs):
    """Each linear's packed rows as a row slice of its group's buffer."""
    views = {}
    for g, names in LAYER_GROUPS:
        r = 0
        for nm in names:
            views[nm] = bufs[g][r:r + lins[nm].n]
            r += lins[nm].n
    return views


def bench_layer_decode(q4, torch, dev, lins, bufs, steps, rotate_bytes, ms=(1, 10)):
    """Decode through the layer's seven linears (q, k, v, o, gate, up, down)
    at M = 1 and 10: seven launches, against four where q/k/v and gate/up run
    as one launch each on their packed rows concatenated (packed rows are
    independent, so a concatenated buffer is simply a taller weight).  Each
    linear's packed copy is a row slice of its group's buffer, so both variants
    stream the same bytes; layer copies are rotated over >= 1 GiB."""
    layer_bytes = sum(packed_bytes(*group_shape(lins, g)) for g, _ in LAYER_GROUPS)
    copies = max(2, -(-rotate_bytes // layer_bytes))
    layers = [bufs] + [{g: b.clone() for g, b in bufs.items()} for _ in range(copies - 1)]
    lviews = [group_views(lins, lay) for lay in layers]
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    res = {}
    for m in ms:
        x = torch.randn((m, lins["q"].k), device=dev, generator=gen).half()
        xd = torch.randn((m, lins["down"].k), device=dev, generator=gen).half()
        ysep = {nm: torch.empty((m, l.n), dtype=torch.float16, device=dev) for nm, l in lins.items()}
        ygrp = {g: torch.empty((m, group_shape(lins, g)[0]), dtype=torch.float16, device=dev)
                for g, _ in LAYER_GROUPS}

        def separate():
            for i in range(steps):
                views = lviews[i % copies]
                for nm in ("q", "k", "v", "o", "gate", "up"):
                    q4.q4_gemv(x, views[nm], y=ysep[nm])
                q4.q4_gemv(xd, views["down"], y=ysep["down"])

        def fused():
            for i in range(steps):
                lay = layers[i % copies]
                for g in ("qkv", "o", "gateup"):
                    q4.q4_gemv(x, lay[g], y=ygrp[g])
                q4.q4_gemv(xd, lay["down"], y=ygrp["down"])

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


def bench_layer_prefill(q4, torch, dev, lins, bufs, reps, ms=(256, 4096)):
    """Prefill through the layer's seven linears at M = 256 (one chunk) and
    4096 rows: seven launches, and four with q/k/v and gate/up each run on
    their concatenated packed rows.  The GEMM is bound by the matrix cores,
    so one copy of the layer's weights serves every call."""
    views = group_views(lins, bufs)
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    flop_per_row = 2.0 * sum(l.n * l.k for l in lins.values())
    res = {}
    for m in ms:
        x = torch.randn((m, lins["q"].k), device=dev, generator=gen).half()
        xd = torch.randn((m, lins["down"].k), device=dev, generator=gen).half()
        ysep = {nm: torch.empty((m, l.n), dtype=torch.float16, device=dev) for nm, l in lins.items()}
        ygrp = {g: torch.empty((m, group_shape(lins, g)[0]), dtype=torch.float16, device=dev)
                for g, _ in LAYER_GROUPS}
        wsz = max([q4.q4_gemm_workspace_size(m, *group_shape(lins, g)) for g, _ in LAYER_GROUPS] +
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


SEPARATOR = "bitwise_not"  # the torch kernel launched between counted launch groups
ATTN_MS = (1, 4, 10, 16)
DECODE_MS = (1, 10)


def traffic_keys():
    """The launch groups of traffic_run, in launch order."""
    keys = ["calib_copy"]
    keys += [f"gemv_layer_{g}_m{m}" for g, _ in LAYER_GROUPS for m in DECODE_MS]
    keys += [f"gemv_5120x5120_m{m}" for m in ATTN_MS]
    keys += ["quantize_fp32_5120x5120"]
    keys += [f"gemm_layer_{g}_m4096" for g, _ in LAYER_GROUPS]
    keys += ["gemm_2048x17408x5120"]
    return keys


TRAFFIC_LAUNCHES = {"gemv": 20, "quantize": 20, "gemm": 3, "calib": 3}


def launches_of(key):
    return TRAFFIC_LAUNCHES[key.split("_")[0]]


def separator(torch, dev):
    a = torch.zeros(64, dtype=torch.int8, device=dev)
    b = torch.empty_like(a)
    return lambda: torch.bitwise_not(a, out=b)


def traffic_run(q4, torch, dev, rotate_bytes):
    """The launches the counter passes (FETCH_SIZE, WRITE_SIZE, SQ) read, in
    the order of traffic_keys(), a separator kernel after each group: a plain
    device copy of known size (torch's negation kernel: reads and writes
    TRAFFIC_CALIB_BYTES once); the headline layer's decode launches (rotated
    copies, as timed); the 5120 x 5120 GEMV at each batch size; the quantiser;
    the layer's prefill launches at M = 4096; the 2048-row prefill."""
    sep = separator(torch, dev)
    src = torch.ones(TRAFFIC_CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(launches_of("calib")):
        torch.neg(src, out=dst)
    sep()
    del src, dst
    lins, bufs, _ = layer_setup(q4, torch, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    for g, _ in LAYER_GROUPS:
        rows, k = group_shape(lins, g)
        copies = rotated(torch, bufs[g], rotate_bytes)
        for m in DECODE_MS:
            x = torch.randn((m, k), device=dev, generator=gen).half()
            y = torch.empty((m, rows), dtype=torch.float16, device=dev)
            for i in range(launches_of("gemv")):
                q4.q4_gemv(x, copies[i % len(copies)], y=y)
            sep()
        del copies
    s = gemv_setup(q4, torch, dev, rotate_bytes)
    for m in ATTN_MS:
        gemv_launches(q4, s, launches_of("gemv"), [m], 0)()
        sep()
    ws = [torch.from_numpy(s["w_host"]).to(dev) for _ in range(2)]
    for i in range(launches_of("quantize")):
        q4.q4_quantize(ws[i % 2], packed=s["packed"][0])
    sep()
    del s, ws
    m = 4096
    x = torch.randn((m, lins["q"].k), device=dev, generator=gen).half()
    xd = torch.randn((m, lins["down"].k), device=dev, generator=gen).half()
    for g, _ in LAYER_GROUPS:
        rows, k = group_shape(lins, g)
        y = torch.empty((m, rows), dtype=torch.float16, device=dev)
        for _ in range(launches_of("gemm")):
            q4.q4_gemm(xd if g == "down" else x, bufs[g], y=y)
        sep()
    del x, xd, bufs
    _, _, _, whole, _ = gemm_setup(q4, torch, dev)
    for _ in range(launches_of("gemm")):
        whole()
    sep()
    torch.cuda.synchronize()
    print("traffic launches done", flush=True)


def mfma_keys():
    return [f"gemm_layer_{g}_m4096" for g, _ in LAYER_GROUPS] + [
        "gemm_2048x17408x5120", "gemm_8x256x17408x5120"]


def mfma_run(q4, torch, dev, reps=3):
    """The launches the matrix-core counter pass (MfmaUtil, MfmaFlopsF16)
    reads, in the order of mfma_keys(), a separator kernel after each group:
    the layer's prefill launches at M = 4096, the 2048 x 17408 x 5120 prefill
    as one launch and as 8 chunks of 256 rows (reps times each)."""
    sep = separator(torch, dev)
    lins, bufs, _ = layer_setup(q4, torch, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    m = 4096
    x = torch.randn((m, lins["q"].k), device=dev, generator=gen).half()
    xd = torch.randn((m, lins["down"].k), device=dev, generator=gen).half()
    for g, _ in LAYER_GROUPS:
        rows, _k = group_shape(lins, g)
        y = torch.empty((m, rows), dtype=torch.float16, device=dev)
        for _ in range(reps):
            q4.q4_gemm(xd if g == "down" else x, bufs[g], y=y)
        sep()
    del x, xd, bufs
    _, _, _, whole, chunked = gemm_setup(q4, torch, dev)
    for _ in range(reps):
        whole()
    sep()
    for _ in range(reps):
        chunked(256)()
    sep()
    torch.cuda.synchronize()
    print("mfma launches done", flush=True)


PHASE_SLOTS = 64  # per computing wave: entry, 31 barriers, 31 phase ends, exit


def trace_lib():
    """libq4trace.so: libq4 with the tile GEMV's computing waves recording the
    shader clock per phase (a measurement build; only --phase-trace loads it)."""
    import ctypes
    import bit_block_quantized_q4_amd as q4
    from bit_block_quantized_q4_amd.build import TRACE_LIB_PATH
    L = ctypes.CDLL(str(TRACE_LIB_PATH))
    for name, (res, args) in q4._SIGS.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    L.q4_phase_trace_set.restype = ctypes.c_int
    L.q4_phase_trace_set.argtypes = [ctypes.c_void_p]
    return L


def phase_summary(stamps, nw=8):
    """Per-phase medians over workgroups (shader-clock cycles) from a
    [workgroups, nw, PHASE_SLOTS] array of one launch's stamps (zeros where
    nothing was recorded): the time from entry to phase 0's barrier, each
    period between consecutive barriers, each phase's products (its slowest
    computing wave's end after the barrier), entry to exit, and the shader
    clock over the launch (shader cycles per tick of the 100 MHz clock read
    at entry and exit, in MHz)."""
    T = np.asarray(stamps, dtype=np.int64)
    T = T[T[:, 0, 0] > 0]  # workgroups that ran
    n = int(np.count_nonzero(T[0, 0, 1:31]))  # phases recorded (at most 30)
    bar = T[:, 0, 1:1 + n]
    done = T[:, :nw, 32:32 + n].max(axis=1)
    ticks = T[:, 0, 62] - T[:, 0, 31]
    ok = ticks > 0
    sclk = (T[ok, 0, 63] - T[ok, 0, 0]) / ticks[ok] * 100.0
    out = {"workgroups": int(T.shape[0]), "phases": n,
           "entry_to_first_barrier": float(np.median(bar[:, 0] - T[:, 0, 0])),
           "period": [float(v) for v in np.median(np.diff(bar, axis=1), axis=0)],
           "products": [float(v) for v in np.median(done - bar, axis=0)],
           "entry_to_exit": float(np.median(T[:, 0, 63] - T[:, 0, 0])),
           "sclk_mhz": float(np.median(sclk)) if sclk.size else None}
    # The 100 MHz clock is common to the whole device (the shader clock's
    # counter is not): the launch's span from the first workgroup's entry to
    # the last one's exit, the spread of entries, and the median and slowest
    # workgroup, in microseconds.
    if ok.all() and T.shape[0] > 0:
        e, x = T[:, 0, 31], T[:, 0, 62]
        out.update({"launch_span_us": float(x.max() - e.min()) / 100.0,
                    "entry_spread_us": float(e.max() - e.min()) / 100.0,
                    "workgroup_us_median": float(np.median(x - e)) / 100.0,
                    "workgroup_us_max": float((x - e).max()) / 100.0})
    return out


def merge_phase_summaries(summs):
    """Element-wise medians of several launches' phase_summary results."""
    out = {}
    for key, v in summs[0].items():
        vals = [s[key] for s in summs if key in s]
        if isinstance(v, list):
            out[key] = [float(np.median(c)) for c in zip(*vals)]
        elif key in ("workgroups", "phases"):
            out[key] = v
        elif any(x is None for x in vals) or len(vals) != len(summs):
            out[key] = None
        else:
            out[key] = float(np.median(vals))
    return out


def phase_trace_run(q4, torch, dev, rotate_bytes, steps=50, replays=5):
    """The headline's m = 10 launches (the tile GEMV) on libq4trace.so, clock
    settled: per group, the phase clocks of the last launch of each of
    `replays` graph replays, summarised by phase_summary and merged by
    element-wise medians, with the replays' mean launch time."""
    import bit_block_quantized_q4_amd.build as qb
    L = trace_lib()
    saved = q4._LIB
    q4._LIB = L
    out = {}
    try:
        lins, bufs, _ = layer_setup(q4, torch, dev)
        gen = torch.Generator(device=dev)
        gen.manual_seed(9)
        m = 10
        for g, _ in LAYER_GROUPS:
            rows, k = group_shape(lins, g)
            x = torch.randn((m, k), device=dev, generator=gen).half()
            y = torch.empty((m, rows), dtype=torch.float16, device=dev)
            copies = rotated(torch, bufs[g], rotate_bytes)
            buf = torch.zeros(((rows + 15) // 16 + 1) * 8 * PHASE_SLOTS, dtype=torch.int64, device=dev)

            def fn(copies=copies, x=x, y=y):
                for i in range(steps):
                    q4.q4_gemv(x, copies[i % len(copies)], y=y)
            gr = capture(torch, fn)
            if L.q4_phase_trace_set(buf.data_ptr()) != 0:
                raise RuntimeError("q4_phase_trace_set failed")
            summs, times = [], []
            for r in range(replays):
                times.append(replay_seconds(torch, gr, settle_s=SETTLE_S if r == 0 else None) / steps)
                summs.append(phase_summary(buf.view(-1, 8, PHASE_SLOTS).cpu().numpy()))
            L.q4_phase_trace_set(None)
            del gr
            summ = merge_phase_summaries(summs)
            summ.update({"group": g, "m": m, "n": rows, "k": k,
                         "mean_us": float(np.median(times)) * 1e6, "replays": replays})
            out[f"gemv_layer_{g}_m{m}"] = summ
            print(json.dumps({kk: summ.get(kk) for kk in ("group", "mean_us", "workgroups", "phases",
                                                          "sclk_mhz", "launch_span_us")}), flush=True)
            del copies, buf
    finally:
        q4._LIB = saved
    data = {"kernel_hash": kernel_hash(), "trace_lib": qb.TRACE_LIB_PATH.name, "launches": out}
    (ROOT / "profiles" / "phase_trace.json").write_text(json.dumps(data, indent=1) + "\n")
    return data


def _ours(name):
    return "q4::" in name or name.startswith("_ZN2q4")


def _kernel_label(name):
    """A short label of one of this library's kernels from its (mangled or
    demangled) name."""
    import re
    for pat, lab in (("gemm_mfma_kernel", "gemm_mfma"), ("gemm_slicek_kernel", "gemm_slicek"),
                     ("gemm_exact_kernel", "gemm_exact"), ("gemm_tile_kernel", "gemm_tile"),
                     ("splitk_reduce", "splitk_reduce"), ("bf16_rows_to_f16", "bf16_stage"),
                     ("gemv_tile_kernel", "gemv_tile"), ("gemv_bal_kernel", "gemv_bal"),
                     ("gemv_stream_kernel", "gemv_stream"), ("gemv_rowwave", "gemv_rowwave"),
                     ("quantize", "quantize")):
        if pat in name:
            if lab == "gemm_mfma":
                lab += "_256x256" if ("ILi256" in name or "<256" in name) else "_128x128"
            if lab in ("gemm_mfma_256x256", "gemm_mfma_128x128", "gemm_slicek", "splitk_reduce"):
                if re.search(r"kernelI(?:Li\d+E)*fE", name) or "float>" in name:
                    lab += "_f32"
            return lab
    return "other"


def _grouped(csv_path, counter, keys):
    """Per launch group (keys, in order), per kernel label, the per-dispatch
    values of one counter: the separator dispatches split the rows."""
    out = {k: {} for k in keys}
    i = 0
    for did, name, cnt, val in _pmc_rows(csv_path):
        if cnt != counter:
            continue
        if SEPARATOR in name:
            i += 1
            continue
        if i >= len(keys):
            break
        key = keys[i]
        if key == "calib_copy":
            if "neg" in name:
                out[key].setdefault("neg", []).append(val)
            continue
        if _ours(name):
            lab = _kernel_label(name)
            # only the kernel family the group launches (set-up work such as
            # quantising the weights shares the segment)
            fam = key.split("_")[0]
            if (fam == "gemv" and lab.startswith("gemv")) or (fam == "quantize" and lab == "quantize") or \
               (fam == "gemm" and (lab.startswith("gemm") or lab in ("splitk_reduce", "splitk_reduce_f32",
                                                                      "bf16_stage"))):
                out[key].setdefault(lab, []).append(val)
    return out


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


def mfma_summary(csv_path, out_path):
    """profiles/mfma.json from the counter pass over mfma_run: per launch group
    and kernel, the median per dispatch of MfmaUtil (matrix-core busy cycles
    over the dispatch's active cycles) and of MfmaFlopsF16 (fp16 matrix flops
    issued)."""
    keys = mfma_keys()
    groups = {}
    for cnt in ("MfmaUtil", "MfmaFlopsF16"):
        for key, by in _grouped(csv_path, cnt, keys).items():
            for lab, vals in by.items():
                e = groups.setdefault(key, {}).setdefault(lab, {})
                e[cnt] = float(np.median(vals))
                e["dispatches"] = len(vals)
    kernels = {}
    for key, by in groups.items():
        # the group's kernel issuing the most matrix flops stands for it (the main tiles)
        main = max(by.items(), key=lambda kv: kv[1].get("MfmaFlopsF16", 0.0))
        kernels[key] = {"main_kernel": main[0], "MfmaUtil": main[1].get("MfmaUtil"), "by_kernel": by}
    data = {"kernel_hash": kernel_hash(),
            "workload": "bench.py --mfma: the layer prefill at M = 4096 (4 launches), and "
                        "2048 x 17408 x 5120 whole and as 8 x 256-row chunks",
            "peak_mfma_f16_tflops": MFMA_F16_PEAK_TFLOPS, "kernels": kernels}
    Path(out_path).write_text(json.dumps(data, indent=1) + "\n")
    return data


SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
               "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT")


def sq_summary(csv_path, out_path):
    """profiles/sq.json from one counter pass of SQ_COUNTERS over traffic_run:
    per launch group, the median per dispatch of each counter over the
    group's kernels, and the ratios read from them (waiting cycles per wave
    cycle; LDS bank-conflict cycles per cycle of LDS instruction activity)."""
    keys = traffic_keys()
    kernels = {}
    for c in SQ_COUNTERS:
        for key, by in _grouped(csv_path, c, keys).items():
            if key == "calib_copy" or not by:
                continue
            vals = [v for vs in by.values() for v in vs]
            kernels.setdefault(key, {})[c] = float(np.median(vals))
            kernels[key]["dispatches"] = len(vals)
    for v in kernels.values():
        wc = v.get("SQ_WAVE_CYCLES") or 0.0
        lds = v.get("SQ_ACTIVE_INST_LDS") or 0.0
        v["wait_any_per_wave_cycle"] = v.get("SQ_WAIT_ANY", 0.0) / wc if wc else None
        v["wait_inst_per_wave_cycle"] = v.get("SQ_WAIT_INST_ANY", 0.0) / wc if wc else None
        v["lds_conflict_per_lds_active"] = v.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds else None
    data = {"kernel_hash": kernel_hash(), "counters": list(SQ_COUNTERS), "kernels": kernels}
    Path(out_path).write_text(json.dumps(data, indent=1) + "\n")
    return data


def traffic_summary(fetch_csv, write_csv, out_path):
    """profiles/traffic.json from the two counter passes: per launch group, the
    FETCH_SIZE and WRITE_SIZE of one launch (all its dispatches, KiB, summed
    over the group and divided by its launches), each scaled by known bytes /
    counted bytes of the plain copy."""
    keys = traffic_keys()
    fetch = _grouped(fetch_csv, "FETCH_SIZE", keys)
    write = _grouped(write_csv, "WRITE_SIZE", keys)
    calf = float(np.median(fetch["calib_copy"]["neg"]))
    calw = float(np.median(write["calib_copy"]["neg"]))
    f_scale = TRAFFIC_CALIB_BYTES / (calf * 1024.0)
    w_scale = TRAFFIC_CALIB_BYTES / (calw * 1024.0)
    kernels = {}
    for key in keys[1:]:
        if not fetch[key] or not write[key]:
            continue
        nl = launches_of(key)
        fk = sum(sum(v) for v in fetch[key].values()) / nl
        wk = sum(sum(v) for v in write[key].values()) / nl
        fb, wb = fk * 1024.0 * f_scale, wk * 1024.0 * w_scale
        kernels[key] = {"fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb,
                        "fetch_kib_raw": fk, "write_kib_raw": wk,
                        "dispatches_per_launch": {lab: len(v) / nl for lab, v in fetch[key].items()}}
    data = {"kernel_hash": kernel_hash(),
            "calibration": {"bytes": TRAFFIC_CALIB_BYTES, "fetch_kib": calf, "write_kib": calw,
                            "fetch_scale": f_scale, "write_scale": w_scale},
            "kernels": kernels}
    Path(out_path).write_text(json.dumps(data, indent=1) + "\n")
    return data


def trace_summary(trace_csv):
    """Per headline launch (group, batch size), the mean duration of the GEMV
    dispatches that bench_headline_decode times, from a rocprofv3 kernel-trace
    CSV of a default run: each timed replay sits between two marker
    (SEPARATOR) kernels, the run's first markers, in LAYER_GROUPS x DECODE_MS
    order."""
    import csv
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            ours = _ours(name) and "gemv_" in name and "_kernel" in name
            if ours or SEPARATOR in name:
                start = int(r.get("Start_Timestamp") or r.get("Start-Timestamp"))
                end = int(r.get("End_Timestamp") or r.get("End-Timestamp"))
                rows.append((start, end - start, name, ours))
    rows.sort()
    marks = [i for i, r in enumerate(rows) if not r[3]]
    out, j = [], 0
    for g, _ in LAYER_GROUPS:
        for m in DECODE_MS:
            rep = [r for r in rows[marks[2 * j] + 1:marks[2 * j + 1]] if r[3]] \
                if 2 * j + 1 < len(marks) else []
            j += 1
            out.append({"group": g, "m": m, "dispatches": len(rep),
                        "mean_us": float(np.mean([r[1] for r in rep])) / 1e3 if rep else None,
                        "kernels": sorted({r[2] for r in rep})})
    return out


def cpu_baseline(budget_s=1.0):
    """The oracle, as it stands, per configuration: quantise and matmul on
    bounded samples of each configuration's own seeded inputs (a seeded
    subset of weight rows; every configuration's batch sizes), with the BLAS
    thread pool set to the cores this process may run on.  Each sample is
    repeated for about budget_s seconds and scaled to the configuration's
    units.  `value` is the layer decode step's packed-weight GB/s, the
    headline's unit."""
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover - threadpoolctl missing
        limiter = None

    def rep(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return el / n

    def sample_rows(w, rows):
        rng = np.random.default_rng(w.shape[0])
        return np.ascontiguousarray(w[np.sort(rng.choice(w.shape[0], size=min(rows, w.shape[0]),
                                                         replace=False))])

    per = []
    try:
        for wid in (1, 2, 3, 4):
            wl = synth.WORKLOADS[wid]
            lin = wl.linears[0]
            w = sample_rows(synth.workload_weights(wl, lin), 1024 if wid != 4 else 256)
            r = w.shape[0]
            tq = rep(lambda: oracle.quantize(w))
            packed = oracle.quantize(w)
            row = {"config": wl.name, "rows_sampled": r, "of_rows": lin.n,
                   "quantize_mweights_per_s": r * lin.k / tq / 1e6}
            mm = {}
            for m in wl.ms:
                x = synth.workload_activations(wl, lin.k, m)
                t = rep(lambda: oracle.matmul_ref(x, packed, r, lin.k))
                mm[f"m{m}"] = {"weight_gbs": packed_bytes(r, lin.k) / t / 1e9,
                               "gflops": 2.0 * m * r * lin.k / t / 1e9,
                               "full_config_s": t * lin.n / r}
            row["matmul"] = mm
            per.append(row)
            del w, packed
        wl = synth.WORKLOADS[5]
        row = {"config": wl.name, "rows_sampled_per_linear": 512, "matmul": {}}
        samples = {}
        tq_tot, wq = 0.0, 0
        for lin in wl.linears:
            w = sample_rows(synth.workload_weights(wl, lin), 512)
            tq_tot += rep(lambda: oracle.quantize(w)) if lin.name in ("q", "down") else 0.0
            wq += w.size if lin.name in ("q", "down") else 0
            samples[lin.name] = (oracle.quantize(w), lin)
            del w
        row["quantize_mweights_per_s"] = wq / tq_tot / 1e6
        for m in (1, 10, 256):
            xs = {kk: synth.workload_activations(wl, kk, m) for kk in {l.k for l in wl.linears}}

            def layer():
                for packed, lin in samples.values():
                    oracle.matmul_ref(xs[lin.k], packed, packed.shape[0], lin.k)

            t = rep(layer)
            wb = sum(packed_bytes(p.shape[0], l.k) for p, l in samples.values())
            fl = sum(2.0 * m * p.shape[0] * l.k for p, l in samples.values())
            row["matmul"][f"m{m}"] = {"weight_gbs": wb / t / 1e9, "gflops": fl / t / 1e9}
        per.append(row)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    dec = per[-1]["matmul"]
    # the layer decode step (M = 1 and 10 back to back) at the oracle's rates
    step_gbs = 2.0 / (1.0 / dec["m1"]["weight_gbs"] + 1.0 / dec["m10"]["weight_gbs"])
    return {"value": step_gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "per configuration, a seeded subset of weight rows (1024 rows of the "
                      "single linears, 256 of the prefill weight, 512 of each layer linear) "
                      "quantised and multiplied by the configuration's activations at each of "
                      f"its batch sizes, each repeated for ~{budget_s:.0f} s; value: the layer "
                      "decode step (M = 1 then 10) at the sampled rates",
            "per_config": per}


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
    ap.add_argument("--phase-trace", action="store_true",
                    help="per-phase clocks of the m = 10 decode launches on libq4trace.so "
                         "(writes profiles/phase_trace.json)")
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
        for r in trace_summary(args.trace_summary):
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
    if args.phase_trace:
        phase_trace_run(q4, torch, dev, rotate)
        return

    t_start = time.perf_counter()

    def progress(leg):
        print(f"[bench] {leg} done at {time.perf_counter() - t_start:.1f} s", file=sys.stderr,
              flush=True)

    out = {"metric": METRIC}
    h = bench_headline_decode(q4, torch, dev, args.steps, args.warmup, rotate)
    lins, bufs = h["lins"], h["bufs"]
    dom = max(h["per_launch"], key=lambda r: r["mean_us"])  # the step's dominant launch
    out.update({
        "value": h["value_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": h["step_s"] * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "layer_27b_dense_7_linears: decode step, q/k/v and gate/up fused "
                               "(4 q4_gemv launches per batch size)",
                   "ms": h["ms"], "linears": {nm: [l.n, l.k] for nm, l in lins.items()},
                   "groups": {g: list(group_shape(lins, g)) for g, _ in LAYER_GROUPS},
                   "weights": "Student-t(3) x 0.02, quantised by q4_quantize",
                   "x_dtype": "f16", "y_dtype": "f16",
                   "weight_bytes_per_batch_size": h["layer_bytes"],
                   "layer_copies_rotated": h["ncopies"]},
        "roofline": {"bound": "hbm", "achieved": dom["alg_gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": dom["alg_gbs"] / HBM_PEAK_GBS,
                     "traffic": load_traffic(f"gemv_layer_{dom['group']}_m{dom['m']}"),
                     "kernel": f"q4_gemv {dom['group']} m={dom['m']} ({dom['n']}x{dom['k']})",
                     "mean_us": dom["mean_us"], "alg_bytes_per_launch": dom["alg_bytes"]},
        "per_launch": h["per_launch"],
    })
    progress("headline decode")
    floor = bench_read_floor(torch, bufs, rotate, min(args.steps, 100))
    floor_step = sum(floor[g]["mean_us"] for g, _ in LAYER_GROUPS) * len(h["ms"])
    out["read_floor"] = {"op": "libq4floor plain streaming read of each group's packed buffer, "
                               "rotated like the GEMV's copies, best of grids "
                               + "/".join(map(str, FLOOR_GRIDS)), "per_group": floor,
                         "step_us": floor_step,
                         "gemv_step_over_floor": h["step_s"] * 1e6 / floor_step}
    progress("read floor")
    out["gemm"] = bench_headline_prefill(q4, torch, dev, lins, bufs, args.gemm_reps)
    ceil = bench_mfma_ceiling(torch, dev)
    out["gemm"]["mfma_ceiling"] = ceil
    out["gemm"]["roofline"]["ceiling_tflops"] = ceil["tflops"]
    out["gemm"]["roofline"]["frac_of_ceiling"] = out["gemm"]["roofline"]["achieved"] / ceil["tflops"]
    progress("headline prefill")
    if args.only in ("all", "gemm"):
        out["gemm"]["prefill_2048x17408x5120"] = bench_gemm(q4, torch, dev, args.gemm_reps)
    if args.only in ("all", "layer"):
        out["layer_decode"] = bench_layer_decode(q4, torch, dev, lins, bufs, min(args.steps, 50), rotate)
        out["layer_prefill"] = bench_layer_prefill(q4, torch, dev, lins, bufs, 3)
    progress("layer legs")
    del h, bufs
    torch.cuda.empty_cache()
    g = bench_gemv(q4, torch, dev, args.steps, args.warmup, rotate)
    out["attn_proj"] = {"workload": g["wl"].name, "n": g["n"], "k": g["k"], "ms": g["ms"],
                        "weight_copies_rotated": g["ncopies"], "step_us": g["step_s"] * 1e6,
                        "weight_gbs": g["value_gbs"], "per_m": g["per_m"]}
    progress("attn proj")
    if args.only in ("all", "quantize"):
        out["quantize"] = bench_quantize(q4, torch, dev, g["w_host"], 20, rotate)
    if args.only in ("all", "other"):
        out["other_configs"] = bench_other_configs(q4, torch, dev, args.steps, rotate)
    if args.only in ("all", "bf16"):
        out["bf16"] = bench_bf16(q4, torch, dev, g["setup"], args.steps, args.gemm_reps)
    if args.only in ("all", "host"):
        out["host_twin"] = bench_host_twin(q4, torch, g["packed0"], g["n"], g["k"], g["ms"])
    progress("gpu legs")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    out["kernel_hash"] = kernel_hash()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
