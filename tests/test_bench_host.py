"""bench.py's host-side logic, without a GPU: attribution of rocprofv3 counter
rows to workloads, the copy-kernel scaling of FETCH_SIZE / WRITE_SIZE, the
wave-state ratios, the source-hash gate on committed summaries, and the
refusal of more than one GPU."""

import csv
import json
import subprocess
import sys
from pathlib import Path

import numpy as np
import pytest

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402

GEMV = "void q4::(anonymous namespace)::gemv_bal_kernel<8, 4, 1, false>(...)"
TILE = "void q4::(anonymous namespace)::gemv_tile_kernel<2, 1, 32, true, 8, 4, false, 32>(...)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)"
QUANT = "void q4::(anonymous namespace)::quantize_kernel<float, 4>(float const*, unsigned char*, long)"
GEMM = "void q4::(anonymous namespace)::gemm_mfma_kernel<256, 256, 2, 4, _Float16>(...)"
OTHER = "void at::native::FillFunctor<float>(...)"


def write_csv(path, rows):
    """rows: (dispatch id, kernel name, {counter: value})."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did, name, cnts in rows:
            for c, v in cnts.items():
                w.writerow([did, did, name, c, v])


SEP = "void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda(...)"
REDUCE = "void q4::(anonymous namespace)::splitk_reduce_kernel<_Float16>(...)"


def kernel_for(key):
    """A kernel name of the family a launch group dispatches."""
    if key.startswith("gemv"):
        return TILE
    if key.startswith("quantize"):
        return QUANT
    return GEMM


def grouped_rows(keys, per_key, counter):
    """A counter pass as bench.py's --traffic / --mfma runs launch it: per key
    launches_of(key) launches (GEMM launches as two dispatches, the main
    kernel and the split-K reduction), a separator after each group, with
    unrelated kernels in between.  per_key(key, i) -> the value of dispatch i."""
    rows, did = [], 1
    for key in keys:
        rows.append((did, OTHER, {counter: 9e9})); did += 1
        n = bench.launches_of(key)
        for i in range(n):
            if key == "calib_copy":
                rows.append((did, NEG, {counter: per_key(key, i)})); did += 1
                continue
            rows.append((did, kernel_for(key), {counter: per_key(key, i)})); did += 1
            if key.startswith("gemm"):
                rows.append((did, REDUCE, {counter: 1.0})); did += 1
        rows.append((did, SEP, {counter: 7e9})); did += 1
    return rows


def test_traffic_summary_attributes_and_scales(tmp_path):
    keys = bench.traffic_keys()
    calib_kib = bench.TRAFFIC_CALIB_BYTES / 1024.0
    fval = {k: 1000.0 * (i + 1) for i, k in enumerate(keys)}
    fval["calib_copy"] = calib_kib * 1.25   # the counter reads 25% high
    wval = {k: 10.0 * (i + 1) for i, k in enumerate(keys)}
    wval["calib_copy"] = calib_kib
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fcsv, grouped_rows(keys, lambda k, i: fval[k], "FETCH_SIZE"))
    write_csv(wcsv, grouped_rows(keys, lambda k, i: wval[k], "WRITE_SIZE"))
    out = tmp_path / "traffic.json"
    d = bench.traffic_summary(fcsv, wcsv, out)
    assert json.loads(out.read_text()) == d
    assert d["kernel_hash"] == bench.kernel_hash()
    assert d["calibration"]["fetch_scale"] == pytest.approx(0.8)
    assert d["calibration"]["write_scale"] == pytest.approx(1.0)
    k = d["kernels"]
    assert set(k) == set(keys[1:])
    for key in keys[1:]:
        extra = 1.0 if key.startswith("gemm") else 0.0   # the reduction's dispatch
        e = k[key]
        assert e["fetch_bytes"] == pytest.approx((fval[key] + extra) * 1024 * 0.8)
        assert e["write_bytes"] == pytest.approx((wval[key] + extra) * 1024)
        assert e["traffic_bytes"] == pytest.approx(e["fetch_bytes"] + e["write_bytes"])
    assert k["gemm_layer_gateup_m4096"]["dispatches_per_launch"] == {"gemm_mfma_256x256": 1.0,
                                                                     "splitk_reduce": 1.0}


def test_sq_summary_ratios(tmp_path):
    keys = bench.traffic_keys()
    counters = {"SQ_WAVE_CYCLES": lambda k, i: 1000.0, "SQ_WAIT_ANY": lambda k, i: 600.0 + keys.index(k),
                "SQ_WAIT_INST_ANY": lambda k, i: 100.0, "SQ_ACTIVE_INST_LDS": lambda k, i: 50.0,
                "SQ_LDS_BANK_CONFLICT": lambda k, i: 25.0 * keys.index(k)}
    rows = []
    for c, f in counters.items():
        rows += [(did + 100000 * list(counters).index(c), name, cnt)
                 for did, name, cnt in grouped_rows(keys, f, c)]
    p = tmp_path / "sq.csv"
    write_csv(p, rows)
    d = bench.sq_summary(p, tmp_path / "sq.json")
    k = d["kernels"]
    e = k["gemv_layer_gateup_m10"]
    i = keys.index("gemv_layer_gateup_m10")
    assert e["dispatches"] == bench.launches_of("gemv_layer_gateup_m10")
    assert e["wait_any_per_wave_cycle"] == pytest.approx((600.0 + i) / 1000.0)
    assert e["wait_inst_per_wave_cycle"] == pytest.approx(0.1)
    assert e["lds_conflict_per_lds_active"] == pytest.approx(0.5 * i)
    assert "calib_copy" not in k


def test_mfma_summary_takes_the_main_kernel(tmp_path):
    keys = bench.mfma_keys()
    rows = []
    for j, c in enumerate(("MfmaUtil", "MfmaFlopsF16")):
        f = (lambda k, i: 40.0 + keys.index(k)) if c == "MfmaUtil" else (lambda k, i: 1e12)
        rows += [(did + 100000 * j, name, cnt) for did, name, cnt in grouped_rows(keys, f, c)]
    p = tmp_path / "mfma.csv"
    write_csv(p, rows)
    d = bench.mfma_summary(p, tmp_path / "mfma.json")
    for i, key in enumerate(keys):
        e = d["kernels"][key]
        assert e["main_kernel"] == "gemm_mfma_256x256"
        assert e["MfmaUtil"] == pytest.approx(40.0 + i)


def test_trace_summary_picks_the_timed_replays(tmp_path):
    """Each timed replay sits between two marker kernels; the settle replays
    and capture launches around them (any number) are not counted."""
    steps = 4
    per_step = len(bench.LAYER_GROUPS) * len(bench.DECODE_MS)
    p = tmp_path / "trace.csv"
    sep = "void at::native::bitwise_not_kernel<signed char>(...)"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for _ in range(37 * per_step):                       # the step graphs, settled
            w.writerow([TILE, t, t + 999_000]); t += 1_000_000
        for j in range(per_step):                            # per launch
            for _ in range(steps * (3 + j)):                 # capture and settle replays
                w.writerow([TILE, t, t + 1]); t += 1_000_000
            w.writerow([sep, t, t + 3]); t += 1_000_000
            for _ in range(steps):                           # the timed replay
                w.writerow([TILE, t, t + 5000 * (j + 1)]); t += 1_000_000
                w.writerow([OTHER, t, t + 7]); t += 1_000_000
            w.writerow([sep, t, t + 3]); t += 1_000_000
        for _ in range(50):                                  # later legs
            w.writerow([TILE, t, t + 2]); t += 1_000_000
    out = bench.trace_summary(p)
    assert [(r["group"], r["m"]) for r in out] == [(g, m) for g, _ in bench.LAYER_GROUPS
                                                  for m in bench.DECODE_MS]
    for j, r in enumerate(out):
        assert r["dispatches"] == steps
        assert r["mean_us"] == pytest.approx(5.0 * (j + 1))


def test_phase_summary_reads_one_launch_of_stamps():
    """Two workgroups ran (the third slot row is zeros): five phases 4000
    cycles apart, products ending 3000-3007 cycles after each barrier; the
    29000 shader cycles from entry to exit span 1450 ticks of the 100 MHz
    clock, i.e. a 2000 MHz shader clock."""
    T = np.zeros((3, 8, bench.PHASE_SLOTS), dtype=np.int64)
    for g in range(2):
        T[g, :, 0] = 1000
        T[g, 0, 31] = 777
        for p in range(5):
            T[g, 0, 1 + p] = 2000 + 4000 * p
            T[g, :, 32 + p] = 5000 + 4000 * p + np.arange(8)
        T[g, 0, 62] = 777 + 1450
        T[g, 0, 63] = 30000
    d = bench.phase_summary(T)
    assert d["workgroups"] == 2 and d["phases"] == 5
    assert d["entry_to_first_barrier"] == 1000
    assert d["period"] == [4000.0] * 4
    assert d["products"] == [3007.0] * 5
    assert d["entry_to_exit"] == 29000
    assert d["sclk_mhz"] == 2000.0
    assert d["launch_span_us"] == 14.5 and d["entry_spread_us"] == 0.0
    assert d["workgroup_us_median"] == 14.5 and d["workgroup_us_max"] == 14.5


def test_merge_phase_summaries_takes_elementwise_medians():
    a = {"workgroups": 4, "phases": 2, "entry_to_first_barrier": 10.0, "period": [5.0],
         "products": [1.0, 2.0], "entry_to_exit": 100.0, "sclk_mhz": 2000.0}
    b = dict(a, entry_to_first_barrier=30.0, period=[7.0], products=[3.0, 6.0], sclk_mhz=None)
    c = dict(a, entry_to_first_barrier=20.0, period=[6.0], products=[2.0, 4.0], entry_to_exit=90.0)
    d = bench.merge_phase_summaries([a, b, c])
    assert d["entry_to_first_barrier"] == 20.0 and d["period"] == [6.0]
    assert d["products"] == [2.0, 4.0] and d["entry_to_exit"] == 100.0
    assert d["sclk_mhz"] is None and d["phases"] == 2 and d["workgroups"] == 4


def test_kernel_hash_follows_the_built_library(tmp_path, monkeypatch):
    """The hash that gates committed counters is the built libq4.so's."""
    pkg = tmp_path / "bit_block_quantized_q4_amd"
    pkg.mkdir()
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    assert bench.kernel_hash() == "unbuilt"
    (pkg / "libq4.so").write_bytes(b"\x7fELF one")
    h1 = bench.kernel_hash()
    (pkg / "libq4.so").write_bytes(b"\x7fELF two")
    assert bench.kernel_hash() != h1 and len(h1) == 16


def test_committed_summaries_gate_on_the_kernel_hash(tmp_path, monkeypatch):
    """A summary taken from other kernel sources is never reported."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(
        {"kernel_hash": "0" * 16, "kernels": {"x": {"traffic_bytes": 1.0}}}))
    (prof / "mfma.json").write_text(json.dumps(
        {"kernel_hash": "0" * 16, "kernels": {"y": {"MfmaUtil": 50.0}}}))
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    monkeypatch.setattr(bench, "kernel_hash", lambda: "1" * 16)
    assert bench.load_traffic("x") is None
    assert bench.load_mfma_util("y") is None
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.load_traffic("x") == {"traffic_bytes": 1.0}
    assert bench.load_mfma_util("y") == 50.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
