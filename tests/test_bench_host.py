"""bench.py's host-side logic, without a GPU: attribution of rocprofv3 counter
rows to workloads, the copy-kernel scaling of FETCH_SIZE / WRITE_SIZE, the
wave-state ratios, the source-hash gate on committed summaries, and the
refusal of more than one GPU."""

import csv
import json
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
import synth  # noqa: E402

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


def traffic_rows(counter, gemv_vals, calib, quant, gemm):
    """A traffic pass as traffic_run launches it: the copy, then per batch size
    (in WORKLOADS[2].ms order) its GEMV dispatches, then the quantiser and the
    GEMM, with unrelated kernels in between."""
    rows, did = [], 1
    rows.append((did, OTHER, {counter: 9e9})); did += 1
    rows.append((did, NEG, {counter: calib})); did += 1
    for v in gemv_vals:
        rows.append((did, GEMV if v < 3000 else TILE, {counter: v})); did += 1
    rows.append((did, QUANT, {counter: quant})); did += 1
    rows.append((did, GEMM, {counter: gemm})); did += 1
    return rows


def test_traffic_summary_attributes_and_scales(tmp_path):
    ms = list(synth.WORKLOADS[2].ms)
    per = 3
    # each batch size's dispatches share a value; medians must pick them out
    gemv_f = [1000.0 * (i + 1) for i in range(len(ms)) for _ in range(per)]
    gemv_w = [10.0 * (i + 1) for i in range(len(ms)) for _ in range(per)]
    calib_kib = bench.TRAFFIC_CALIB_BYTES / 1024.0 * 1.25   # counter reads 25% high
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fcsv, traffic_rows("FETCH_SIZE", gemv_f, calib_kib, 500.0, 7000.0))
    write_csv(wcsv, traffic_rows("WRITE_SIZE", gemv_w, bench.TRAFFIC_CALIB_BYTES / 1024.0, 50.0, 70.0))
    out = tmp_path / "traffic.json"
    d = bench.traffic_summary(fcsv, wcsv, out)
    assert json.loads(out.read_text()) == d
    assert d["source_hash"] == bench.kernel_source_hash()
    assert d["calibration"]["fetch_scale"] == pytest.approx(0.8)
    assert d["calibration"]["write_scale"] == pytest.approx(1.0)
    k = d["kernels"]
    assert set(k) == {f"gemv_5120x5120_m{m}" for m in ms} | {"quantize_fp32_5120x5120",
                                                             "gemm_2048x17408x5120"}
    for i, m in enumerate(ms):
        e = k[f"gemv_5120x5120_m{m}"]
        assert e["dispatches"] == per
        assert e["fetch_bytes"] == pytest.approx(1000.0 * (i + 1) * 1024 * 0.8)
        assert e["write_bytes"] == pytest.approx(10.0 * (i + 1) * 1024)
        assert e["traffic_bytes"] == pytest.approx(e["fetch_bytes"] + e["write_bytes"])
    assert k["quantize_fp32_5120x5120"]["fetch_bytes"] == pytest.approx(500.0 * 1024 * 0.8)


def test_sq_summary_ratios(tmp_path):
    ms = list(synth.WORKLOADS[2].ms)
    rows, did = [], 1
    for i, m in enumerate(ms):
        for _ in range(2):
            rows.append((did, GEMV, {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 600.0 + i,
                                     "SQ_WAIT_INST_ANY": 100.0, "SQ_ACTIVE_INST_LDS": 50.0,
                                     "SQ_LDS_BANK_CONFLICT": 25.0 * (i + 1)}))
            did += 1
    rows.append((did, QUANT, {"SQ_WAVE_CYCLES": 400.0, "SQ_WAIT_ANY": 100.0,
                              "SQ_WAIT_INST_ANY": 50.0, "SQ_ACTIVE_INST_LDS": 0.0,
                              "SQ_LDS_BANK_CONFLICT": 0.0}))
    p = tmp_path / "sq.csv"
    write_csv(p, rows)
    d = bench.sq_summary(p, tmp_path / "sq.json")
    k = d["kernels"]
    for i, m in enumerate(ms):
        e = k[f"gemv_5120x5120_m{m}"]
        assert e["dispatches"] == 2
        assert e["wait_any_per_wave_cycle"] == pytest.approx((600.0 + i) / 1000.0)
        assert e["wait_inst_per_wave_cycle"] == pytest.approx(0.1)
        assert e["lds_conflict_per_lds_active"] == pytest.approx(0.5 * (i + 1))
    assert k["quantize_fp32_5120x5120"]["lds_conflict_per_lds_active"] is None
    assert k["quantize_fp32_5120x5120"]["wait_any_per_wave_cycle"] == pytest.approx(0.25)


def test_committed_summaries_gate_on_the_source_hash(tmp_path, monkeypatch):
    """A summary taken from other kernel sources is never reported."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic.json").write_text(json.dumps(
        {"source_hash": "0" * 16, "kernels": {"x": {"traffic_bytes": 1.0}}}))
    (prof / "mfma.json").write_text(json.dumps(
        {"source_hash": "0" * 16, "kernels": {"y": {"MfmaUtil": 50.0}}}))
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "1" * 16)
    assert bench.load_traffic("x") is None
    assert bench.load_mfma_util("y") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("x") == {"traffic_bytes": 1.0}
    assert bench.load_mfma_util("y") == 50.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
