"""Host-side analysis modes of bench.py on small synthetic counter files (CPU).

`--clock-from` turns one rocprofv3 --pmc pass (GRBM_GUI_ACTIVE and
SQ_VALU_MFMA_BUSY_CYCLES per dispatch) into a per-kernel clock and MFMA busy
fraction; `--traffic-from` turns a FETCH_SIZE and a WRITE_SIZE pass into
bytes per launch, scaled by the calibration copy.  The files here are written
by hand with known values.
"""
import csv
import importlib.util
import json
import os
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(tmp_path, dispatches):
    with open(tmp_path / "c_agent_info.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Node_Id", "Name", "Num_Xcc", "Simd_Count", "Cu_Count"])
        w.writerow(["0", "cpu", "0", "0", "0"])
        w.writerow(["1", "gfx950", "8", "1024", "256"])
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(tmp_path / "c_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(hdr)
        for i, (name, ns, ghz, busy) in enumerate(dispatches):
            cycles = ghz * ns                      # per XCD
            start = 1_000_000 * (i + 1)
            w.writerow([i, name, "GRBM_GUI_ACTIVE", 8 * cycles, start, start + ns])
            w.writerow([i, name, "SQ_VALU_MFMA_BUSY_CYCLES", busy * cycles * 1024, start, start + ns])


def test_clock_report_recovers_clock_and_busy(tmp_path, capsys):
    nt = "void muon::(anonymous namespace)::k_nt<256, 256, 2, 4, unsigned short, false>(muon::GemmParams)"
    ew = "muon::(anonymous namespace)::k_ew_momentum(muon::EwMat const*, float*)"
    _write(tmp_path, [
        (nt, 2_000_000, 1.6, 0.5),
        (nt, 2_000_000, 1.8, 0.7),
        (nt, 100_000, 3.0, 0.1),          # shorter than 200 us: left out
        (ew, 1_000_000, 2.4, 0.0),
    ])
    _bench().clock_report(str(tmp_path))
    out = json.loads(capsys.readouterr().out)
    assert out["xcds"] == 8 and out["simds"] == 1024
    by = {k["kernel"]: k for k in out["kernels"]}
    k = by["k_nt<256, 256, 2, 4, unsigned short, false>"]
    assert k["dispatches"] == 2
    assert k["clock_ghz"] == pytest.approx(1.7, abs=1e-3)
    assert k["clock_range"] == pytest.approx([1.6, 1.8], abs=1e-3)
    assert k["mfma_busy"] == pytest.approx(0.6, abs=1e-3)
    # the MFMA pipes issue peak * (clock / 2.4 GHz) * busy
    assert k["bf16_mfma_tflops_issued"] == pytest.approx(2500 * 1.7 / 2.4 * 0.6, abs=0.2)
    e = by["k_ew_momentum"]
    assert e["clock_ghz"] == pytest.approx(2.4, abs=1e-3) and e["mfma_busy"] == 0.0
    # the longest total time comes first
    assert out["kernels"][0]["kernel"].startswith("k_nt<256")


def test_clock_report_without_counters_fails(tmp_path):
    with pytest.raises(SystemExit):
        _bench().clock_report(str(tmp_path))


NT256 = "void muon::(anonymous namespace)::k_nt<256, 256, 2, 4, unsigned short, false>(muon::GemmParams)"
NT256QT = "void muon::(anonymous namespace)::k_nt<256, 256, 2, 4, unsigned short, true>(muon::GemmParams)"
NT128F = "void muon::(anonymous namespace)::k_nt<128, 128, 2, 2, float, false>(muon::GemmParams)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>(int)"


def test_kernel_labels_match_profiler_names():
    b = _bench()
    assert b.demangled("k_nt<256,256,bf16>").search(NT256)
    assert not b.demangled("k_nt<256,256,bf16>").search(NT256QT)
    assert b.demangled("k_nt<256,256,bf16,qt>").search(NT256QT)
    assert b.demangled("k_nt<128,128,f32>").search(NT128F)
    assert not b.demangled("k_nt<128,128,bf16>").search(NT128F)
    assert b.demangled("k_ew_momentum").search("muon::(anonymous namespace)::k_ew_momentum(muon::EwMat const*)")


def _pmc(dirpath, counter, rows):
    dirpath.mkdir()
    with open(dirpath / "x_counter_collection.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, kib) in enumerate(rows):
            w.writerow([i, name, counter, kib])


def test_traffic_record_scales_by_the_calibration_copy(tmp_path, capsys):
    b = _bench()
    gib_kib = (1 << 30) / 1024
    # warmup 1 + 2 steps, 2 launches per step; the copy reads twice its size
    # (the fetch counter's factor is then 1/2) and writes exactly its size
    fetch = [(NT256, 1000.0), (NT256, 3000.0)] * 3 + [(NT256QT, 9e9), (COPY, 2 * gib_kib)]
    write = [(NT256, 500.0)] * 6 + [(COPY, gib_kib)]
    _pmc(tmp_path / "f", "FETCH_SIZE", fetch)
    _pmc(tmp_path / "w", "WRITE_SIZE", write)
    args = types.SimpleNamespace(kernel="k_nt<256,256,bf16>", warmup=1,
                                 traffic_from=[str(tmp_path / "f"), str(tmp_path / "w")])
    wl = types.SimpleNamespace(name="synthetic set")
    out = tmp_path / "traffic.json"
    b.write_traffic(args, wl, path=str(out))
    rec = json.loads(out.read_text())["entries"]
    assert len(rec) == 1
    e = rec[0]
    assert e["launches_per_step"] == 2
    assert e["fetch_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 0.5)
    assert e["write_bytes_per_launch"] == pytest.approx(500.0 * 1024)
    assert e["source"] == b.source_digest() and e["workload"] == "synthetic set"
    # a second record for the same kernel and workload replaces the first
    b.write_traffic(args, wl, path=str(out))
    assert len(json.loads(out.read_text())["entries"]) == 1
    # dispatch counts that do not fit warmup + 2 steps are refused
    args.warmup = 2
    with pytest.raises(SystemExit):
        b.write_traffic(args, wl, path=str(out))
