"""The measurement harness on the CPU: the one-GPU rule, the rocprofv3
counter arithmetic that turns FETCH_SIZE / WRITE_SIZE into HBM-side bytes
per launch (calibrated against a plain copy of known size), and the
refusal of a counter file that holds no dispatch of the kernel asked for."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def write_counters(d, counter, rows):
    """rows: (kernel name, dispatch id, value in KiB); one CSV as rocprofv3 writes it."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for name, di, v in rows:
            w.writerow([di, name, counter, v])


def test_traffic_arithmetic(bench, tmp_path, monkeypatch):
    # a 1 GiB copy that reads 2^19 KiB of FETCH_SIZE (2 bytes per counted
    # byte) and writes 2^20 KiB of WRITE_SIZE (1 byte per counted byte)
    kname = "void moe::k_gate_up_sw<4, 1, 1, 1, false>(moe::GemvArgs, moe::ChunkCfg, moe::PlanDims)"
    write_counters(str(tmp_path / "cf"), "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1, 2 ** 19)])
    write_counters(str(tmp_path / "cw"), "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1, 2 ** 20)])
    # the kernel: two dispatches of 1000 and 3000 KiB fetched (mean 2000), 10 KiB written, plus other kernels
    write_counters(str(tmp_path / "kf"), "FETCH_SIZE", [(kname, 5, 1000.0), (kname, 9, 3000.0),
                                                        ("moe::k_router_logits_small(...)", 4, 77.0)])
    write_counters(str(tmp_path / "kw"), "WRITE_SIZE", [(kname, 5, 10.0), (kname, 9, 10.0)])
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda path: "h")
    args = bench.argparse.Namespace(workload="decode_int4", kernel="gate_up_swiglu_quant",
                                    pmc_fetch=str(tmp_path / "kf"), pmc_write=str(tmp_path / "kw"),
                                    copy_fetch=str(tmp_path / "cf"), copy_write=str(tmp_path / "cw"),
                                    commands=["c1"])
    bench.write_traffic(args)
    d = json.load(open(out / "traffic_decode_int4.json"))
    assert d["fetch_size"]["dispatches"] == 2 and d["fetch_size"]["kib_per_dispatch"] == 2000.0
    assert d["fetch_size"]["bytes_per_counted_byte"] == pytest.approx(2.0)
    assert d["write_size"]["bytes_per_counted_byte"] == pytest.approx(1.0)
    assert d["hbm_bytes_per_launch"] == pytest.approx(2000 * 1024 * 2.0 + 10 * 1024 * 1.0)
    assert bench.traffic_from_profiles("decode_int4", "gate_up_swiglu_quant") == d["hbm_bytes_per_launch"]
    # a stale source hash or another kernel gives no figure
    monkeypatch.setattr(bench, "kernel_source_hash", lambda path: "other")
    assert bench.traffic_from_profiles("decode_int4", "gate_up_swiglu_quant") is None


def test_missing_kernel_is_refused(bench, tmp_path, monkeypatch):
    write_counters(str(tmp_path / "k"), "FETCH_SIZE", [("moe::k_router_logits_small(...)", 1, 5.0)])
    write_counters(str(tmp_path / "c"), "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1, 2 ** 19)])
    write_counters(str(tmp_path / "w"), "WRITE_SIZE", [("moe::k_router_logits_small(...)", 1, 5.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda path: "h")
    args = bench.argparse.Namespace(workload="decode_int4", kernel="gate_up_swiglu_quant",
                                    pmc_fetch=str(tmp_path / "k"), pmc_write=str(tmp_path / "w"),
                                    copy_fetch=str(tmp_path / "c"), copy_write=str(tmp_path / "c"), commands=[])
    with pytest.raises(SystemExit):
        bench.write_traffic(args)
