"""The measurement harness on the CPU: the one-GPU rule, the rocprofv3
counter arithmetic that turns FETCH_SIZE / WRITE_SIZE into HBM-side bytes
per launch (calibrated against a plain copy of known size), and the
refusal of a counter file that holds no dispatch of the kernel asked for,
and the default run's records of the other workloads."""
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


def test_secondary_records(bench, monkeypatch):
    """The default run's child runs: a child's last JSON line becomes its
    record; a failed or timed-out child leaves an error entry, and every
    workload of SECONDARY is run once with the defaults."""
    calls = []

    def fake_run(cmd, stdout=None, text=None, timeout=None):
        w = cmd[cmd.index("--workload") + 1]
        calls.append(cmd)
        assert "--no-secondary" in cmd and "--no-cpu-baseline" in cmd and timeout == bench.SECONDARY_TIMEOUT_S
        if w == "stack_int2":
            raise subprocess.TimeoutExpired(cmd, timeout)
        if w == "verify_int8":
            return subprocess.CompletedProcess(cmd, 1, stdout="", stderr=None)
        line = {"value": 2.0, "unit": "tokens/s", "ms_per_step": 0.5, "steps": 3, "warmup": 1,
                "higher_is_better": True, "dtype": "i8", "config": {"workload": w},
                "roofline": {"bound": "hbm", "kernel": "k", "achieved": 1.0, "peak": 8.0, "unit": "GB/s",
                             "frac": 0.125, "traffic": None, "extra": 7},
                "detail": {"stage_us": {"a": 1.0}, "other": 3}}
        return subprocess.CompletedProcess(cmd, 0, stdout="progress\n" + json.dumps(line) + "\n", stderr=None)

    monkeypatch.setattr(subprocess, "run", fake_run)
    res = bench.run_secondary()
    assert [c[c.index("--workload") + 1] for c in calls] == bench.SECONDARY
    assert set(res) == set(bench.SECONDARY)
    assert "timed out" in res["stack_int2"]["error"]
    assert res["verify_int8"]["error"] == "exit status 1"
    r = res["prefill_int4"]
    assert r["value"] == 2.0 and r["config"] == {"workload": "prefill_int4"} and r["stage_us"] == {"a": 1.0}
    assert r["roofline"]["frac"] == 0.125 and "extra" not in r["roofline"] and "other" not in r
