"""The one-token down kernel's per-slot record (slot_record.h), packed and
unpacked on the host: offsets of either sign (a tiered expert's rows can lie
below the routed base pointer), every staged-pair index a record can hold,
the shared flag and the weight bits.  Built with hipcc as host code."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_records_round_trip(tmp_path):
    exe = str(tmp_path / "slot_record_check")
    src = os.path.join(ROOT, "tests", "slot_record_check.cpp")
    inc = os.path.join(ROOT, "quantized_moe_noaux_amd", "csrc")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", inc, src, "-o", exe],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout
    assert r.stdout.startswith("432 of 432 records round-trip")
