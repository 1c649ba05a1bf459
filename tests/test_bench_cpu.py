"""Host-side checks of the benchmark harness: the one-GPU guard, the roofline entry, the
committed rocprofv3 summaries it reads, and the CPU baseline timing of the oracle."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "exactly one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.parametrize("name", sorted(bench.WORKLOADS) + sorted(bench.LATENT_WORKLOADS))
def test_every_workload_has_a_profile_summary(name):
    # each bench workload's rocprofv3 summary records the kernel-source hash it was taken
    # on and the dominant stage's HBM bytes per launch, in the form bench.py parses
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    text = open(path).read()
    assert "rocprofv3 --kernel-trace --stats" in text and "--pmc FETCH_SIZE" in text
    assert "kernel source hash" in text
    assert "traffic bytes per launch:" in text
    if bench.kernel_source_hash() in text:
        assert bench.profiled_traffic(name) > 0


def test_roofline_entry_fields():
    r = {"gate_up_gbs": 6000.0, "gate_up_us": 29.4, "gate_up_alg_bytes": 176586752,
         "gate_up_tflops": 1200.0, "gate_up_flops": 1443109011456}
    e = bench.roofline_entry("decode_rep_m16", r)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["peak"] == 8000.0
    assert abs(e["frac"] - 0.75) < 1e-9
    e = bench.roofline_entry("prefill_rep_m8192", r)
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s" and abs(e["frac"] - 0.48) < 1e-9
