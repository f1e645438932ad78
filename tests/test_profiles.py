"""The committed rocprofv3 summaries under profiles/ are consistent: every
counter summary has the machine-read lines bench.py takes, its HBM bytes per
launch follow from the two counters and the copy calibration, and every
workload the bench runs has a kernel trace and a counter summary."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
WORKLOADS = ["gqa_int8", "int4_asym", "paged_mixed", "asym_kv", "int2_super", "int2_group",
             "int4_tiered"]


def fields(path):
    out = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^([a-z_]+): `?([0-9a-f.]+)`?\s*$", line)
            if m:
                out[m.group(1)] = m.group(2)
    return out


@pytest.mark.parametrize("workload", WORKLOADS)
def test_counter_summary_consistent(workload):
    f = fields(os.path.join(PROFILES, f"decode_split_{workload}_counters.md"))
    for key in ("source_sha", "fetch_kib_per_dispatch", "write_kib_per_dispatch",
                "copy_fetch_factor", "copy_write_factor", "hbm_bytes_per_launch",
                "algorithmic_bytes_per_launch"):
        assert key in f, f"{workload}: {key} missing"
    hbm = (float(f["fetch_kib_per_dispatch"]) * float(f["copy_fetch_factor"])
           + float(f["write_kib_per_dispatch"]) * float(f["copy_write_factor"])) * 1024
    # the summary rounds the KiB figures to 0.1 and the factors to 1e-4
    assert abs(hbm - int(f["hbm_bytes_per_launch"])) <= 2e-4 * hbm
    ratio = int(f["hbm_bytes_per_launch"]) / int(f["algorithmic_bytes_per_launch"])
    assert 1.0 <= ratio < 1.1, f"{workload}: traffic {ratio:.3f} x the algorithmic bytes"


@pytest.mark.parametrize("workload", WORKLOADS)
def test_trace_summary_matches_counters(workload):
    trace = os.path.join(PROFILES, f"decode_split_{workload}_kernel_trace.md")
    with open(trace) as f:
        text = f.read()
    assert "rocprofv3 --kernel-trace --stats" in text
    sha = re.search(r"Kernel sources: `([0-9a-f]+)`", text).group(1)
    f = fields(os.path.join(PROFILES, f"decode_split_{workload}_counters.md"))
    assert sha == f["source_sha"], f"{workload}: trace and counters taken at different sources"
