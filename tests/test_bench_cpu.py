"""Host-side checks of bench.py: the one-GPU guard and the rule that counter
traffic is reported only for the workload and kernel variant it was taken on,
and only while the GEMM sources are unchanged."""

import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _fields(path):
    out = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_traffic_only_for_profiled_variant_and_current_sources():
    h = hashlib.sha256()
    for f in ("kernels_gemm.hip", "mx_device.h", "internal.h", "topk_device.h"):
        h.update(open(os.path.join(ROOT, "mxfp4_expert_grouped_amd", "csrc", f), "rb").read())
    current = h.hexdigest()
    prof = os.path.join(ROOT, "profiles")
    names = [f[len("gate_up_"):-len("_hbm_traffic.txt")] for f in os.listdir(prof)
             if f.startswith("gate_up_") and f.endswith("_hbm_traffic.txt")]
    assert "decode256" in names
    for n in names:
        f = _fields(os.path.join(prof, f"gate_up_{n}_hbm_traffic.txt"))
        got = bench.profiled_traffic(n)
        if f["source_sha256"] == current:
            assert got == int(f["traffic_bytes_per_launch"])
        else:
            assert got is None
    # a variant with no summary of its own reports nothing
    assert bench.profiled_traffic("decode256_canonical") is None
    assert bench.profiled_traffic("no_such_workload") is None
