"""Host-side checks of bench.py (no GPU): the algorithmic byte and flop model
on the headline workload, and the one-GPU guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_algorithmic_work_headline_workload():
    """T = 4096, H = 16, Hv = 32, bf16, 64 chunks. Stage 1 per token: k and v
    (bf16), g and beta, w (2 bytes) and u (4 bytes, fp32) per value; stage 2
    per token: q and k, w, u, g and o (fp32), plus the final states. These
    are the per-stage byte figures of the scope table's measurement model
    (152,043,520 and 203,948,032 bytes). With u as stored here (3 bytes), the
    smaller stored-byte figures."""
    wl = workloads.make(1)
    T, H, Hv, D = 4096, 16, 32, 128
    for u, s1_want, s2_want in ((4, 152_043_520, 203_948_032), (3, 135_266_304, 187_170_816)):
        work = bench.algorithmic_work(wl, 64, 2, u_bytes=u)
        s1 = T * (H * D * 2 + Hv * D * 2 + Hv * 4 + Hv * 4 + Hv * D * 2 + Hv * D * u)
        s2 = T * (2 * H * D * 2 + Hv * D * 2 + Hv * D * u + Hv * 4 + Hv * D * 4) + Hv * D * D * 4
        assert work["intra"][0] == s1 == s1_want
        assert work["inter"][0] == s2 == s2_want
    assert bench.algorithmic_work(wl, 64, 2)["inter"][0] == 203_948_032  # default: u at 4 bytes
    assert work["inter"][1] == 64 * Hv * (3 * 2 * 64 * D * D + 2 * 2 * 64 * 64 * D)
    assert work["intra"][1] == 5_539_364_864


def test_cpu_baseline_reports_all_cores_and_one_thread():
    """The CPU baseline leg on a small workload: the oracle's own thread count
    and a one-thread figure, both positive, the front workload included."""
    wl = workloads.make_custom([300, 200], 2, 4, seed=3)
    r = bench.cpu_baseline(wl, max_seconds=0.3, min_seconds=0.1, one_thread_seconds=0.2)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["value"] > 0
    assert r["one_thread"]["cores"] == 1 and r["one_thread"]["value"] > 0
    wf = workloads.make_custom([200, 200], 2, 4, seed=4, front=True)
    rf = bench.cpu_baseline(wf, max_seconds=0.3, min_seconds=0.1, one_thread_seconds=0.2)
    assert rf["value"] > 0 and "front" in rf["sample"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
