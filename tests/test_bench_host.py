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
    (bf16), g and beta, w (2 bytes) and u (3 bytes) per value; stage 2 per
    token: q and k, w, u, g and o (fp32), plus the final states."""
    wl = workloads.make(1)
    work = bench.algorithmic_work(wl, 64, 2)
    T, H, Hv, D = 4096, 16, 32, 128
    s1 = T * (H * D * 2 + Hv * D * 2 + Hv * 4 + Hv * 4 + Hv * D * 2 + Hv * D * 3)
    s2 = T * (2 * H * D * 2 + Hv * D * 2 + Hv * D * 3 + Hv * 4 + Hv * D * 4) + Hv * D * D * 4
    assert work["intra"][0] == s1 == 135_266_304
    assert work["inter"][0] == s2 == 187_170_816
    assert work["inter"][1] == 64 * Hv * (3 * 2 * 64 * D * D + 2 * 2 * 64 * 64 * D)
    assert work["intra"][1] == 5_539_364_864


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
