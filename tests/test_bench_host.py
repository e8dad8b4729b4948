"""Host-side logic of bench.py (no GPU): the algorithmic work it prices the
roofline with, and the one-GPU guard."""
import subprocess
import sys
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import configs  # noqa: E402


def test_gemm_work_bf16_by_hand():
    cfg = configs.MIXTRAL
    counts = [3, 0, 5, 0, 0, 0, 0, 2]
    f1, b1 = bench.gemm_work(cfg, counts, 1)
    H, I = 4096, 14336
    assert f1 == 2.0 * 10 * (2 * I) * H
    # three touched experts' w1, 10 rows of x_perm read, 10 rows of h written
    assert b1 == 3 * (2 * I) * H * 2 + 10 * H * 2 + 10 * I * 2
    f2, b2 = bench.gemm_work(cfg, counts, 2)
    assert f2 == 2.0 * 10 * H * I
    assert b2 == 3 * H * I * 2 + 10 * I * 2 + 10 * H * 2


def test_gemm_work_mxfp4_counts_packed_bytes_and_scales():
    cfg = configs.DEEPSEEK_MXFP4
    counts = np.zeros(256, dtype=np.int32)
    counts[[0, 7]] = [64, 1]
    _, b1 = bench.gemm_work(cfg, counts, 1)
    H, I = 7168, 2048
    assert b1 == 2 * (2 * I) * (H // 2 + H // 32) + 65 * H * 2 + 65 * I * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
