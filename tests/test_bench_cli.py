"""The bench script's contract on the CPU (no GPU needed): the multi-GPU refusal, the algorithmic
byte counts it prices the kernels with, and that the committed HBM-traffic summary was taken on the
GEMM source as it stands (otherwise the bench line's roofline.traffic would silently be null)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert not r.stdout.strip().startswith("{"), "no bench line may be printed for N > 1"


def test_algorithmic_bytes():
    # W4A16 adaLN projection: codes K N / 2, bf16 scales (K / 64) N, bf16 X and Y
    assert bench.awq_bytes(16, 3072, 18432) == 3072 * 18432 // 2 + 48 * 18432 * 2 + 16 * 3072 * 2 + 16 * 18432 * 2
    assert bench.awq_bytes(16, 3072, 18432) == 30769152
    # the up projection's quantizer (X, codes, scales, T, L1, smoothing) and GEMM (codes, scales, T, L2,
    # bias, Y): the 36.78 MB and 143.55 MB the kernels' HBM fractions and traffic ratios are priced on
    assert round(bench.quant_bytes(4608, 3072, 32) / 1e6, 2) == 36.78
    assert round(bench.gemm_bytes(4608, 3072, 12288, 32) / 1e6, 2) == 143.55


def test_committed_gemm_traffic_matches_the_gemm_source():
    t = bench.load_traffic("w4a4_gemm.hip", "up")
    assert t is not None, "profiles/traffic.txt was not taken on the current GEMM source"
    # the GEMM writes Y (113.25 MB) and reads at least its algorithmic inputs
    assert 143.5e6 < t < 400e6
