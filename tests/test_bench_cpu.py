"""Host-side checks of bench.py's roofline arithmetic and its one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_exp_issue_bound_and_issue_floors():
    exp = bench.N_CU * bench.CLOCK_HZ * bench.EXP_LANES_PER_CLK_CU
    assert exp == pytest.approx(19.6608e12)
    # the matrix-core d = 3 path is rated against the exp issue bound ...
    peak, bound, _, algo = bench.roofline_evals_per_s(3, "lse3m_kernel")
    assert peak == exp and bound == "alu"
    # ... and the metric's min(FP32 / 9 flops, exp) stays reported beside it
    assert algo == pytest.approx(min(157.3e12 / 9, exp))
    # bf16 features: MFMA 2.5 PFLOP/s over 2d flops, just below the exp bound at d = 64
    peak, bound, _, _ = bench.roofline_evals_per_s(64, "lseFs_kernel")
    assert bound == "mfma" and peak == pytest.approx(2.5e15 / 128)
    # each kernel's issue floor (its measured tile mix) is below the exp bound; the
    # d = 3 tile costs 220 SIMD cycles per 1024 entries, the d = 64 feature tile 314
    for k in bench.TILE_CYCLES:
        assert bench.issue_floor_evals_per_s(k) < exp
    assert bench.issue_floor_evals_per_s("lse3m_kernel") == pytest.approx(
        1024 * 2.4e9 * 1024 / 220)
    assert bench.issue_floor_evals_per_s("lseFs_kernel") == pytest.approx(
        1024 * 2.4e9 * 1024 / 314)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
