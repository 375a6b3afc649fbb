"""Host-side checks of bench.py: the byte and operation counts its roofline
uses, and the one-GPU contract of its command line (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_tile_pair_bytes_match_the_stored_format():
    # K4V2 at head_dim 128: K codes 128*128/2, V codes 128*128/4, K meta
    # (SK, ZK: D each, RK: 128) and V meta (SV, ZV: 128 each, CV: D) in fp16
    b = bench.per_tile_bytes(128)
    assert b["packed_pair"] == 8192 + 4096 + 2 * (2 * 128 + 128) + 2 * (256 + 128) == 13824
    assert b["fp16_pair"] == 2 * 2 * 128 * 128 == 65536
    # the 4.74x byte ratio of K4V2 against fp16
    assert abs(b["fp16_pair"] / b["packed_pair"] - 4.74) < 0.01


def test_quantiser_operation_count():
    # log2(D) butterflies + 3 per pass (2n passes for K, 2n - 1 for V) + 5 to quantise
    k = 7 + 3 * 10 + 5
    v = 7 + 3 * 9 + 5
    assert bench.quant_ops_per_elem(128, 5) == (k + v) / 2 == 40.5
    assert bench.quant_ops_per_elem(64, 3) == ((6 + 18 + 5) + (6 + 15 + 5)) / 2


def test_alu_peak_is_the_dual_issue_fp32_rate():
    # 256 CUs x 4 SIMDs x 32 lanes (two wave64 FMA/MUL/ADD per 4-cycle slot) x 2.4 GHz
    assert bench.VALU_PEAK == pytest.approx(78.6432e12)
    assert bench.HBM_PEAK == 8.0e12


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
