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
    """bench.py takes its byte counts from the library's layout query; they
    must equal the oracle's own format sizes, and at K4V2, head_dim 128 the
    13 824 B per tile pair (0.211x of fp16: the pages' 'under a quarter')."""
    import oracle
    for D in (64, 128, 256):
        for kb, vb in ((4, 2), (4, 4), (2, 2), (2, 4)):
            b = bench.per_tile_bytes(D, kb, vb)
            want = (oracle.code_bytes(D, kb) + oracle.code_bytes(D, vb)
                    + 2 * oracle.meta_halves(D, True) + 2 * oracle.meta_halves(D, False))
            assert b["packed_pair"] == want, (D, kb, vb)
    b = bench.per_tile_bytes(128)
    assert b["packed_pair"] == 13824 and b["fp16_pair"] == 65536
    assert bench.per_tile_bytes(64)["packed_pair"] == 7296
    assert bench.per_tile_bytes(256)["packed_pair"] == 26880


def test_quantiser_operation_count():
    # worked by hand from the count stated in bench.quant_ops_per_elem:
    # D 128, 5 it: K 7 + 30 + 5 = 42, V 7 + 27 + 5 = 39 -> 40.5
    # D 64, 3 it:  K 6 + 18 + 5 = 29, V 6 + 15 + 5 = 26 -> 27.5
    # D 256, 5 it: K 8 + 30 + 5 = 43, V 8 + 27 + 5 = 40 -> 41.5
    assert bench.quant_ops_per_elem(128, 5) == 40.5
    assert bench.quant_ops_per_elem(64, 3) == 27.5
    assert bench.quant_ops_per_elem(256, 5) == 41.5


def test_alu_peak_is_the_dual_issue_fp32_rate():
    # 256 CUs x 4 SIMDs x 32 lanes (two wave64 FMA/MUL/ADD per 4-cycle slot) x 2.4 GHz
    assert bench.VALU_PEAK == pytest.approx(78.6432e12)
    assert bench.HBM_PEAK == 8.0e12


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
