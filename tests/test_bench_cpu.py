"""bench.py's host-side contract: the one-GPU refusal and the algorithmic
work counts its roofline figures divide by (no device needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and r.stdout == ""


def test_prefill_flops_per_token():
    """Hk = 16, Hv = 32, dk = dv = 128, C = 64: the scan's W H, Q H and
    K_d^T U (2 dk dv each) plus P U ((C + 1) dv) per value head, and the
    prep's Grams per key head, triangular solve and W, U~ per value head:
    3.41 + 0.84 = 4.25 MFLOP per token."""
    scan, prep = bench.prefill_flops_per_token(16, 32, 128, 128, 64)
    assert scan == 32 * (6 * 128 * 128 + 65 * 128) == 3_411_968
    assert prep == pytest.approx(16 * (63 + 65) * 128 + 32 * (64 * 64 / 3 + 65 * 256))
    assert (scan + prep) / 1e6 == pytest.approx(4.2496, abs=1e-3)


def test_decode_bytes_per_sequence():
    """One decode step of one sequence and layer: the fp32 state read and
    written (2 x 2 MiB), the bf16 conv state read and written (2 x 3 x 8192
    x 2 B), the bf16 token inputs and the fp32 output."""
    total, state = bench.decode_bytes_per_seq(16, 32, 128, 128)
    assert state == 2 * 32 * 128 * 128 * 4 == 4_194_304
    assert total == state + 2 * 3 * 8192 * 2 + (2 * 2048 + 2 * 4096 + 64) * 2 + 4096 * 4
    assert total == 4_333_696
