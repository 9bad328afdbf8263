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


def test_prefill_bytes_per_token():
    """Compulsory bytes per token at the 16/32-head, 128/128 shape with bf16
    inputs and fp32 out: prep reads q, k (2 x 16 x 128), v (32 x 128), a and
    b (2 x 32) bf16 values; the epilogue reads z (32 x 128 bf16) and writes
    out (32 x 128 fp32); the path is both."""
    b = bench.prefill_bytes_per_token(16, 32, 128, 128)
    assert b["prep"] == (2 * 16 * 128 + 32 * 128 + 2 * 32) * 2 == 16_512
    assert b["epi"] == 32 * 128 * (2 + 4) == 24_576
    assert b["path"] == 41_088


def test_binding_roofline_takes_the_larger_ceiling():
    # 1 GFLOP and 8 MB in 1 ms: the matrix cores need 0.4 us, HBM 1 us
    r = bench.binding_roofline(1e9, 8e6, 1e-3)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(8.0) and r["frac"] == pytest.approx(1e-3)
    assert r["ceiling_ms"] == pytest.approx(1e-3)
    # 100 GFLOP and 8 MB in 1 ms: the matrix cores need 40 us
    r = bench.binding_roofline(1e11, 8e6, 1e-3)
    assert r["bound"] == "mfma" and r["achieved"] == pytest.approx(100.0)
    assert r["frac"] == pytest.approx(0.04)
