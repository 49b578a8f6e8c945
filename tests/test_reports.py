"""The benchmark's error report (per-block error, signed errors, SQNR,
flush-to-zero rate) on a hand-worked example, CPU only.

Row 1 holds the only nonzero block (16 elements, block scale 1):
  x    = [1, -1, 3, -3, 0.2, 0, ...],  xhat = [0.5, -1.5, 3, -2, 0, 0, ...]
  err  = xhat - x = [-0.5, -0.5, 0, 1, -0.2, 0, ...]
Row 0 is all zeros with block scale 0 (a block coded as zeros).  By hand,
over the 32 elements:
  mean(sign(x) * err) = (-0.5 + 0.5 + 0 - 1 - 0.2) / 32 = -1.2 / 32
  mean(err)           = (-0.5 - 0.5 + 1 - 0.2) / 32     = -0.2 / 32
  gain  = <xhat, x> / <x, x> = (0.5 + 1.5 + 9 + 6) / (1 + 1 + 9 + 9 + 0.04) = 17 / 20.04
  SQNR  = 10 log10(20.04 / (0.25 + 0.25 + 1 + 0.04)) = 10 log10(20.04 / 1.54)
  flush to zero: 1 of the 5 nonzero inputs (0.2) codes as zero = 0.2
  normalized magnitude bias over the one block with d_b > 0:
        mean(|xhat| - |x|) = (-0.5 + 0.5 + 0 - 1 - 0.2) / 16 = -1.2 / 16
  per block: MSE [0, 1.54 / 16], max |err| [0, 1], signed magnitude mean
        [0, -1.2 / 16]; the worst block is block 1, in row 1.
"""
import math

import torch

import bench


def test_error_report_hand_worked():
    x = torch.zeros(2, 16, dtype=torch.float64)
    xhat = torch.zeros(2, 16, dtype=torch.float64)
    x[1, :5] = torch.tensor([1.0, -1.0, 3.0, -3.0, 0.2], dtype=torch.float64)
    xhat[1, :5] = torch.tensor([0.5, -1.5, 3.0, -2.0, 0.0], dtype=torch.float64)
    d_b = torch.zeros(2, 16, dtype=torch.float64)
    d_b[1] = 1.0
    r = bench.error_report(x, x, xhat, xhat, d_b, 16)
    close = lambda a, b: math.isclose(a, b, rel_tol=1e-12, abs_tol=1e-15)
    assert close(r["mean_signed_error_magnitude"], -1.2 / 32)
    assert close(r["mean_error"], -0.2 / 32)
    assert close(r["gain"], 17.0 / 20.04)
    assert close(r["sqnr_db"], 10.0 * math.log10(20.04 / 1.54))
    assert math.isclose(r["flush_to_zero_rate"], 0.2, rel_tol=1e-6)  # a binary32 ratio
    assert close(r["normalized_magnitude_bias"], -1.2 / 16)
    mse = r["per_block_mse"]
    assert math.isclose(mse["max"], 1.54 / 16, rel_tol=1e-6)
    assert math.isclose(mse["p50"], 1.54 / 32, rel_tol=1e-6)  # halfway between the two blocks
    assert math.isclose(r["per_block_max_abs_error"]["max"], 1.0, rel_tol=1e-6)
    assert math.isclose(r["per_block_signed_magnitude_mean"]["p50"], -1.2 / 32, rel_tol=1e-6)
    assert r["worst_block_mse"]["block"] == 1 and r["worst_block_mse"]["row"] == 1


def test_error_report_exact_codes():
    """Values already on the grid: no error, infinite SQNR, gain 1."""
    x = torch.tensor([[0.5, -1.0, 1.5, -2.0, 3.0, -4.0, 6.0, 0.0] * 2], dtype=torch.float64)
    d_b = torch.ones_like(x)
    r = bench.error_report(x, x, x, x, d_b, 16)
    assert r["mean_signed_error_magnitude"] == 0.0 and r["mean_error"] == 0.0
    assert r["gain"] == 1.0 and math.isinf(r["sqnr_db"])
    assert r["flush_to_zero_rate"] == 0.0 and r["normalized_magnitude_bias"] == 0.0
