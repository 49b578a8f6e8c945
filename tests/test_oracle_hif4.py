"""Pins for the oracle's HiF4 format (CPU only).

The HiFloat page ("Unleashing Low-Bit Inference on Ascend NPUs ...", 2.
Metodologia) gives HiF4's structure -- an E6M2 scale per 64 elements, E1M0
scales per 8 and per 4 elements, E1M2 elements -- but no rule for choosing
or rounding the scales; the reading is in tests/golden/hif4_worked.txt.
Pinned by: the E6M2 value set from the format's definition (exact
rationals) and its round-to-nearest-even encoding against an exact nearest
search; hand-derived worked blocks; an independent brute-force quantizer
in exact rationals on tiny inputs (RHT on and off, RTNE and SR with draws
from rocRAND's Philox); on-grid round trips; COL = ROW(x^T); and the page's
direction (HiF4 loses less signal than MXFP4 everywhere, and than NVFP4
under the RHT).
"""
import bisect
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.linalg import hadamard

import oracle
import workloads
from tests.conftest import read_golden
from tests.test_oracle_tensor import _kat_draws, _kat_signs, _rht_exact_bf16

H16 = hadamard(16).astype(np.float64)


def _e6m2_exact(b: int) -> Fraction:
    e, m = b >> 2, b & 3
    if e == 0:
        return Fraction(m, 4) * Fraction(2) ** (1 - 31)
    return (1 + Fraction(m, 4)) * Fraction(2) ** (e - 31)


E6M2 = [_e6m2_exact(b) for b in range(256)]


def _e6m2_nearest(r: Fraction) -> int:
    """Nearest E6M2 byte, ties to the even byte, saturating at the largest."""
    if r >= E6M2[255]:
        return 255
    hi = bisect.bisect_left(E6M2, r)  # E6M2[hi - 1] < r <= E6M2[hi]
    if hi == 0 or E6M2[hi] == r:
        return hi
    lo = hi - 1
    dl, dh = r - E6M2[lo], E6M2[hi] - r
    return lo if dl < dh else hi if dh < dl else (lo if lo % 2 == 0 else hi)


def test_e6m2_values():
    for b in range(256):
        assert Fraction(oracle.e6m2_decode(b)) == E6M2[b], b
    assert all(E6M2[b] < E6M2[b + 1] for b in range(255))
    assert E6M2[4] == Fraction(1, 2 ** 30) and E6M2[1] == Fraction(1, 2 ** 32)
    assert E6M2[255] == Fraction(7, 4) * 2 ** 32


def test_e6m2_encode_nearest_even():
    """Every binary32 within 32 ulps of each value and each midpoint, plus
    log-uniform values over the range and past the saturation point."""
    pts = []
    for b in range(255):
        for q in (E6M2[b], (E6M2[b] + E6M2[b + 1]) / 2):
            v = np.float32(float(q))
            bits = np.array([v], dtype=np.float32).view(np.uint32)[0]
            pts.append(((bits + np.arange(-32, 33, dtype=np.int64)).clip(0, 0x7F7FFFFF))
                       .astype(np.uint32).view(np.float32))
    rng = np.random.default_rng(3)
    pts.append(np.exp2(rng.uniform(-40, 40, 4000)).astype(np.float32))
    pts.append(np.array([0.0, 2.0 ** 33, 1.875 * 2 ** 32, 3e38], dtype=np.float32))
    v = np.unique(np.concatenate(pts))
    v = v[v >= 0]
    got = oracle.e6m2_encode(v)
    for x, g in zip(v, got):
        assert g == _e6m2_nearest(Fraction(float(x))), float(x)


def test_hif4_worked_blocks():
    for name, entries, sbytes, codes in read_golden("hif4_worked.txt"):
        x = np.zeros((1, 64), dtype=np.float32)
        for e in entries.split(","):
            i, v = e.split(":")
            x[0, int(i)] = np.float32(float(v))
        c, s, ts = oracle.quantize(x, "hif4")
        assert ts is None
        assert list(s[0]) == [int(b) for b in sbytes.split(",")], name
        k = oracle.unpack_codes(c)[0]
        want = np.zeros(64, dtype=np.uint8)
        for e in codes.split(","):
            i, v = e.split(":")
            want[int(i)] = int(v)
        assert np.array_equal(k, want), name


# ------------------------------------------------ brute force, exact rationals
def _hif4_brute(y: np.ndarray, rounding="rtne", draws=None):
    """Independent HiF4 quantizer of the rows of y (float32, already rotated
    when the RHT is on), in exact rationals, following the reading in
    tests/golden/hif4_worked.txt.  Returns (codes [R, W], scale bytes [R, W/16])."""
    R, W = y.shape
    codes = np.zeros((R, W), dtype=np.uint8)
    sc = np.zeros((R, W // 16), dtype=np.uint8)
    for i in range(R):
        for b in range(W // 64):
            blk = [Fraction(float(v)) for v in y[i, 64 * b:64 * b + 64]]
            amax = max(abs(v) for v in blk)
            r = Fraction(float(np.float32(np.float32(float(amax)) / np.float32(1.75))))
            sb = _e6m2_nearest(r)
            S = E6M2[sb]
            word = sb
            f4s = []
            for s in range(8):
                a8 = max(abs(v) for v in blk[8 * s:8 * s + 8])
                keep8 = a8 > Fraction(7, 8) * S
                word |= int(keep8) << (8 + s)
                f8 = 1 if keep8 else Fraction(1, 2)
                for u in (2 * s, 2 * s + 1):
                    a4 = max(abs(v) for v in blk[4 * u:4 * u + 4])
                    keep4 = a4 > Fraction(7, 8) * S * f8
                    word |= int(keep4) << (16 + u)
                    f4s.append(f8 * (1 if keep4 else Fraction(1, 2)))
            for j in range(4):
                sc[i, 4 * b + j] = (word >> (8 * j)) & 0xFF
            for e in range(64):
                v = blk[e]
                d = S * f4s[e // 4] / 4
                k = 0
                if d != 0 and v != 0:
                    inv = np.float32(np.float32(1.0) / np.float32(float(d)))
                    m = Fraction(float(np.float32(abs(np.float32(float(v)) * inv))))
                    if m >= 7:
                        k = 7
                    elif rounding == "sr":
                        fl = int(m)  # floor, m >= 0
                        p = m - fl
                        u16 = int(draws[i * W + 64 * b + e])
                        k = fl + (1 if Fraction(64 * u16 + 1, 1 << 22) <= p else 0)
                    else:
                        fl = int(m)
                        frac = m - fl
                        k = fl + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2)
                                  else 0)
                codes[i, 64 * b + e] = (8 if np.signbit(np.float32(float(y[i, 64 * b + e])))
                                        else 0) | k
    return codes, sc


@pytest.mark.parametrize("kind", ["normal", "wide_range", "tiny", "zeros_mixed", "grid_ties",
                                  "outlier_cols"])
def test_hif4_brute_force_tiny(kind):
    x = workloads.small_case(kind, 3, 128, 23)
    c, s, _ = oracle.quantize(x, "hif4")
    bc, bs = _hif4_brute(x)
    assert np.array_equal(s, bs)
    assert np.array_equal(oracle.unpack_codes(c), bc)


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
@pytest.mark.parametrize("spikes", [False, True])
def test_hif4_brute_force_rht_and_sr(rocrand_kat, rounding, spikes):
    rht_seed, sr_seed = 0xABCDEF, 0x5151
    x = _rht_exact_bf16(3, 128, 51 + int(spikes), spikes)
    R, C = x.shape
    signs = _kat_signs(rocrand_kat, rht_seed)
    a = workloads.bf16_bits_to_f32(x).astype(np.float64).reshape(R, C // 16, 16) * signs
    y64 = 0.25 * np.einsum("rgj,ij->rgi", a, H16)
    y = y64.astype(np.float32)
    assert np.array_equal(y.astype(np.float64), y64)
    draws = _kat_draws(rocrand_kat, sr_seed, R * C) if rounding == "sr" else None
    c, s, _ = oracle.quantize(x, "hif4", "row", rounding, True, rht_seed, sr_seed)
    bc, bs = _hif4_brute(y.reshape(R, C), rounding, draws)
    assert np.array_equal(s, bs)
    assert np.array_equal(oracle.unpack_codes(c), bc)


def test_hif4_round_trip_on_grid():
    """Blocks built on the hierarchy's own grid come back exactly: S from the
    E6M2 set, the first micro-block unrefined with its maximum at the top
    level (so the block scale is S again), every other micro-block at
    random factors with its maximum on its own top level (the selection
    then finds the same step S * f8 * f4 / 4, whichever bits express it),
    elements k * d."""
    rng = np.random.default_rng(9)
    rows = []
    for _ in range(24):
        sb = int(rng.integers(20, 240))
        S = float(E6M2[sb])
        blk = np.zeros(64)
        f8 = rng.choice([0.5, 1.0], 8)
        f8[0] = 1.0
        for s in range(8):
            for u in (2 * s, 2 * s + 1):
                f4 = 1.0 if (u == 0 or rng.random() < 0.5) else 0.5
                d = S * f8[s] * f4 / 4
                k = rng.integers(0, 8, 4)
                k[0] = 7  # each piece's maximum sits on its top level
                blk[4 * u:4 * u + 4] = rng.choice([-1.0, 1.0], 4) * k * d
        rows.append(blk)
    x = np.array(rows).astype(np.float32).reshape(4, 384)
    c, s, _ = oracle.quantize(x, "hif4")
    y = oracle.dequantize(c, s, None, 4, 384, "hif4")
    assert np.array_equal(y, x)


def test_hif4_col_equals_row_of_transpose():
    x = workloads.to_bf16_bits(workloads.small_case("t3", 128, 64, 2))
    for rounding, rht in (("rtne", False), ("sr", True)):
        col = oracle.quantize(x, "hif4", "col", rounding, rht, 5, 77)
        row = oracle.quantize(np.ascontiguousarray(x.T), "hif4", "row", rounding, rht, 5, 77)
        assert np.array_equal(col[0], row[0]) and np.array_equal(col[1], row[1])
        bc = oracle.dequantize(col[0], col[1], None, 128, 64, "hif4", "col", rht, 5, rht)
        br = oracle.dequantize(row[0], row[1], None, 64, 128, "hif4", "row", rht, 5, rht)
        assert np.array_equal(bc, br.T)


def _sqnr(x, fmt, rht):
    c, s, ts = oracle.quantize(x, fmt, rht=rht)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    xh = oracle.dequantize(c, s, ts, *x.shape, fmt, rht=rht, inverse_rht=rht).astype(np.float64)
    return 10 * np.log10((xf ** 2).sum() / ((xh - xf) ** 2).sum())


@pytest.mark.parametrize("maker", [
    lambda: workloads.activation_with_outlier_channels(256, 1024, 1),
    lambda: workloads.student_t_bf16(256, 1024, 2, 4.0),
    lambda: workloads.normal_bf16(256, 1024, 3, 0.02),
    lambda: workloads.weight_with_spikes(256, 1024, 0)])
def test_hif4_direction(maker):
    """HiFloat page, 4.B: HiF4's hierarchy keeps 4-bit quantization usable
    where a single-level format degrades: it loses less signal than MXFP4
    on every tensor, and than NVFP4 once the RHT spreads the outliers."""
    x = maker()
    for rht in (False, True):
        assert _sqnr(x, "hif4", rht) > _sqnr(x, "mxfp4", rht)
    assert _sqnr(x, "hif4", True) > _sqnr(x, "nvfp4", True)
