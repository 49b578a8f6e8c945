"""Pins for the oracle's single-pass scale hierarchies (CPU only).

Double block ([TJ2] 2.A): an FP32 outer scale per 128 elements of an A-row
takes the place of the per-tensor scale.  Pinned by (i) reduction to the
per-tensor mode, which the other oracle tests pin, on 1 x 128 operands;
(ii) locality: every 128-piece of every A-row gives the bytes of that piece
quantized alone; (iii) an independent recomputation of a small case from
numpy float32 arithmetic, torch's E4M3 cast and a brute-force nearest-level
search; (iv) the largest inner block of each piece takes the top E4M3 byte.

Overflow-aware MXFP4 ([MXFP4] 2.A): the worked examples in
tests/golden/mxfp4_oas_worked.txt, and the defining interval 3.5 < amax/2^e
<= 7 checked with exact rational arithmetic over many fp32 values.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import read_golden

E2M1 = np.array(oracle.E2M1_LEVELS, dtype=np.float64)
UNIF = np.array(oracle.UNIFORM_LEVELS, dtype=np.float64)


# ---------------------------------------------------------------- OAS
def test_oas_worked_examples():
    for amax, e, byte, k, lvl in read_golden("mxfp4_oas_worked.txt"):
        amax, e, byte, k, lvl = float(amax), int(e), int(byte), int(k), float(lvl)
        assert oracle.e8m0_exponent_oas(amax) == e, amax
        # the block: amax followed by 31 small values
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, 0] = amax
        x[0, 1:] = amax / 64
        codes, scales, _ = oracle.quantize(x, "mxfp4_oas")
        assert scales[0, 0] == byte
        kk = oracle.unpack_codes(codes)[0, 0]
        assert kk == k
        assert oracle.E2M1_LEVELS[kk] == lvl
        y = oracle.dequantize(codes, scales, None, 1, 32, "mxfp4_oas")
        assert y[0, 0] == lvl * 2.0 ** e


def _oas_exact(a: float) -> int:
    """Smallest e with a <= 7 * 2^e, in exact rational arithmetic."""
    q = Fraction(a)
    e = q.numerator.bit_length() - q.denominator.bit_length() - 4
    while q > 7 * Fraction(2) ** e:
        e += 1
    while q <= 7 * Fraction(2) ** (e - 1):
        e -= 1
    return e


def test_oas_defining_interval():
    rng = np.random.default_rng(21)
    bits = rng.integers(0x00800000, 0x7F7FFFFF, 20000, dtype=np.uint32)
    edges = np.array([3.5, 7.0, 7.0000005, 6.9999995, 14.0, 0.4375], dtype=np.float32)
    vals = np.concatenate([bits.view(np.float32), edges,
                           (edges[None, :] * np.exp2(np.arange(-60, 61))[:, None])
                           .astype(np.float32).ravel()])
    for a in vals:
        a = float(a)
        want = min(max(_oas_exact(a), -127), 127)
        assert oracle.e8m0_exponent_oas(a) == want, a
        if -127 < want < 127:
            r = Fraction(a) / Fraction(2) ** want
            assert Fraction(7, 2) < r <= 7
        # one above the standard exponent exactly when amax/2^e_std > 7
        es = oracle.e8m0_exponent(a)
        if -127 < es < 126:
            up = Fraction(a) / Fraction(2) ** es > 7
            assert oracle.e8m0_exponent_oas(a) == es + (1 if up else 0)
    assert oracle.e8m0_exponent_oas(0.0) == -127


def test_oas_round_trip_on_grid():
    """Blocks whose largest level is 4 or 6 times 2^e come back exactly."""
    rng = np.random.default_rng(3)
    for top in (4.0, 6.0):
        for e in (-10, -1, 0, 5):
            k = rng.integers(0, 8, 32)
            v = E2M1[k] * rng.choice([-1.0, 1.0], 32)
            v[7] = top
            v = np.clip(v, -top, top)
            x = (v * 2.0 ** e).astype(np.float32)[None, :]
            codes, scales, _ = oracle.quantize(x, "mxfp4_oas")
            assert scales[0, 0] == e + 127
            y = oracle.dequantize(codes, scales, None, 1, 32, "mxfp4_oas")
            assert (y == x).all()


# ------------------------------------------------------- double block
def test_outer_reduces_to_tensor_scale_on_one_piece():
    rng = np.random.default_rng(4)
    for fmt in ("nvfp4", "ufp4"):
        for rht, rnd in ((False, "rtne"), (True, "rtne"), (True, "sr")):
            x = (rng.standard_t(3, (1, 128)) * 0.3).astype(np.float32)
            a = oracle.quantize(x, fmt, "row", rnd, rht, 7, 11)
            b = oracle.quantize(x, fmt, "row", rnd, rht, 7, 11, outer=True)
            assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
            assert b[2].shape == (1, 1) and b[2][0, 0] == np.float32(a[2])


@pytest.mark.parametrize("axis", ["row", "col"])
def test_outer_locality(axis):
    """Each 128-piece of each A-row equals that piece quantized alone as a
    1 x 128 operand in the per-tensor mode (RTNE: SR draws are keyed on the
    position in the whole operand, so they would differ)."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((256, 384)) * np.exp(rng.uniform(-3, 3, (256, 1)))).astype(np.float32)
    x[:, 5] *= 40.0
    A = x if axis == "row" else np.ascontiguousarray(x.T)
    for fmt in ("nvfp4", "ufp4"):
        for rht in (False, True):
            codes, scales, so = oracle.quantize(x, fmt, axis, "rtne", rht, 3, 0, outer=True)
            assert so.shape == (A.shape[0], A.shape[1] // 128)
            for i in range(0, A.shape[0], 37):
                for o in range(A.shape[1] // 128):
                    piece = np.ascontiguousarray(A[i:i + 1, o * 128:(o + 1) * 128])
                    c1, s1, t1 = oracle.quantize(piece, fmt, "row", "rtne", rht, 3, 0)
                    assert (codes[i, o * 64:(o + 1) * 64] == c1[0]).all()
                    assert (scales[i, o * 8:(o + 1) * 8] == s1[0]).all()
                    assert so[i, o] == np.float32(t1)
            y = oracle.dequantize(codes, scales, so, *x.shape, fmt, axis, rht, 3, rht)
            # dequantize: per-piece reconstruction
            Y = y if axis == "row" else y.T
            i, o = 5, 1
            piece = np.ascontiguousarray(A[i:i + 1, o * 128:(o + 1) * 128])
            c1, s1, t1 = oracle.quantize(piece, fmt, "row", "rtne", rht, 3, 0)
            y1 = oracle.dequantize(c1, s1, t1, 1, 128, fmt, "row", rht, 3, rht)
            assert (Y[i, o * 128:(o + 1) * 128] == y1[0]).all()


def _nearest_code(m: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Brute force: the level nearest to m, ties to the even index; past the
    top level the top index."""
    d = np.abs(m[:, None] - levels[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.where(cand, np.arange(8)[None, :], 99)
    even = np.where(cand & (np.arange(8)[None, :] % 2 == 0), np.arange(8)[None, :], 99)
    k = np.where((cand.sum(axis=1) > 1), even.min(axis=1), idx.min(axis=1))
    return np.where(m >= levels[-1], 7, k)


@pytest.mark.parametrize("fmt", ["nvfp4", "ufp4"])
def test_outer_independent_recomputation(fmt):
    G = np.float32(6.0 if fmt == "nvfp4" else 7.0)
    levels = E2M1 if fmt == "nvfp4" else UNIF
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((3, 256)) * np.array([[1e-3], [1.0], [50.0]])).astype(np.float32)
    x[1, 130] = 900.0
    codes, scales, so = oracle.quantize(x, fmt, outer=True)
    got = oracle.unpack_codes(codes)
    for i in range(3):
        for o in range(2):
            y = x[i, o * 128:(o + 1) * 128]
            s_o = np.float32(np.float32(np.abs(y).max()) / np.float32(G * np.float32(448.0)))
            assert so[i, o] == s_o
            for b in range(8):
                yb = y[b * 16:(b + 1) * 16]
                r = np.float32(np.float32(np.abs(yb).max()) / np.float32(s_o * G))
                S = torch.tensor([r]).to(torch.float8_e4m3fn)
                Sb = int(S.view(torch.uint8).item())
                assert scales[i, o * 8 + b] == Sb
                d = np.float32(s_o * np.float32(S.to(torch.float32).item()))
                v = (yb * np.float32(np.float32(1.0) / d)).astype(np.float32)
                k = _nearest_code(np.abs(v).astype(np.float64), levels)
                want = k | (np.signbit(yb).astype(np.int64) << 3)
                assert (got[i, o * 128 + b * 16:o * 128 + (b + 1) * 16] == want).all()


def test_outer_top_inner_scale():
    rng = np.random.default_rng(2)
    x = (rng.standard_t(4, (64, 512)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    for fmt in ("nvfp4", "ufp4"):
        _, scales, so = oracle.quantize(x, fmt, "row", "rtne", True, 1, 0, outer=True)
        per_piece = scales.reshape(64, 4, 8).max(axis=2)
        assert (per_piece == 0x7E).all()
        assert (so > 0).all()


def test_outer_rejects_ragged_width():
    x = np.zeros((2, 144), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.quantize(x, "nvfp4", outer=True)
    # MXFP4 ignores the tensor-scale mode
    oracle.quantize(np.zeros((2, 160), dtype=np.float32), "mxfp4")
