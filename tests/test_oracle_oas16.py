"""Pins for the oracle's overflow-aware MXFP4 on 16-element blocks (CPU only).

The MXFP4 page ("Unveiling the Potential of Quantization with MXFP4", 2.
Methodologie et Analyse) applies its techniques at a block granularity of
16; OAS (2.A) maps each block's amax into (3.5, 7].  Pinned by hand-derived
worked examples (tests/golden/mxfp4_oas16_worked.txt), by the relation to
the (separately pinned) 32-element OAS -- a 16-block quantized alone equals
that block duplicated into a 32-element OAS block -- with and without the
RHT, by on-grid round trips, and by the page's direction: 16-element blocks
flush fewer small values to zero and lose less signal than 32-element ones.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.conftest import read_golden

E2M1 = np.array(oracle.E2M1_LEVELS, dtype=np.float64)


def test_oas16_worked_examples():
    for a0, a1, b0, b1, k0, k1, l0, l1 in read_golden("mxfp4_oas16_worked.txt"):
        a0, a1, l0, l1 = float(a0), float(a1), float(l0), float(l1)
        b0, b1, k0, k1 = int(b0), int(b1), int(k0), int(k1)
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, 0], x[0, 1:16] = a0, a0 / 64
        x[0, 16], x[0, 17:] = a1, a1 / 64
        codes, scales, ts = oracle.quantize(x, "mxfp4_oas16")
        assert ts is None
        assert scales.shape == (1, 2) and tuple(scales[0]) == (b0, b1)
        c = oracle.unpack_codes(codes)[0]
        assert (c[0], c[16]) == (k0, k1)
        y = oracle.dequantize(codes, scales, None, 1, 32, "mxfp4_oas16")
        assert y[0, 0] == l0 * (2.0 ** (b0 - 127) if b0 else 0.0)
        assert y[0, 16] == l1 * 2.0 ** (b1 - 127)


@pytest.mark.parametrize("kind", ["normal", "t3", "wide_range", "zeros_mixed", "grid_ties"])
@pytest.mark.parametrize("rht", [False, True])
def test_oas16_block_equals_duplicated_oas32_block(kind, rht):
    """OAS16 of each 16-block equals the first half of the 32-element OAS of
    that block written twice (same amax, so the same exponent and codes)."""
    x = workloads.small_case(kind, 6, 64, 17)
    c16, s16, _ = oracle.quantize(x, "mxfp4_oas16", rht=rht, rht_seed=9)
    dup = np.repeat(x.reshape(6, 4, 1, 16), 2, axis=2).reshape(6, 128)
    c32, s32, _ = oracle.quantize(dup, "mxfp4_oas", rht=rht, rht_seed=9)
    assert np.array_equal(s16, s32)
    k16 = oracle.unpack_codes(c16).reshape(6, 4, 16)
    k32 = oracle.unpack_codes(c32).reshape(6, 4, 2, 16)
    assert np.array_equal(k16, k32[:, :, 0]) and np.array_equal(k16, k32[:, :, 1])


def test_oas16_round_trip_on_grid():
    rng = np.random.default_rng(5)
    rows = []
    es = []
    for _ in range(32):
        e = int(rng.integers(-60, 60))
        k = rng.integers(0, 8, 16)
        k[rng.integers(0, 16)] = 7
        rows.append((rng.choice([-1.0, 1.0], 16) * E2M1[k] * 2.0 ** e))
        es.append(e)
    x = np.concatenate(rows).astype(np.float32).reshape(2, 256)
    codes, scales, _ = oracle.quantize(x, "mxfp4_oas16")
    assert np.array_equal(scales.ravel(), np.array(es) + 127)   # 6 * 2^e: 6 in (3.5, 7]
    assert np.array_equal(oracle.dequantize(codes, scales, None, 2, 256, "mxfp4_oas16"), x)


def test_oas16_col_equals_row_of_transpose():
    x = workloads.to_bf16_bits(workloads.small_case("t3", 96, 64, 2))
    for rounding in ("rtne", "sr"):
        col = oracle.quantize(x, "mxfp4_oas16", "col", rounding, True, 5, 77)
        row = oracle.quantize(np.ascontiguousarray(x.T), "mxfp4_oas16", "row", rounding, True,
                              5, 77)
        assert np.array_equal(col[0], row[0]) and np.array_equal(col[1], row[1])


def _sqnr_ftz(x, fmt):
    codes, scales, _ = oracle.quantize(x, fmt)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    xh = oracle.dequantize(codes, scales, None, *x.shape, fmt).astype(np.float64)
    nz = xf != 0
    return (10 * np.log10((xf ** 2).sum() / ((xh - xf) ** 2).sum()),
            ((xh == 0) & nz).sum() / nz.sum())


@pytest.mark.parametrize("maker", [lambda: workloads.activation_with_outlier_channels(256, 1024, 1),
                                   lambda: workloads.student_t_bf16(256, 1024, 2, 4.0),
                                   lambda: workloads.normal_bf16(256, 1024, 3, 0.02)])
def test_oas16_direction(maker):
    """MXFP4 page, 2. Methodologie et Analyse: smaller blocks reduce the
    flush-to-zero rate of low-magnitude values, and OAS reduces the error;
    16-element OAS beats 32-element OAS and plain MXFP4 on SQNR."""
    x = maker()
    q16, f16 = _sqnr_ftz(x, "mxfp4_oas16")
    q32, f32 = _sqnr_ftz(x, "mxfp4_oas")
    qmx, fmx = _sqnr_ftz(x, "mxfp4")
    assert q16 > q32 > qmx
    assert f16 < f32
