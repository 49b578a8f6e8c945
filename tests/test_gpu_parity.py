"""GPU parity: the HIP path through the C ABI against the oracle, byte for
byte (codes, scale bytes, tensor scale, dequantized values, RHT outputs).

Sizes are small enough for the oracle to finish in well under a second, yet
span many workgroups and leave ragged tails; the data kinds cover heavy
tails, outlier channels, wide dynamic range, subnormals, zeros and exact
rounding ties."""
import itertools

import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import (DEV, assert_bytes_equal, f32_bits, note, quantize_both, to_device,
                            to_host)

pytestmark = pytest.mark.gpu

# (48, 80): rows and cols = 16 mod 32 (16-element row pieces, unaligned
# column code rows); 1056 rows leave a 32-row tail below the 128-row runs.
SHAPES = [(32, 32), (96, 160), (224, 64), (1056, 352), (48, 80)]
KINDS = workloads.SMALL_KINDS

COMBOS = list(itertools.product(["nvfp4", "mxfp4", "ufp4", "mxfp4_oas", "e2m1_cap2",
                                 "mxfp4_oas16"], ["row", "col"],
                                ["rtne", "sr"], [False, True], ["bf16", "f32"]))

# Double-block (outer scale per 128) shapes: W % 128 == 0 on the axis used.
# (128, 256) col: no whole column tile (run kernel only); (640, 200) col:
# tiles plus a right strip of 8 columns and a bottom strip of 128 rows;
# (384, 1152) row: nine outer pieces per row; (256, 384): whole tiles.
OUTER_SHAPES = [(128, 256), (640, 200), (384, 1152), (256, 384)]
OUTER_COMBOS = list(itertools.product(["nvfp4", "ufp4", "e2m1_cap2", "mxfp4_mbs"], ["row", "col"], ["rtne", "sr"],
                                      [False, True], ["bf16", "f32"]))


def _input(kind, shape, seed, dtype):
    a = workloads.small_case(kind, shape[0], shape[1], seed)
    return workloads.to_bf16_bits(a) if dtype == "bf16" else a


@pytest.mark.parametrize("fmt,axis,rounding,rht,dtype", COMBOS,
                         ids=["-".join(map(str, c)) for c in COMBOS])
def test_quantize_dequantize_parity(fmt, axis, rounding, rht, dtype):
    for i, shape in enumerate(SHAPES):
        W = shape[1] if axis == "row" else shape[0]
        if W % fp4.BLOCK[fmt]:
            continue
        kind = KINDS[(i + len(fmt) + (3 if rht else 0) + (1 if axis == "col" else 0)) % len(KINDS)]
        x = _input(kind, shape, 100 + i, dtype)
        note("parity %s %s %s rht=%s %s %s %s" % (fmt, axis, rounding, rht, dtype, shape, kind))
        c, s, ts, (oc, osc, ots) = quantize_both(x, fmt, axis, rounding, rht, 3, 5 + i)
        rows, cols = shape
        for inv in ([False, True] if rht else [False]):
            for odt in (torch.float32, torch.bfloat16):
                out = fp4.dequantize(c, s, ts, rows, cols, fmt, axis, rht, 3, inv, odt)
                torch.cuda.synchronize()
                want = oracle.dequantize(oc, osc, ots, rows, cols, fmt, axis, rht, 3, inv,
                                         "f32" if odt == torch.float32 else "bf16")
                got = to_host(out)
                if odt == torch.float32:
                    got, want = got.view(np.uint32), want.view(np.uint32)
                assert_bytes_equal(got, want, "dequant inv=%s %s %s" % (inv, odt, shape))


@pytest.mark.parametrize("fmt,axis,rounding,rht,dtype", OUTER_COMBOS,
                         ids=["-".join(map(str, c)) for c in OUTER_COMBOS])
def test_outer_scale_parity(fmt, axis, rounding, rht, dtype):
    for i, shape in enumerate(OUTER_SHAPES):
        W = shape[1] if axis == "row" else shape[0]
        if W % 128:
            continue
        kind = KINDS[(i + 2 * len(fmt) + (1 if rht else 0) + (2 if axis == "col" else 0))
                     % len(KINDS)]
        x = _input(kind, shape, 200 + i, dtype)
        note("outer %s %s %s rht=%s %s %s %s" % (fmt, axis, rounding, rht, dtype, shape, kind))
        c, s, ts, (oc, osc, ots) = quantize_both(x, fmt, axis, rounding, rht, 4, 9 + i,
                                                 outer=True)
        rows, cols = shape
        for inv in ([False, True] if rht else [False]):
            out = fp4.dequantize(c, s, ts, rows, cols, fmt, axis, rht, 4, inv, torch.float32)
            torch.cuda.synchronize()
            want = oracle.dequantize(oc, osc, ots, rows, cols, fmt, axis, rht, 4, inv, "f32")
            assert_bytes_equal(to_host(out).view(np.uint32), want.view(np.uint32),
                               "outer dequant inv=%s %s" % (inv, shape))


# Row dequantize to BF16 with 64 or more 16-element blocks per row (the
# path whose waves trade block halves so that each store instruction writes
# one contiguous 1 KB): 64 and 128 blocks per row, every 16-element format,
# outer scales, the inverse RHT on and off, and an output pitch above the
# width.
WAVE_ROW_CASES = list(itertools.product(["nvfp4", "ufp4", "e2m1_cap2", "mxfp4_oas16",
                                         "mxfp4_mbs"], [False, True]))


@pytest.mark.parametrize("fmt,rht", WAVE_ROW_CASES,
                         ids=["%s-rht%d" % (f, r) for f, r in WAVE_ROW_CASES])
def test_dequant_bf16_whole_wave_rows(fmt, rht):
    for i, (shape, pitch) in enumerate([((64, 1024), 1024), ((40, 2048), 2048),
                                        ((24, 1024), 1152)]):
        kind = KINDS[(i + len(fmt)) % len(KINDS)]
        x = _input(kind, shape, 300 + i, "bf16")
        rows, cols = shape
        outer = fmt == "mxfp4_mbs" or (fmt != "mxfp4_oas16" and i == 1)
        note("wave rows %s rht=%s %s outer=%s %s" % (fmt, rht, shape, outer, kind))
        c, s, ts, (oc, osc, ots) = quantize_both(x, fmt, "row", "rtne", rht, 6, 1,
                                                 outer=outer)
        for inv in ([False, True] if rht else [False]):
            full = torch.zeros((rows, pitch), dtype=torch.bfloat16, device=DEV)
            out = full[:, :cols]
            fp4.dequantize(c, s, ts, rows, cols, fmt, "row", rht, 6, inv, torch.bfloat16,
                           out=out)
            torch.cuda.synchronize()
            want = oracle.dequantize(oc, osc, ots, rows, cols, fmt, "row", rht, 6, inv, "bf16")
            assert_bytes_equal(to_host(out), want, "wave rows inv=%s %s" % (inv, shape))
            if pitch > cols:  # the padding is left alone
                assert not to_host(full[:, cols:]).any()


def test_outer_scale_rejects_ragged_width():
    x = to_device(np.zeros((64, 144), dtype=np.float32))
    with pytest.raises(fp4.FP4Error):
        fp4.quantize(x, "nvfp4", "row", outer=True)


@pytest.mark.parametrize("kind", KINDS)
def test_every_kind_nvfp4_rht(kind):
    for rounding in ("rtne", "sr"):
        x = _input(kind, (320, 256), 7, "bf16")
        note("kind %s %s" % (kind, rounding))
        quantize_both(x, "nvfp4", "row", rounding, True, 1, 1)
        quantize_both(x, "ufp4", "col", rounding, True, 1, 1)


@pytest.mark.parametrize("fmt", ["nvfp4", "ufp4", "e2m1_cap2"])
def test_given_tensor_scale(fmt):
    x = _input("t3", (128, 256), 3, "bf16")
    # 1e-39 (subnormal): 1/d overflows, blocks take the per-element careful
    # path; 1e38: decoded block scales overflow to infinity.
    for ts in (1e-3, 2.0 ** -20, 0.37, 1e4, 0.0, 1e-39, 1e38):
        note("given ts %s %g" % (fmt, ts))
        quantize_both(x, fmt, "row", "rtne", True, 0, 0, given=ts)
        quantize_both(x, fmt, "col", "sr", False, 0, 9, given=ts)


def test_poison_and_determinism():
    x = _input("outlier_cols", (512, 512), 1, "bf16")
    for fmt in ("nvfp4", "mxfp4"):
        note("poison %s" % fmt)
        a = quantize_both(x, fmt, "col", "sr", True, 2, 3, poison=0xAA)
        b = quantize_both(x, fmt, "col", "sr", True, 2, 3, poison=0x55)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_col_equals_row_of_transpose_on_gpu():
    x = _input("t3", (256, 160), 4, "bf16")
    xt = np.ascontiguousarray(x.T)
    for fmt in ("nvfp4", "mxfp4", "ufp4", "e2m1_cap2", "mxfp4_oas16"):
        note("transpose %s" % fmt)
        c1, s1, t1 = fp4.quantize(to_device(x), fmt, "col", "sr", True, 6, 8)
        c2, s2, t2 = fp4.quantize(to_device(xt), fmt, "row", "sr", True, 6, 8)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2) and torch.equal(s1, s2)
        if t1 is not None:
            assert torch.equal(t1, t2)


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rht_parity(axis, dtype):
    for kind, shape in (("t3", (64, 48)), ("wide_range", (208, 352)), ("tiny", (32, 32))):
        x = _input(kind, shape, 2, dtype)
        for inv in (False, True):
            note("rht %s %s %s inv=%s" % (axis, dtype, shape, inv))
            y = fp4.rht(to_device(x), axis, 11, inv)
            torch.cuda.synchronize()
            want = oracle.rht(x, axis, 11, inv)
            assert_bytes_equal(to_host(y).view(np.uint32), want.view(np.uint32), "rht")


def test_strided_input():
    base = workloads.to_bf16_bits(workloads.small_case("normal", 64, 96, 5))
    note("strided")
    xd = to_device(base)[:, :64]
    assert xd.stride(0) == 96
    c, s, ts = fp4.quantize(xd, "nvfp4", "row", "rtne", True, 0, 0)
    torch.cuda.synchronize()
    oc, osc, ots = oracle.quantize(np.ascontiguousarray(base[:, :64]), "nvfp4", "row", "rtne",
                                   True, 0, 0)
    assert_bytes_equal(to_host(c), oc, "codes")
    assert_bytes_equal(to_host(s), osc, "scales")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4", "ufp4", "e2m1_cap2"])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_column_axis_odd_column_count(fmt, rounding):
    """cols odd (one column per lane) through a strided view, ld = 40."""
    base = _input("t3", (160, 40), 8, "bf16")
    x = np.ascontiguousarray(base[:, :33])
    note("odd cols %s %s" % (fmt, rounding))
    xd = to_device(base)[:, :33]
    c, s, ts = fp4.quantize(xd, fmt, "col", rounding, True, 2, 7)
    torch.cuda.synchronize()
    oc, osc, ots = oracle.quantize(x, fmt, "col", rounding, True, 2, 7)
    assert_bytes_equal(to_host(c), oc, "codes")
    assert_bytes_equal(to_host(s), osc, "scales")
    if ts is not None:
        assert f32_bits(float(ts.item())) == f32_bits(ots)


def test_empty_and_single_block():
    note("empty")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s, ts = fp4.quantize(x, "nvfp4")
    torch.cuda.synchronize()
    assert c.numel() == 0 and float(ts.item()) == 0.0
    x1 = _input("normal", (1, 16), 0, "bf16")
    note("single block")
    quantize_both(x1, "nvfp4", "row", "sr", True, 0, 4)
    x2 = _input("normal", (32, 1), 0, "f32")
    with pytest.raises(fp4.FP4Error):
        fp4.quantize(to_device(x2), "nvfp4", "row")  # W = 1


def test_all_zero_tensor():
    x = np.zeros((64, 64), dtype=np.float32)
    x[3, 5] = -0.0
    for fmt in ("nvfp4", "mxfp4", "ufp4", "e2m1_cap2"):
        note("zeros %s" % fmt)
        quantize_both(x, fmt, "row", "sr", True, 0, 0)
        quantize_both(x, fmt, "col", "rtne", False, 0, 0)


def test_error_statuses_through_binding():
    x = to_device(_input("normal", (32, 48), 0, "bf16"))
    with pytest.raises(fp4.FP4Error) as e:
        fp4.quantize(x, "mxfp4")  # 48 % 32
    assert e.value.status == -3


def _same_or_both_nan(got, want, bits, tag):
    """Byte parity, except that NaN payloads may differ: positions must agree."""
    if bits == 32:
        g, w = got.view(np.uint32), want.view(np.uint32)
        gn = ((g & 0x7F800000) == 0x7F800000) & ((g & 0x007FFFFF) != 0)
        wn = ((w & 0x7F800000) == 0x7F800000) & ((w & 0x007FFFFF) != 0)
    else:
        g, w = got.view(np.uint16), want.view(np.uint16)
        gn = ((g & 0x7F80) == 0x7F80) & ((g & 0x007F) != 0)
        wn = ((w & 0x7F80) == 0x7F80) & ((w & 0x007F) != 0)
    assert np.array_equal(gn, wn), "NaN positions " + tag
    assert np.array_equal(g[~gn], w[~wn]), "values " + tag


@pytest.mark.parametrize("fmt", ["nvfp4", "ufp4", "mxfp4", "e2m1_cap2"])
def test_dequant_arbitrary_codes_and_scales(fmt):
    """Dequantize of random codes with every scale byte and tensor scales
    far from 1: decoded block scales below 2^-100, above 2^100 and infinite
    take the path that applies the inverse RHT's 1/4 after the butterfly,
    moderate ones fold it into d.  Against the oracle, both axes and
    output types."""
    rows, cols = 256, 384
    rng = np.random.default_rng(21)
    for axis in ("row", "col"):
        cshape, sshape = fp4.output_shapes(rows, cols, fmt, axis)
        codes = rng.integers(0, 256, cshape, dtype=np.uint8)
        hi = 255 if fmt in fp4.MX else 127
        scales = rng.integers(0, hi, sshape, dtype=np.uint8)
        tss = (None,) if fmt in fp4.MX else (2.0 ** -20, 0.37, 1e4, 1e-35, 1e-39, 1e30, 1e38)
        for ts in tss:
            for inv in (False, True):
                for odt, name, bits in ((torch.float32, "f32", 32), (torch.bfloat16, "bf16", 16)):
                    note("dequant codes %s %s ts=%s inv=%s %s" % (fmt, axis, ts, inv, name))
                    tsd = None if ts is None else torch.tensor([ts], dtype=torch.float32,
                                                               device=DEV)
                    out = fp4.dequantize(to_device(codes), to_device(scales), tsd, rows, cols,
                                         fmt, axis, True, 2, inv, odt)
                    torch.cuda.synchronize()
                    want = oracle.dequantize(codes, scales,
                                             None if ts is None else np.float32(ts), rows,
                                             cols, fmt, axis, True, 2, inv, name)
                    _same_or_both_nan(to_host(out), want, bits, "%s %s ts=%s inv=%s %s" % (
                        fmt, axis, ts, inv, name))


def test_dequant_mbs_arbitrary_codes_scales_and_macro():
    """MBS-Static dequantize of random codes, every E8M0 byte and macro scales
    from zero and subnormals to 1e30: d_b = M * 2^(byte - 127) underflows,
    overflows and lands on subnormals; the inverse RHT's 1/4 folds into d or
    not.  Against the oracle, both axes and output types."""
    rows, cols = 256, 384
    rng = np.random.default_rng(22)
    macros = np.array([0.0, 1e-44, 3e-39, 2.0 ** -100, 0.37, 6.5, 2.0 ** 60, 1e30], np.float32)
    for axis in ("row", "col"):
        cshape, sshape = fp4.output_shapes(rows, cols, "mxfp4_mbs", axis)
        oshape = fp4.outer_shape(rows, cols, axis)
        codes = rng.integers(0, 256, cshape, dtype=np.uint8)
        scales = rng.integers(0, 255, sshape, dtype=np.uint8)
        macro = rng.choice(macros, oshape).astype(np.float32)
        for inv in (False, True):
            for odt, name, bits in ((torch.float32, "f32", 32), (torch.bfloat16, "bf16", 16)):
                note("dequant mbs %s inv=%s %s" % (axis, inv, name))
                out = fp4.dequantize(to_device(codes), to_device(scales), to_device(macro), rows,
                                     cols, "mxfp4_mbs", axis, True, 2, inv, odt)
                torch.cuda.synchronize()
                want = oracle.dequantize(codes, scales, macro, rows, cols, "mxfp4_mbs", axis,
                                         True, 2, inv, name)
                _same_or_both_nan(to_host(out), want, bits,
                                  "mbs %s inv=%s %s" % (axis, inv, name))
