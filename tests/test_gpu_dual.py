"""GPU parity of fp4_quantize_dual (row-axis and column-axis quantization in
one call) against the oracle's two single-axis quantizations, byte for
byte: fused BF16 tiles (rows and cols multiples of 128) and the shapes,
dtypes and formats that run as two single-axis calls."""
import itertools

import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import DEV, assert_bytes_equal, f32_bits, note, to_device, to_host

pytestmark = pytest.mark.gpu

FUSED = [(128, 128), (256, 384), (384, 256), (512, 128)]
SPLIT = [((96, 160), "bf16"), ((128, 256), "f32"), ((1056, 352), "bf16")]
COMBOS = list(itertools.product(["nvfp4", "ufp4", "e2m1_cap2"], ["rtne", "sr"], [False, True],
                                ["compute", "given", "outer"]))
# MBS-Static exists only with its 128-element macro scales
COMBOS += list(itertools.product(["mxfp4_mbs"], ["rtne", "sr"], [False, True], ["outer"]))


def _check(x, fmt, rounding, rht, mode, seed):
    rows, cols = x.shape
    given = (0.37, 1e-3) if mode == "given" else None
    outer = mode == "outer"
    (cr, sr_, tr), (cc, sc, tc) = fp4.quantize_dual(to_device(x), fmt, rounding, rht, 5, seed,
                                                    tensor_scale=given, outer=outer)
    torch.cuda.synchronize()
    for axis, (c, s, t) in (("row", (cr, sr_, tr)), ("col", (cc, sc, tc))):
        g = None if given is None else given[0 if axis == "row" else 1]
        oc, osc, ots = oracle.quantize(x, fmt, axis, rounding, rht, 5, seed, tensor_scale=g,
                                       outer=outer)
        tag = "dual %s %s %s rht=%s %s %s %s" % (axis, fmt, rounding, rht, mode, x.shape, x.dtype)
        assert_bytes_equal(to_host(s), osc, "scales " + tag)
        assert_bytes_equal(to_host(c), oc, "codes " + tag)
        if outer:
            assert_bytes_equal(to_host(t).view(np.uint32), ots.view(np.uint32), "outer " + tag)
        elif fmt not in fp4.NO_TENSOR_SCALE:
            assert f32_bits(float(to_host(t)[0])) == f32_bits(ots), "tensor scale " + tag


@pytest.mark.parametrize("fmt,rounding,rht,mode", COMBOS,
                         ids=["-".join(map(str, c)) for c in COMBOS])
def test_dual_fused_parity(fmt, rounding, rht, mode):
    for i, shape in enumerate(FUSED):
        kind = workloads.SMALL_KINDS[(i + len(mode) + (2 if rht else 0)) % len(workloads.SMALL_KINDS)]
        x = workloads.to_bf16_bits(workloads.small_case(kind, shape[0], shape[1], 300 + i))
        note("dual fused %s %s rht=%s %s %s %s" % (fmt, rounding, rht, mode, shape, kind))
        _check(x, fmt, rounding, rht, mode, 11 + i)


@pytest.mark.parametrize("fmt", ["nvfp4", "ufp4", "mxfp4", "mxfp4_oas", "mxfp4_mbs", "mxfp4_oas16"])
def test_dual_split_parity(fmt):
    mbs = fmt == "mxfp4_mbs"  # macro scales only: both dims multiples of 128
    for (shape, dt), rounding, rht in itertools.product(SPLIT, ["rtne", "sr"], [False, True]):
        unit = 128 if mbs else fp4.BLOCK[fmt]
        if shape[0] % unit or shape[1] % unit:
            continue
        a = workloads.small_case("t3", shape[0], shape[1], 9)
        x = workloads.to_bf16_bits(a) if dt == "bf16" else a
        note("dual split %s %s rht=%s %s %s" % (fmt, rounding, rht, shape, dt))
        _check(x, fmt, rounding, rht, "outer" if mbs else "compute", 3)


def test_dual_matches_single_calls_full_operand():
    """The 16384 x 4096 activation operand of the linear layer: the dual call
    equals the two single-axis calls of the same library."""
    w = workloads.workload("linear_layer")
    x = to_device(w.make("X"))
    note("dual vs single, linear-layer X")
    for outer in (False, True):
        (cr, sr_, tr), (cc, sc, tc) = fp4.quantize_dual(x, "nvfp4", "rtne", True, 0, 0,
                                                        outer=outer)
        r = fp4.quantize(x, "nvfp4", "row", "rtne", True, 0, 0, outer=outer)
        c = fp4.quantize(x, "nvfp4", "col", "rtne", True, 0, 0, outer=outer)
        torch.cuda.synchronize()
        for got, want in zip((cr, sr_, tr, cc, sc, tc), r + c):
            assert torch.equal(got.view(torch.uint8) if got.dtype != torch.float32 else got.view(torch.int32),
                               want.view(torch.uint8) if want.dtype != torch.float32 else want.view(torch.int32))


def test_dual_rejects_bad_arguments():
    x = to_device(np.zeros((128, 144), dtype=np.float32))
    with pytest.raises(fp4.FP4Error):
        fp4.quantize_dual(x, "nvfp4", outer=True)       # cols % 128
    x = to_device(np.zeros((120, 128), dtype=np.float32))
    with pytest.raises(fp4.FP4Error):
        fp4.quantize_dual(x, "nvfp4")                   # rows % 16
