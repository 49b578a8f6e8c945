"""GPU parity of HiF4 (E6M2 per 64, E1M0 per 8 and per 4, E1M2 elements)
against the oracle, byte for byte: codes, the 4-byte scale words and the
dequantized values (FP32 and BF16, with and without the inverse RHT), on
both axes, RTNE and SR, BF16 and FP32 input.  Row-axis shapes have W % 64
== 0 with ragged row counts; column-axis shapes leave a bottom strip of
one 64-row block below the 256-row tiles and a right strip of columns."""
import itertools

import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import assert_bytes_equal, note, quantize_both

pytestmark = pytest.mark.gpu

ROW_SHAPES = [(33, 64), (130, 384), (1000, 1088)]
COL_SHAPES = [(64, 40), (320, 136), (1088, 200)]
KINDS = workloads.SMALL_KINDS
COMBOS = list(itertools.product(["row", "col"], ["rtne", "sr"], [False, True], ["bf16", "f32"]))


@pytest.mark.parametrize("axis,rounding,rht,dtype", COMBOS,
                         ids=["-".join(map(str, c)) for c in COMBOS])
def test_hif4_quantize_dequantize_parity(axis, rounding, rht, dtype):
    for i, shape in enumerate(ROW_SHAPES if axis == "row" else COL_SHAPES):
        kind = KINDS[(i + 3 * rht + (axis == "col")) % len(KINDS)]
        a = workloads.small_case(kind, shape[0], shape[1], 700 + i)
        x = workloads.to_bf16_bits(a) if dtype == "bf16" else a
        note("hif4 parity %s %s rht=%s %s %s %s" % (axis, rounding, rht, dtype, shape, kind))
        c, s, ts, (oc, osc, ots) = quantize_both(x, "hif4", axis, rounding, rht, 3, 5 + i)
        assert ts is None and ots is None
        rows, cols = shape
        for inv in ([False, True] if rht else [False]):
            for odt in (torch.float32, torch.bfloat16):
                out = fp4.dequantize(c, s, None, rows, cols, "hif4", axis, rht, 3, inv, odt)
                torch.cuda.synchronize()
                want = oracle.dequantize(oc, osc, None, rows, cols, "hif4", axis, rht, 3, inv,
                                         "f32" if odt == torch.float32 else "bf16")
                got = out.cpu()
                got = (got.view(torch.int16).numpy().view(np.uint16) if odt == torch.bfloat16
                       else got.numpy().view(np.uint32))
                want = want if odt == torch.bfloat16 else want.view(np.uint32)
                assert_bytes_equal(got, want, "hif4 dequant %s inv=%s %s" % (axis, inv, odt))


def test_hif4_col_equals_row_of_transpose_on_gpu():
    x = workloads.to_bf16_bits(workloads.small_case("t3", 512, 192, 4))
    xt = np.ascontiguousarray(x.T)
    from tests.gpu_util import to_device
    c1, s1, _ = fp4.quantize(to_device(x), "hif4", "col", "sr", True, 6, 8)
    c2, s2, _ = fp4.quantize(to_device(xt), "hif4", "row", "sr", True, 6, 8)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


def test_hif4_rejects_ragged_blocks():
    from tests.gpu_util import to_device
    with pytest.raises(fp4.FP4Error):
        fp4.quantize(to_device(np.zeros((4, 96), dtype=np.float32)), "hif4")  # 96 % 64
