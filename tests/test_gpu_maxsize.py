"""A 2^31-element operand (65536 x 32768 BF16, 4 GiB): every element offset
past 2^31 must be formed in 64 bits in the row kernel, the column tiles,
the tensor-amax passes and the outer scales.  The operand repeats one
seeded 4096 x 4096 Student-t block, each of the 128 copies scaled by its own
power of two (exact in BF16), so a wrapped offset reads the wrong copy.
Every output byte is compared with the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import DEV, assert_bytes_equal, f32_bits, note, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROWS, COLS, T = 65536, 32768, 4096


def _operand() -> np.ndarray:
    base = workloads.student_t_bf16(T, T, 5, 3.0)
    live = (base & 0x7F80) != 0  # leave zeros and subnormals alone
    big = np.empty((ROWS, COLS), dtype=np.uint16)
    for i in range(ROWS // T):
        for j in range(COLS // T):
            k = (i * (COLS // T) + j) % 8          # scale by 2^k: exponent field + k
            big[i * T:(i + 1) * T, j * T:(j + 1) * T] = np.where(live, base + (k << 7), base)
    return big


@pytest.fixture(scope="module")
def operand():
    note("max-size operand: generating %dx%d BF16" % (ROWS, COLS))
    x = _operand()
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return x, xd


@pytest.mark.parametrize("axis,rounding,outer", [("row", "sr", False), ("col", "rtne", True)])
def test_two_gib_elements(operand, axis, rounding, outer):
    x, xd = operand
    note("max-size %s %s outer=%s" % (axis, rounding, outer))
    c, s, ts = fp4.quantize(xd, "nvfp4", axis, rounding, True, 3, 1, outer=outer)
    torch.cuda.synchronize()
    gc, gs, gt = to_host(c), to_host(s), to_host(ts)
    del c, s, ts
    oc, osc, ots = oracle.quantize(x, "nvfp4", axis, rounding, True, 3, 1, outer=outer)
    assert_bytes_equal(gs, osc, "scales")
    assert_bytes_equal(gc, oc, "codes")
    if outer:
        assert_bytes_equal(gt.view(np.uint32), ots.view(np.uint32), "outer scales")
    else:
        assert f32_bits(float(gt[0])) == f32_bits(ots)
