"""Block scales at the rounding midpoints of the E4M3 grid.

A two-level block scale is the E4M3 code (round to nearest even) of the
binary32 quotient r = amax_b / (s_t * G) ([NGPT] per-tensor dynamic
scaling; [TJ2] 2.A).  The kernels select it from amax_b times a reciprocal
of s_t * G and divide the quotient out only near a midpoint of the grid, in
the subnormal range and at saturation, so these blocks are built to put r
on every midpoint of the normal and subnormal E4M3 ranges and within a few
units in the last place of it, on either side: FP32 operands, the RHT off
(the block maximum is the constructed value), given and computed tensor
scales, both axes, both roundings.  Every byte must be the oracle's."""
import numpy as np
import pytest

from tests.gpu_util import note, quantize_both

pytestmark = pytest.mark.gpu

G = np.float32(6.0)


def _midpoints():
    mids = []
    for e in range(-6, 9):
        for j in range(8):
            m = np.float32(np.ldexp(1.0 + (j + 0.5) / 8.0, e))
            if m < 448.0:
                mids.append(m)
    for k in range(8):
        mids.append(np.float32((k + 0.5) * 2.0 ** -9))
    return mids


def _operand(den, top):
    """Rows of 64 FP32 elements, four 16-element blocks per row.  Block i's
    largest magnitude is a = RN(m * den) moved by d patterns, d in [-6, 6],
    for every E4M3 midpoint m; the other elements are smaller.  The first
    block holds `top` (the tensor maximum for a computed scale)."""
    rng = np.random.default_rng(5)
    amax = []
    for m in _midpoints():
        base = int(np.float32(m * den).view(np.uint32))
        for d in range(-6, 7):
            amax.append(np.uint32(base + d).view(np.float32))
    amax = np.array([np.float32(top)] + amax, dtype=np.float32)
    nblk = -(-len(amax) // 16) * 16  # rows a multiple of 4: 16-byte rows of the transpose
    amax = np.concatenate([amax, np.full(nblk - len(amax), np.float32(1.0) * den, np.float32)])
    blocks = (rng.uniform(-0.9, 0.9, (nblk, 16)) * amax[:, None]).astype(np.float32)
    pos = rng.integers(0, 16, nblk)
    sign = np.where(rng.integers(0, 2, nblk) == 0, np.float32(1), np.float32(-1))
    blocks[np.arange(nblk), pos] = amax * sign
    return blocks.reshape(nblk // 4, 64)


@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
@pytest.mark.parametrize("given", [True, False])
def test_block_scales_at_e4m3_midpoints(axis, rounding, given):
    top = np.float32(1000.0)
    if given:
        s_t = np.float32(0.37)
    else:
        s_t = np.float32(top / np.float32(G * np.float32(448.0)))
    den = np.float32(s_t * G)
    x = _operand(den, top if not given else np.float32(448.0) * den)
    if axis == "col":
        x = np.ascontiguousarray(x.T)
    note("e4m3 midpoints %s %s given=%s %s" % (axis, rounding, given, x.shape))
    quantize_both(x, "nvfp4", axis, rounding, False, 0, 3,
                  given=np.float32(s_t) if given else None)
