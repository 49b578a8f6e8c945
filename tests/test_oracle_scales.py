"""Pins for the oracle's scale bytes (CPU only).

E4M3: torch's float8_e4m3fn cast (a library routine: round to nearest even,
subnormals kept) agrees with the oracle below 464, where that cast does not
overflow; at and above 448 the oracle saturates by rule.  E8M0: the defining
inequality 2^(e+2) <= amax < 2^(e+3) over many fp32 values, plus the worked
examples in tests/golden/mxfp4_worked.txt.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.conftest import read_golden


def _torch_e4m3_bytes(r: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(r.astype(np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_for_every_byte():
    b = np.arange(0, 0x7F, dtype=np.uint8)  # 0x7F is NaN
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_decode(int(x)) for x in b], dtype=np.float32)
    assert (got == want).all()
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9


def _e4m3_probe_values() -> np.ndarray:
    vals = torch.from_numpy(np.arange(0, 0x7F, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float32).numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    anchors = np.concatenate([vals, mids])
    off = np.arange(-256, 257, dtype=np.int64)
    bits = anchors.view(np.int32).astype(np.int64)[:, None] + off[None, :]
    bits = bits[bits >= 0].astype(np.uint32)
    rng = np.random.default_rng(5)
    logu = np.exp2(rng.uniform(-20, np.log2(463.9), 3_000_000)).astype(np.float32)
    tiny = rng.integers(0, np.float32(2.0 ** -9).view(np.uint32), 200_000, dtype=np.uint32)
    r = np.concatenate([bits.view(np.float32), logu, tiny.view(np.float32)])
    return np.unique(r[(r >= 0) & (r < 464.0)])


def test_e4m3_encode_matches_torch_below_464():
    r = _e4m3_probe_values()
    got = oracle.e4m3_encode(r)
    want = _torch_e4m3_bytes(r)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (r[bad[:8]], got[bad[:8]], want[bad[:8]])


def test_e4m3_saturates():
    r = np.array([448.0, 448.5, 463.99, 464.0, 480.0, 1e6, 3e38, np.inf], dtype=np.float32)
    assert (oracle.e4m3_encode(r) == 0x7E).all()


def test_e8m0_defining_inequality():
    rng = np.random.default_rng(9)
    bits = rng.integers(1, 0x7F800000, 2_000_000, dtype=np.uint32)
    amax = bits.view(np.float32)
    e = np.array([oracle.e8m0_exponent(float(a)) for a in amax[:200_000]])
    a64 = amax[:200_000].astype(np.float64)
    free = e > -127
    assert (np.ldexp(1.0, e[free] + 2) <= a64[free]).all()
    assert (a64[free] < np.ldexp(1.0, e[free] + 3)).all()
    # clamped only where floor(log2 amax) - 2 < -127
    assert (a64[~free] < 2.0 ** -124).all()
    assert oracle.e8m0_exponent(0.0) == -127
    assert oracle.e8m0_exponent(float(np.float32(2.0 ** -149))) == -127
    assert oracle.e8m0_exponent(float(np.finfo(np.float32).max)) == 125


@pytest.mark.parametrize("row", read_golden("mxfp4_worked.txt"))
def test_mxfp4_worked_examples(row):
    amax, e, byte, k, level = float(row[0]), int(row[1]), int(row[2]), int(row[3]), float(row[4])
    assert oracle.e8m0_exponent(amax) == e
    assert e + 127 == byte
    # a block whose largest element is amax: quantize it and read the code back
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 3] = amax
    x[0, 4] = -amax
    codes, scales, _ = oracle.quantize(x, "mxfp4")
    assert scales[0, 0] == byte
    c = oracle.unpack_codes(codes)[0]
    assert c[3] == k and c[4] == (8 | k)
    assert oracle.E2M1_LEVELS[k] == level
