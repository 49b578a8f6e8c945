"""Pins for the oracle's BF16 output (CPU only).

Dequantize writes FP32 or BF16; the BF16 output is the binary32 value
rounded to nearest even.  The conversion is pinned against torch's CPU
bfloat16 cast (round to nearest even) on every binary32 pattern within 512
units in the last place of each of the 65,536 BF16 rounding midpoints, on
every binary32 subnormal, and on infinities and NaNs; then end to end through
``dequantize``: its BF16 output is the torch cast of its FP32 output, with
and without the inverse RHT, and on outputs that equal chosen binary32
patterns exactly.
"""
import numpy as np
import torch

import oracle


def _torch_bf16(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _check_patterns(bits: np.ndarray):
    v = bits.view(np.float32)
    got = oracle.f32_to_bf16(v)
    want = _torch_bf16(v)
    nan_in = np.isnan(v)
    # NaN inputs: both sides give a NaN (payloads are not part of the contract)
    got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x007F) != 0)
    want_nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x007F) != 0)
    assert (got_nan[nan_in]).all() and (want_nan[nan_in]).all()
    bad = (got != want) & ~nan_in
    assert not bad.any(), "first mismatch at fp32 pattern 0x%08x: 0x%04x vs torch 0x%04x" % (
        int(bits[bad][0]), int(got[bad][0]), int(want[bad][0]))


def test_every_pattern_near_every_midpoint():
    """All 2^16 BF16 values b: the patterns b.8000 + d, |d| <= 512 (ties,
    both neighbours of every tie, and the round-up carry into the next
    binade, into infinity past the largest finite BF16, and the NaN range)."""
    d = np.arange(-512, 513, dtype=np.int64)
    for start in range(0, 1 << 16, 4096):
        b = np.arange(start, start + 4096, dtype=np.int64)
        bits = ((b[:, None] << 16) + 0x8000 + d[None, :]).astype(np.uint32).ravel()
        _check_patterns(bits)


def test_every_subnormal_and_the_specials():
    sub = np.arange(1, 1 << 23, dtype=np.uint32)
    _check_patterns(sub)
    _check_patterns(sub | np.uint32(0x80000000))
    specials = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF,
                         0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7FC00000, 0xFFC00001, 0x7F800001,
                         0x00800000, 0x007FFFFF, 0x007F8000, 0x007F7FFF], dtype=np.uint32)
    _check_patterns(specials)
    v = specials.view(np.float32)
    out = oracle.f32_to_bf16(v)
    assert out[2] == 0x7F80 and out[3] == 0xFF80          # infinities stay infinite
    assert out[4] == 0x7F80 and out[5] == 0xFF80          # past the largest BF16: overflow
    assert out[6] == 0x7F7F and out[7] == 0x7F80          # below / at the top midpoint


def test_dequantize_bf16_is_the_rounded_fp32_output():
    """Random codes and scales of every format (outer scales for the
    two-level formats, inverse RHT on and off): dequantize's BF16 output is
    the RNE cast of its FP32 output, element by element."""
    rng = np.random.default_rng(11)
    R, C = 8, 256
    for fmt in ("nvfp4", "ufp4", "mxfp4", "e2m1_cap2", "mxfp4_oas"):
        B = oracle.BLOCK[fmt]
        codes = rng.integers(0, 256, (R, C // 2), dtype=np.uint8)
        if fmt in oracle.MX:
            scales = rng.integers(0, 255, (R, C // B), dtype=np.uint8)
            ts = None
        else:
            scales = rng.integers(0, 0x7F, (R, C // B), dtype=np.uint8)
            ts = np.exp2(rng.uniform(-140, 60, (R, C // oracle.OUTER))).astype(np.float32)
        for inv in (False, True):
            f32 = oracle.dequantize(codes, scales, ts, R, C, fmt, rht=inv, rht_seed=3,
                                    inverse_rht=inv, out_dtype="f32")
            b16 = oracle.dequantize(codes, scales, ts, R, C, fmt, rht=inv, rht_seed=3,
                                    inverse_rht=inv, out_dtype="bf16")
            ok = ~np.isnan(f32)
            assert np.array_equal(b16[ok], _torch_bf16(f32)[ok]), (fmt, inv)


def test_dequantize_bf16_on_chosen_patterns():
    """Outer scale s, scale byte 0x38 (E4M3 1.0) and code 2 (level 1) give the
    value s exactly, so the BF16 output is the cast of s itself: 4096 chosen
    patterns near midpoints, subnormal, and near the overflow threshold."""
    rng = np.random.default_rng(12)
    n = 4096
    b = rng.integers(0, 0x7F80, n, dtype=np.int64)
    b[:64] = 0x7F7F                      # the largest finite BF16: midpoint goes to infinity
    b[64:256] = rng.integers(0, 0x80, 192)  # subnormal and smallest normal BF16 values
    d = rng.integers(-512, 513, n)
    d[::7] = 0                           # exact ties
    bits = ((b << 16) + 0x8000 + d).astype(np.uint32)
    bits[::2] |= np.uint32(0x80000000)   # both signs
    s = bits.view(np.float32).reshape(32, 128)
    rows, W = 32, 128 * oracle.OUTER
    codes = np.full((rows, W // 2), 0x22, dtype=np.uint8)
    scales = np.full((rows, W // 16), 0x38, dtype=np.uint8)
    f32 = oracle.dequantize(codes, scales, s, rows, W, "nvfp4", out_dtype="f32")
    assert np.array_equal(f32.view(np.uint32), np.repeat(s, oracle.OUTER, axis=1).view(np.uint32))
    b16 = oracle.dequantize(codes, scales, s, rows, W, "nvfp4", out_dtype="bf16")
    assert np.array_equal(b16, np.repeat(_torch_bf16(s.ravel()).reshape(32, 128), oracle.OUTER,
                                         axis=1))
