"""Helpers shared by the GPU tests: host<->device marshalling and the
byte-exact comparison against the oracle."""
import sys

import numpy as np
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle

DEV = "cuda:0"


def note(msg: str):
    """Name the case on stderr before a GPU step, so a fault is attributable."""
    print(msg, file=sys.stderr, flush=True)


def to_device(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    if got.shape != want.shape:
        raise AssertionError("%s: shape %s vs %s" % (what, got.shape, want.shape))
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError("%s: %d mismatching entries, first at %s: gpu %r oracle %r"
                             % (what, len(bad), i, got[i], want[i]))


def quantize_both(x: np.ndarray, fmt, axis="row", rounding="rtne", rht=False, rht_seed=0,
                  sr_seed=0, given=None, poison=0xAA, outer=False):
    """Quantize on the GPU (through the C ABI) and in the oracle; compare
    codes, scales and the tensor (or outer) scales byte for byte.  Returns
    the GPU tensors."""
    xd = to_device(x)
    rows, cols = x.shape
    cshape, sshape = fp4.output_shapes(rows, cols, fmt, axis)
    codes = torch.full(cshape, poison, dtype=torch.uint8, device=DEV)
    scales = torch.full(sshape, poison, dtype=torch.uint8, device=DEV)
    ts_out = None
    if outer:
        ts_out = torch.full(fp4.outer_shape(rows, cols, axis), float("nan"),
                            dtype=torch.float32, device=DEV)
    c, s, ts = fp4.quantize(xd, fmt, axis, rounding, rht, rht_seed, sr_seed,
                            tensor_scale=given, codes=codes, scales=scales, ts_out=ts_out,
                            outer=outer)
    torch.cuda.synchronize()
    oc, osc, ots = oracle.quantize(x, fmt, axis, rounding, rht, rht_seed, sr_seed,
                                   tensor_scale=given, outer=outer)
    tag = "%s %s %s rht=%s %s %s%s" % (fmt, axis, rounding, rht, x.dtype, x.shape,
                                       " outer" if outer else "")
    assert_bytes_equal(to_host(s), osc, "scales " + tag)
    assert_bytes_equal(to_host(c), oc, "codes " + tag)
    if outer:
        assert_bytes_equal(to_host(ts).view(np.uint32), ots.view(np.uint32), "outer scales " + tag)
    elif fmt not in fp4.NO_TENSOR_SCALE:
        assert f32_bits(float(to_host(ts)[0])) == f32_bits(ots), "tensor scale " + tag
    return c, s, ts, (oc, osc, ots)


def gemm_bound(a_codes, a_scales, b_codes, b_scales, M, N, K):
    """Binary32 summation bound of an MXFP4 GEMM against the exact product:
    K * 2^-23 * (|A| . |B|^T) (each product of two codes and two power-of-two
    scales is exact; only the order and rounding of the K-term sum differ)."""
    a = np.abs(oracle.dequantize(a_codes, a_scales, None, M, K, "mxfp4", "row")).astype(np.float64)
    b = np.abs(oracle.dequantize(b_codes, b_scales, None, N, K, "mxfp4", "row")).astype(np.float64)
    return K * 2.0 ** -23 * (a @ b.T)


def check_gemm(c_gpu, a, sa, b, sb, M, N, K, dtype, tag):
    """GPU GEMM output against the oracle's float64 product within
    gemm_bound, plus half a BF16 unit (at most 2^-8 of |C|) for BF16."""
    ref = oracle.gemm_mx(a, sa, b, sb, M, N, K)
    bound = gemm_bound(a, sa, b, sb, M, N, K)
    if dtype == torch.bfloat16:
        got = (to_host(c_gpu).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        bound = bound * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(ref)
    else:
        got = to_host(c_gpu).astype(np.float64)
    err = np.abs(got - ref)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "%s: %d entries out of bound, first %s: gpu %r ref %r bound %r" % (
        tag, len(bad), tuple(bad[0]), got[tuple(bad[0])], ref[tuple(bad[0])],
        bound[tuple(bad[0])])
