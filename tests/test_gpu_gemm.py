"""GPU parity of the MXFP4 GEMM consumer (C = A · Bᵀ on gfx950 scaled
MFMA) against the oracle's float64 product of the dequantized operands.

Every product of two codes is exact and the instruction accumulates in
binary32, so the bound is the binary32 summation bound: |C - C_ref| <=
K * 2^-23 * (|A| · |B|ᵀ) (a generous form of gamma_K), plus, for BF16
output, half a BF16 unit in the last place (at most 2^-8 of |C_ref|)."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import DEV, check_gemm, note, to_device, to_host

pytestmark = pytest.mark.gpu


def _check(c_gpu, a, sa, b, sb, M, N, K, dtype, tag):
    check_gemm(c_gpu, a, sa, b, sb, M, N, K, dtype, tag)


# K = 128 x (1, 4, 9, 21, 33) steps: one step, whole and partial 16-step
# scale groups, and groups past the first
@pytest.mark.parametrize("shape", [(128, 128, 128), (256, 384, 512), (384, 256, 1152),
                                   (256, 256, 2688), (128, 384, 4224)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_random_codes(shape, dtype):
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = rng.integers(112, 142, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(112, 142, (N, K // 32), dtype=np.uint8)
    note("gemm random codes %s %s" % (shape, dtype))
    c = fp4.gemm_mx(to_device(a), to_device(sa), to_device(b), to_device(sb), out_dtype=dtype)
    torch.cuda.synchronize()
    _check(c, a, sa, b, sb, M, N, K, dtype, "random %s" % (shape,))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp4_oas"])
@pytest.mark.parametrize("rht", [False, True])
def test_quantized_operands(fmt, rht):
    """Operands straight from the GPU quantizer (row axis along K), as a
    linear layer's forward GEMM would take them."""
    M, N, K = 256, 384, 768
    x = workloads.to_bf16_bits(workloads.small_case("t3", M, K, 5))
    w = workloads.to_bf16_bits(workloads.small_case("normal", N, K, 6))
    note("gemm quantized %s rht=%s" % (fmt, rht))
    a, sa, _ = fp4.quantize(to_device(x), fmt, "row", "rtne", rht, 3, 0)
    b, sb, _ = fp4.quantize(to_device(w), fmt, "row", "rtne", rht, 3, 0)
    c = fp4.gemm_mx(a, sa, b, sb)
    torch.cuda.synchronize()
    _check(c, to_host(a), to_host(sa), to_host(b), to_host(sb), M, N, K, torch.float32,
           "quantized %s rht=%s" % (fmt, rht))


def test_leading_dimension_and_rejects():
    M, N, K = 128, 256, 256
    rng = np.random.default_rng(9)
    a = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = rng.integers(120, 134, (M, K // 32), dtype=np.uint8)
    sb = rng.integers(120, 134, (N, K // 32), dtype=np.uint8)
    big = torch.full((M, N + 64), 7.0, dtype=torch.float32, device=DEV)
    note("gemm ldc")
    fp4.gemm_mx(to_device(a), to_device(sa), to_device(b), to_device(sb), out=big[:, :N])
    torch.cuda.synchronize()
    _check(big[:, :N].contiguous(), a, sa, b, sb, M, N, K, torch.float32, "ldc")
    assert torch.all(big[:, N:] == 7.0)
    for m, n, k in ((100, 128, 128), (128, 96, 128), (128, 128, 64)):
        with pytest.raises(fp4.FP4Error):
            fp4.gemm_mx(torch.zeros((m, k // 2), dtype=torch.uint8, device=DEV),
                        torch.zeros((m, k // 32), dtype=torch.uint8, device=DEV),
                        torch.zeros((n, k // 2), dtype=torch.uint8, device=DEV),
                        torch.zeros((n, k // 32), dtype=torch.uint8, device=DEV))


def test_linear_layer_shape_sampled():
    """The forward GEMM of the linear-layer operands at full size (M = 16384
    tokens, N = 14336, K = 4096), MXFP4 + RHT; 256 sampled outputs against
    the oracle's per-element dot products."""
    M, N, K = 16384, 14336, 4096
    note("gemm linear-layer shape")
    x = workloads.student_t_bf16(M, K, 0, 4.0)
    w = workloads.normal_bf16(N, K, 2, 0.02)
    a, sa, _ = fp4.quantize(to_device(x), "mxfp4", "row", "rtne", True, 0, 0)
    b, sb, _ = fp4.quantize(to_device(w), "mxfp4", "row", "rtne", True, 0, 0)
    c = fp4.gemm_mx(a, sa, b, sb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    ms = rng.integers(0, M, 16)
    ns = rng.integers(0, N, 16)
    ah, sah = to_host(a[torch.tensor(ms, device=DEV)]), to_host(sa[torch.tensor(ms, device=DEV)])
    bh, sbh = to_host(b[torch.tensor(ns, device=DEV)]), to_host(sb[torch.tensor(ns, device=DEV)])
    sub = c[torch.tensor(ms, device=DEV)][:, torch.tensor(ns, device=DEV)]
    _check(sub, ah, sah, bh, sbh, 16, 16, K, torch.float32, "linear layer sampled")
