"""The single-pass row path of a computed tensor scale (row axis,
width a multiple of 32, operand small enough to stay in the registers of one
resident grid): byte parity with the oracle and with the two-pass path, at
grids of 1 and 2 units per lane, after the workspace held other bytes, with
the waits cut to zero so that workgroups compute the partial maxima they did
not see posted, and beside long kernels on another stream that hold the
compute units (not every workgroup resident at once): parity and a bounded
call time.  The two-pass path is selected by a workspace of kAmaxPartials
floats, too small for the slot exchange."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import DEV, assert_bytes_equal, f32_bits, note, quantize_both, to_device, to_host

pytestmark = pytest.mark.gpu

TWO_PASS_WS = 4096  # bytes: the amax-pass partials only


def _run(xd, fmt, rounding, rht, workspace):
    c, s, ts = fp4.quantize(xd, fmt, "row", rounding, rht, 7, 11, workspace=workspace)
    torch.cuda.synchronize()
    return to_host(c), to_host(s), f32_bits(float(to_host(ts)[0]))


def _bf16(shape, seed, kind="normal"):
    return workloads.to_bf16_bits(workloads.small_case(kind, shape[0], shape[1], seed))


# 1024-lane workgroups: (2048, 4096) one unit per lane on 256 workgroups,
# (4096, 4096) two units per lane (with and without the RHT).  (4096, 8192)
# does not fit one resident grid: both sides are the two-pass path there.
# (1056, 352): a ragged last workgroup.
@pytest.mark.parametrize("shape", [(1056, 352), (2048, 4096), (4096, 4096), (4096, 8192)])
@pytest.mark.parametrize("fmt,rounding,rht", [("nvfp4", "rtne", True), ("nvfp4", "sr", True),
                                              ("ufp4", "rtne", False), ("e2m1_cap2", "sr", True)])
def test_single_pass_matches_oracle_and_two_pass(shape, fmt, rounding, rht):
    x = _bf16(shape, 300 + shape[0] % 97)
    note("single pass %s %s rht=%s %s" % (fmt, rounding, rht, shape))
    quantize_both(x, fmt, "row", rounding, rht, 7, 11)
    xd = to_device(x)
    two = torch.empty(TWO_PASS_WS, dtype=torch.uint8, device=DEV)
    a = _run(xd, fmt, rounding, rht, None)
    b = _run(xd, fmt, rounding, rht, two)
    assert_bytes_equal(a[0], b[0], "codes single vs two-pass")
    assert_bytes_equal(a[1], b[1], "scales single vs two-pass")
    assert a[2] == b[2]


def test_stale_workspace_is_not_read_as_posted():
    """One workspace, calls on operands of very different maxima in turn, and
    a workspace filled with random bytes: each call's tensor scale is its
    own operand's."""
    shape = (512, 1024)
    ws = torch.empty(fp4.workspace_bytes(*shape, fp4.make_params("nvfp4")), dtype=torch.uint8,
                     device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(5)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=gen))
    for i, scale in enumerate([1e4, 1e-3, 1.0, 1e4]):
        a = workloads.small_case("normal", shape[0], shape[1], 40 + i) * scale
        x = workloads.to_bf16_bits(a)
        note("stale workspace call %d scale %g" % (i, scale))
        got = _run(to_device(x), "nvfp4", "rtne", True, ws)
        oc, osc, ots = oracle.quantize(x, "nvfp4", "row", "rtne", True, 7, 11)
        assert got[2] == f32_bits(ots), "tensor scale, call %d" % i
        assert_bytes_equal(got[1], osc, "scales, call %d" % i)
        assert_bytes_equal(got[0], oc, "codes, call %d" % i)


@pytest.mark.parametrize("shape", [(96, 160), (1056, 352), (512, 4096)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_zero_wait_computes_missing_partials(monkeypatch, shape, rounding):
    """With every wait cut to zero, a workgroup that finds a partial maximum
    (or the tensor maximum) not yet posted computes it from the input; the
    bytes are still the oracle's."""
    monkeypatch.setenv("FP4_AMAX_WAIT_US", "0")
    x = _bf16(shape, 60 + shape[1] % 13, "outlier_cols")
    note("zero wait %s %s" % (shape, rounding))
    for _ in range(3):
        quantize_both(x, "nvfp4", "row", rounding, True, 7, 11)


@pytest.mark.parametrize("shape", [(1056, 352), (2048, 2048)])
@pytest.mark.parametrize("rounding,rht", [("rtne", True), ("sr", True), ("rtne", False)])
def test_single_pass_fp32_input(shape, rounding, rht):
    x = workloads.small_case("normal", shape[0], shape[1], 500 + shape[1] % 89)
    note("single pass f32 %s rht=%s %s" % (rounding, rht, shape))
    quantize_both(x, "nvfp4", "row", rounding, rht, 7, 11)
    xd = to_device(x)
    two = torch.empty(TWO_PASS_WS, dtype=torch.uint8, device=DEV)
    a = _run(xd, "nvfp4", rounding, rht, None)
    b = _run(xd, "nvfp4", rounding, rht, two)
    assert_bytes_equal(a[0], b[0], "codes single vs two-pass")
    assert_bytes_equal(a[1], b[1], "scales single vs two-pass")
    assert a[2] == b[2]


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
@pytest.mark.parametrize("wait_us", [None, "1"])
def test_single_pass_beside_a_busy_stream(monkeypatch, rounding, wait_us):
    """A same-priority stream runs a sequence of float32 matrix products
    (finite kernels, a few milliseconds in all) that hold compute units while
    the single-pass call is launched on the current stream.  Workgroups that
    are not resident at first, and waits that give up (a 1 us wait forces
    the recomputation of missing partial maxima), still give the oracle's
    bytes, and the call ends within the products' time plus a margin."""
    if wait_us is not None:
        monkeypatch.setenv("FP4_AMAX_WAIT_US", wait_us)
    x = _bf16((4096, 4096), 77, "outlier_cols")
    xd = to_device(x)
    a = torch.randn(4096, 4096, device=DEV)
    b = torch.randn(4096, 4096, device=DEV)
    busy = torch.cuda.Stream()
    torch.cuda.synchronize()
    note("single pass beside a busy stream: %s wait=%s" % (rounding, wait_us))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    with torch.cuda.stream(busy):
        ev[0].record(busy)
        for _ in range(6):
            torch.mm(a, b)
        ev[1].record(busy)
    cur = torch.cuda.current_stream()
    ev[2].record(cur)
    c, s, ts = fp4.quantize(xd, "nvfp4", "row", rounding, True, 7, 11)
    ev[3].record(cur)
    torch.cuda.synchronize()
    busy_ms = ev[0].elapsed_time(ev[1])
    call_ms = ev[2].elapsed_time(ev[3])
    note("  products %.2f ms, quantize call %.3f ms" % (busy_ms, call_ms))
    oc, osc, ots = oracle.quantize(x, "nvfp4", "row", rounding, True, 7, 11)
    assert f32_bits(float(to_host(ts)[0])) == f32_bits(ots)
    assert_bytes_equal(to_host(s), osc, "scales beside a busy stream")
    assert_bytes_equal(to_host(c), oc, "codes beside a busy stream")
    assert call_ms < busy_ms + 20.0


# Strided views (row pitch above the width): unit u is then not element 32u
# of the buffer, and the kernel divides by the units per row; one and two
# units per lane, and a ragged last workgroup.
@pytest.mark.parametrize("shape,pitch", [((1056, 352), 384), ((2048, 4096), 4160),
                                         ((4096, 4096), 4128)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_single_pass_strided_rows(shape, pitch, rounding):
    full = _bf16((shape[0], pitch), 500 + shape[0] % 89, "outlier_cols")
    x = np.ascontiguousarray(full[:, :shape[1]])
    note("single pass strided %s pitch %d %s" % (shape, pitch, rounding))
    xd = to_device(full)[:, :shape[1]]
    two = torch.empty(TWO_PASS_WS, dtype=torch.uint8, device=DEV)
    a = _run(xd, "nvfp4", rounding, True, None)
    b = _run(xd, "nvfp4", rounding, True, two)
    oc, osc, ots = oracle.quantize(x, "nvfp4", "row", rounding, True, 7, 11)
    assert a[2] == f32_bits(ots)
    assert_bytes_equal(a[1], osc, "scales strided single pass")
    assert_bytes_equal(a[0], oc, "codes strided single pass")
    assert_bytes_equal(a[0], b[0], "codes single vs two-pass")
    assert a[2] == b[2]
