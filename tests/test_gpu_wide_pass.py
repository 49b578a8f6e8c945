"""The wide single pass of a computed tensor scale: contiguous BF16 row
operands past the reach of the plain single pass (more than 2^24 elements),
one 1024-lane workgroup per compute unit, with part of each lane's units held
in registers and LDS and the rest read a second time.  Byte parity with the
oracle and with the two-pass path, at unit counts per lane that leave the
LDS slots partly used, that stream an odd and an even number of units, and
with a ragged last round; with the waits cut to zero (the workgroups then
recompute the partial maxima they do not see posted), and beside long
kernels on another stream.  A strided operand (row pitch above the width)
takes the two-pass path and is checked too.  The two-pass path is selected
by a workspace too small for the slot exchange."""
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


# With 256 workgroups of 1024 lanes (one per compute unit) a lane takes
# ceil(units / 262144) units of 32 elements; with the RHT it holds 3 in
# registers and 2 in LDS, without it 4 and 2:
#   (4104, 4128): 3 units per lane (the held ones only, LDS slots unused);
#   (4096, 8192): 4 per lane; (6144, 8192): 6 per lane (with the RHT one
#     unit streamed, read in the held-unit loop of the first pass);
#   (7168, 8192): 7 per lane; (8192, 8192): 8 per lane (3 streamed with the
#     RHT, 2 without); (8256, 8224): 9 per lane, the last round ragged.
WIDE_SHAPES = [(4104, 4128), (4096, 8192), (6144, 8192), (7168, 8192), (8192, 8192),
               (8256, 8224)]


@pytest.mark.parametrize("shape", WIDE_SHAPES)
@pytest.mark.parametrize("fmt,rounding,rht", [("nvfp4", "rtne", True), ("nvfp4", "sr", True),
                                              ("nvfp4", "rtne", False), ("ufp4", "rtne", True),
                                              ("e2m1_cap2", "sr", False)])
def test_wide_pass_matches_oracle_and_two_pass(shape, fmt, rounding, rht):
    x = _bf16(shape, 800 + shape[1] % 97, "outlier_cols")
    note("wide pass %s %s rht=%s %s" % (fmt, rounding, rht, shape))
    quantize_both(x, fmt, "row", rounding, rht, 7, 11)
    xd = to_device(x)
    two = torch.empty(TWO_PASS_WS, dtype=torch.uint8, device=DEV)
    a = _run(xd, fmt, rounding, rht, None)
    b = _run(xd, fmt, rounding, rht, two)
    assert_bytes_equal(a[0], b[0], "codes wide vs two-pass")
    assert_bytes_equal(a[1], b[1], "scales wide vs two-pass")
    assert a[2] == b[2]


def test_wide_pass_max_in_every_share():
    """The tensor maximum sits in a held unit, an LDS unit or a streamed unit
    in turn (one element of 2^20 planted in a unit of each kind of lane 0's
    units): the tensor scale is the oracle's every time."""
    shape = (8192, 8192)
    base = _bf16(shape, 901)
    stride_units = 256 * 1024
    for k in (0, 2, 3, 4, 5, 6, 7):  # held (k < 3), LDS (3, 4), streamed (k >= 5), RHT
        x = base.copy()
        u = k * stride_units + 5
        x.reshape(-1)[32 * u + 17] = workloads.to_bf16_bits(np.array([[2.0 ** 20]],
                                                                     dtype=np.float32))[0, 0]
        note("wide pass planted maximum in unit %d" % k)
        quantize_both(x, "nvfp4", "row", "rtne", True, 7, 11)


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_wide_pass_zero_wait(monkeypatch, rounding):
    """Every wait cut to zero: the workgroups compute the partial maxima
    they do not see posted, over all of a lane's units; the bytes are still
    the oracle's."""
    monkeypatch.setenv("FP4_AMAX_WAIT_US", "0")
    x = _bf16((8256, 8224), 902, "outlier_cols")
    note("wide pass zero wait %s" % rounding)
    for _ in range(2):
        quantize_both(x, "nvfp4", "row", rounding, True, 7, 11)


def test_wide_pass_beside_a_busy_stream():
    """A same-priority stream runs float32 matrix products (finite kernels,
    a few milliseconds in all) that hold compute units while the wide call
    is launched on the current stream: the oracle's bytes, and the call
    ends within the products' time plus a margin."""
    x = _bf16((8192, 8192), 903, "outlier_cols")
    xd = to_device(x)
    a = torch.randn(4096, 4096, device=DEV)
    b = torch.randn(4096, 4096, device=DEV)
    busy = torch.cuda.Stream()
    torch.cuda.synchronize()
    note("wide pass beside a busy stream")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    with torch.cuda.stream(busy):
        ev[0].record(busy)
        for _ in range(6):
            torch.mm(a, b)
        ev[1].record(busy)
    cur = torch.cuda.current_stream()
    ev[2].record(cur)
    c, s, ts = fp4.quantize(xd, "nvfp4", "row", "rtne", True, 7, 11)
    ev[3].record(cur)
    torch.cuda.synchronize()
    busy_ms = ev[0].elapsed_time(ev[1])
    call_ms = ev[2].elapsed_time(ev[3])
    note("  products %.2f ms, quantize call %.3f ms" % (busy_ms, call_ms))
    oc, osc, ots = oracle.quantize(x, "nvfp4", "row", "rtne", True, 7, 11)
    assert f32_bits(float(to_host(ts)[0])) == f32_bits(ots)
    assert_bytes_equal(to_host(s), osc, "scales beside a busy stream")
    assert_bytes_equal(to_host(c), oc, "codes beside a busy stream")
    assert call_ms < busy_ms + 20.0


def test_strided_large_operand_takes_two_pass():
    """A view with a row pitch above its width (columns 0..8191 of an
    8192 x 8320 operand) is quantized by the two-pass path: oracle bytes."""
    full = _bf16((8192, 8320), 904)
    x = np.ascontiguousarray(full[:, :8192])
    xd = to_device(full)[:, :8192]
    note("strided large operand")
    c, s, ts = fp4.quantize(xd, "nvfp4", "row", "rtne", True, 7, 11)
    torch.cuda.synchronize()
    oc, osc, ots = oracle.quantize(x, "nvfp4", "row", "rtne", True, 7, 11)
    assert f32_bits(float(to_host(ts)[0])) == f32_bits(ots)
    assert_bytes_equal(to_host(s), osc, "scales strided")
    assert_bytes_equal(to_host(c), oc, "codes strided")


@pytest.mark.parametrize("shape", [(10240, 8192), (11264, 8192)])
def test_wide_pass_threshold(shape):
    """Either side of the wide pass's reach with the RHT (5 of 10 units per
    lane held: wide; 5 of 11: two-pass): the oracle's bytes both times."""
    x = _bf16(shape, 905, "outlier_cols")
    note("wide pass threshold %s" % (shape,))
    quantize_both(x, "nvfp4", "row", "rtne", True, 7, 11)


def test_input_bytes_follow_the_path():
    """fp4_quantize_input_bytes reports the input bytes of the path the call
    takes: once for the single pass, in between for the wide pass (the units
    it does not hold are read twice), twice for the two-pass path."""
    P = fp4.make_params
    p = P("nvfp4", "row", "rtne", True)
    ws = fp4.workspace_bytes(1, 1, p)
    bf = torch.bfloat16
    n = 4096 * 4096 * 2
    assert fp4.input_bytes(4096, 4096, 4096, bf, p, ws) == n            # single pass
    assert fp4.input_bytes(4096, 4096, 4096, bf, p, TWO_PASS_WS) == 2 * n
    # FP32 rows take the single pass while they fit one resident grid
    assert fp4.input_bytes(4096, 4096, 4096, torch.float32, p, ws) in (2 * n, 4 * n)
    for rows in (8192, 10240):                                         # wide
        n = rows * 8192 * 2
        r = fp4.input_bytes(rows, 8192, 8192, bf, p, ws)
        assert n < r < 2 * n and (r - n) % 64 == 0, (rows, r)
    n = 11264 * 8192 * 2
    assert fp4.input_bytes(11264, 8192, 8192, bf, p, ws) == 2 * n        # past the wide reach
    n = 8192 * 8192 * 2
    assert fp4.input_bytes(8192, 8192, 8320, bf, p, ws) == 2 * n         # strided: two-pass
    assert fp4.input_bytes(8192, 8192, 8192, bf, P("nvfp4", "col", "rtne", True), ws) == 2 * n
    assert fp4.input_bytes(8192, 8192, 8192, bf, P("mxfp4", "row", "rtne", True), 0) == n
    assert fp4.input_bytes(8192, 8192, 8192, bf, P("nvfp4", outer=True), 0) == n
    assert fp4.input_bytes(8192, 8192, 8192, bf, P("nvfp4", ts_given=True), 0) == n
