"""The allocation-free quantize entry point (fp4_quantize_noalloc) against
fp4_quantize with a workspace of its own: byte-identical codes, scales and
tensor scale, two calls in a row (the second on a smaller operand), on the
single-pass path, the two-pass path (an operand too large for one resident
grid) and under HIP graph capture (two-pass, replayed with eager work in
between); and the call allocates no device memory through torch."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import workloads
from tests.gpu_util import DEV, assert_bytes_equal, f32_bits, note, to_device, to_host

pytestmark = pytest.mark.gpu


def _outputs(rows, cols, fmt, axis):
    cs, ss = fp4.output_shapes(rows, cols, fmt, axis)
    return (torch.full(cs, 0xAA, dtype=torch.uint8, device=DEV),
            torch.full(ss, 0xAA, dtype=torch.uint8, device=DEV),
            torch.full((1,), float("nan"), dtype=torch.float32, device=DEV))


def _both(xd, fmt, axis, rounding, rht):
    rows, cols = xd.shape
    c1, s1, t1 = _outputs(rows, cols, fmt, axis)
    c2, s2, t2 = _outputs(rows, cols, fmt, axis)
    fp4.quantize(xd, fmt, axis, rounding, rht, 5, 9, codes=c1, scales=s1, ts_out=t1)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fp4.quantize_noalloc(xd, fmt, axis, rounding, rht, 5, 9, codes=c2, scales=s2, ts_out=t2)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    tag = "%s %s %s rht=%s %s" % (fmt, axis, rounding, rht, tuple(xd.shape))
    assert_bytes_equal(to_host(c2), to_host(c1), "codes " + tag)
    assert_bytes_equal(to_host(s2), to_host(s1), "scales " + tag)
    if fmt not in fp4.NO_TENSOR_SCALE:
        assert f32_bits(float(to_host(t2)[0])) == f32_bits(float(to_host(t1)[0])), tag


# (4096, 4096): single pass, two units per lane; (1056, 352): single pass,
# ragged; (4096, 8192): too large for one resident grid, two-pass.
@pytest.mark.parametrize("shapes", [((4096, 4096), (1056, 352)), ((4096, 8192), (512, 1024))])
@pytest.mark.parametrize("fmt,rounding,rht", [("nvfp4", "rtne", True), ("nvfp4", "sr", True),
                                              ("ufp4", "rtne", False)])
def test_noalloc_matches_quantize_twice(shapes, fmt, rounding, rht):
    for i, shape in enumerate(shapes):
        note("noalloc call %d %s %s %s rht=%s" % (i, shape, fmt, rounding, rht))
        x = workloads.to_bf16_bits(workloads.small_case("outlier_cols", shape[0], shape[1],
                                                        80 + i))
        _both(to_device(x), fmt, "row", rounding, rht)


@pytest.mark.parametrize("fmt,axis", [("nvfp4", "col"), ("mxfp4", "row"), ("e2m1_cap2", "col")])
def test_noalloc_other_paths(fmt, axis):
    for i, shape in enumerate(((768, 512), (256, 256))):
        note("noalloc %s %s %s" % (fmt, axis, shape))
        x = workloads.to_bf16_bits(workloads.small_case("t3", shape[0], shape[1], 90 + i))
        _both(to_device(x), fmt, axis, "sr", True)


def test_noalloc_under_graph_capture():
    """Captured into a HIP graph the call takes the two-pass path with its
    partial maxima in the scratch array; every replay, with eager calls on
    other operands in between, equals the eager result."""
    x = workloads.to_bf16_bits(workloads.small_case("t3", 1024, 2048, 7))
    y = workloads.to_bf16_bits(workloads.small_case("normal", 512, 512, 8) * 1e3)
    xd, yd = to_device(x), to_device(y)
    ref = _outputs(1024, 2048, "nvfp4", "row")
    fp4.quantize(xd, "nvfp4", "row", "sr", True, 5, 9, codes=ref[0], scales=ref[1],
                 ts_out=ref[2])
    out = _outputs(1024, 2048, "nvfp4", "row")
    side = _outputs(512, 512, "nvfp4", "row")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    note("noalloc graph capture")
    with torch.cuda.graph(g, stream=s):
        fp4.quantize_noalloc(xd, "nvfp4", "row", "sr", True, 5, 9, codes=out[0], scales=out[1],
                             ts_out=out[2], stream=s)
    for r in range(3):
        for t in out[:2]:
            t.fill_(0x55)
        out[2].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert_bytes_equal(to_host(out[0]), to_host(ref[0]), "codes replay %d" % r)
        assert_bytes_equal(to_host(out[1]), to_host(ref[1]), "scales replay %d" % r)
        assert f32_bits(float(to_host(out[2])[0])) == f32_bits(float(to_host(ref[2])[0]))
        # eager work on the same scratch array between replays
        fp4.quantize_noalloc(yd, "nvfp4", "row", "rtne", True, 1, 2, codes=side[0],
                             scales=side[1], ts_out=side[2])
        torch.cuda.synchronize()
