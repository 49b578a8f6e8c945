"""Prepared calls (arguments marshalled once, then only the C call): the
bytes of the oracle, over several launches into the same buffers, for a
single-pass, an MX, an outer-scale and a column quantize, and for the
dequantize with the inverse RHT."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import DEV, assert_bytes_equal, f32_bits, note, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,axis,rounding,outer", [("nvfp4", "row", "sr", False),
                                                     ("mxfp4", "row", "rtne", False),
                                                     ("nvfp4", "row", "rtne", True),
                                                     ("ufp4", "col", "rtne", False)])
def test_prepared_quantize_and_dequantize(fmt, axis, rounding, outer):
    rows, cols = 512, 768
    x = workloads.to_bf16_bits(workloads.small_case("outlier_cols", rows, cols, 31))
    xd = to_device(x)
    cs, ss = fp4.output_shapes(rows, cols, fmt, axis)
    codes = torch.empty(cs, dtype=torch.uint8, device=DEV)
    scales = torch.empty(ss, dtype=torch.uint8, device=DEV)
    ts = torch.empty(fp4.outer_shape(rows, cols, axis) if outer else (1,), dtype=torch.float32,
                     device=DEV)
    p = fp4.make_params(fmt, axis, rounding, True, 5, 9, outer=outer)
    nws = fp4.workspace_bytes(rows, cols, p)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV) if nws else None
    stream = torch.cuda.current_stream()
    q = fp4.prepare_quantize(xd, fmt, axis, rounding, True, 5, 9, codes, scales, ts, ws,
                             stream, outer=outer)
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    dq = fp4.prepare_dequantize(codes, scales, ts if fmt not in fp4.NO_TENSOR_SCALE else None,
                                rows, cols, fmt, axis, True, 5, True, y, stream)
    oc, osc, ots = oracle.quantize(x, fmt, axis, rounding, True, 5, 9, outer=outer)
    want = oracle.dequantize(oc, osc, ots, rows, cols, fmt, axis, True, 5, True, "bf16")
    note("prepared %s %s %s outer=%s" % (fmt, axis, rounding, outer))
    for rep in range(3):
        q()
        dq()
        torch.cuda.synchronize()
        assert_bytes_equal(to_host(codes), oc, "codes rep %d" % rep)
        assert_bytes_equal(to_host(scales), osc, "scales rep %d" % rep)
        if fmt not in fp4.NO_TENSOR_SCALE:
            got_ts = to_host(ts).view(np.uint32)
            want_ts = np.asarray(ots, dtype=np.float32).reshape(got_ts.shape).view(np.uint32)
            assert np.array_equal(got_ts, want_ts), "tensor scale rep %d" % rep
        assert_bytes_equal(to_host(y), want, "dequantize rep %d" % rep)


def test_prepared_calls_need_their_buffers():
    xd = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    c = torch.empty((64, 32), dtype=torch.uint8, device=DEV)
    s = torch.empty((64, 4), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        fp4.prepare_quantize(xd, "nvfp4", "row", "rtne", False, 0, 0, c, s, None, None)
    ts = torch.empty(1, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        fp4.prepare_quantize(xd, "nvfp4", "row", "rtne", False, 0, 0, c, s, ts, None)
