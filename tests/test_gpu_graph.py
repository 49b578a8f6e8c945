"""Quantize calls captured in a HIP graph (torch.cuda.graph) and replayed:
every replay must equal the eager result, with eager work and
synchronizations between replays and new input contents written in place
(the graph re-reads x through the same pointer).  The library records no
memset node: partial maxima need no initialization."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import workloads
from tests.gpu_util import DEV, note, to_device

pytestmark = pytest.mark.gpu

CASES = [  # (fmt, axis, rounding, rht, outer); axis "both" = dual call
    ("nvfp4", "row", "sr", True, False),
    ("nvfp4", "col", "rtne", True, False),
    ("ufp4", "row", "rtne", True, True),
    ("mxfp4_oas", "col", "sr", False, False),
    ("nvfp4", "both", "rtne", True, False),
]


def _inputs(seed):
    return to_device(workloads.to_bf16_bits(workloads.small_case("outlier_cols", 512, 768, seed)))


def _call(x, fmt, axis, rounding, rht, outer, outs, ws):
    if axis == "both":
        fp4.quantize_dual(x, fmt, rounding, rht, 2, 7, outer=outer, out_row=outs[0],
                          out_col=outs[1], workspace=ws)
    else:
        c, s, t = outs[0]
        fp4.quantize(x, fmt, axis, rounding, rht, 2, 7, codes=c, scales=s, ts_out=t,
                     workspace=ws, outer=outer)


def _alloc(x, fmt, axis, outer):
    rows, cols = x.shape
    outs = []
    for ax in (("row", "col") if axis == "both" else (axis,)):
        cs, ss = fp4.output_shapes(rows, cols, fmt, ax)
        ts = fp4.outer_shape(rows, cols, ax) if outer else (1,)
        outs.append((torch.full(cs, 0xAA, dtype=torch.uint8, device=DEV),
                     torch.full(ss, 0xAA, dtype=torch.uint8, device=DEV),
                     torch.full(ts, float("nan"), dtype=torch.float32, device=DEV)))
    p = fp4.make_params(fmt, "row" if axis == "both" else axis, "rtne", True, outer=outer)
    n = (fp4.workspace_bytes_dual if axis == "both" else fp4.workspace_bytes)(rows, cols, p)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
    return outs, ws


@pytest.mark.parametrize("fmt,axis,rounding,rht,outer", CASES,
                         ids=["-".join(map(str, c)) for c in CASES])
def test_graph_replays_equal_eager(fmt, axis, rounding, rht, outer):
    note("graph %s %s %s rht=%s outer=%s" % (fmt, axis, rounding, rht, outer))
    x = _inputs(1)
    outs, ws = _alloc(x, fmt, axis, outer)
    # warm up on a side stream, as torch requires before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(x, fmt, axis, rounding, rht, outer, outs, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(x, fmt, axis, rounding, rht, outer, outs, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        src = _inputs(10 + rep % 2)
        x.copy_(src)                       # new contents, same pointer
        for o in outs:                     # poison the outputs eagerly
            o[0].fill_(0x55)
            o[1].fill_(0x55)
            o[2].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_outs, ref_ws = _alloc(x, fmt, axis, outer)
        _call(x, fmt, axis, rounding, rht, outer, ref_outs, ref_ws)
        torch.cuda.synchronize()
        for (c, s, t), (rc, rs, rt) in zip(outs, ref_outs):
            assert torch.equal(c, rc), "codes, replay %d" % rep
            assert torch.equal(s, rs), "scales, replay %d" % rep
            if fmt not in fp4.MX:
                assert torch.equal(t.view(torch.int32), rt.view(torch.int32)), "scale, replay %d" % rep
