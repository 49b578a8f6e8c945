"""GPU parity on seeded random cases.

Each case draws a format, axis, rounding, RHT on or off, input type, data
kind, shape and row pitch, then compares the HIP path with the oracle byte
for byte: codes, scale bytes, the tensor scale or the outer scales, and the
dequantized output (FP32 or BF16, with or without the inverse RHT).  The
block-aligned length W runs up to 2048 and the other side from 1 to 600,
so column operands land on whole column tiles plus right and bottom strips
of every width, and row operands on single-pass grids of one or two units
per lane with ragged last workgroups.  Pitches are padded past the width so
no row starts where the previous one ends."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import assert_bytes_equal, f32_bits, note, to_device, to_host

pytestmark = pytest.mark.gpu

# NVFP4, the format of the training operands, is drawn three times as often
FORMATS = ["nvfp4", "nvfp4", "nvfp4", "mxfp4", "ufp4", "mxfp4_oas", "e2m1_cap2", "mxfp4_oas16",
           "mxfp4_mbs", "hif4"]
OUTER_OK = ("nvfp4", "ufp4", "e2m1_cap2")  # also with 128-element outer scales
N_CASES = 200


def draw_case(i):
    rng = np.random.default_rng(9000 + i)
    fmt = FORMATS[int(rng.integers(len(FORMATS)))]
    axis = "row" if rng.random() < 0.5 else "col"
    rounding = "sr" if rng.random() < 0.5 else "rtne"
    rht = bool(rng.random() < 0.6)
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    kind = workloads.SMALL_KINDS[int(rng.integers(len(workloads.SMALL_KINDS)))]
    outer = fmt in fp4.ALWAYS_OUTER or (fmt in OUTER_OK and rng.random() < 0.3)
    if outer:
        W = 128 * int(rng.integers(1, 17))
    else:
        B = fp4.BLOCK[fmt]
        W = B * int(rng.integers(1, 2048 // B + 1))
    n = int(rng.integers(1, 601))
    rows, cols = (n, W) if axis == "row" else (W, n)
    step = 8 if dtype == "bf16" else 4  # pitch in 16-byte units
    ld = -(-cols // step) * step + step * int(rng.integers(0, 3))
    return dict(fmt=fmt, axis=axis, rounding=rounding, rht=rht, dtype=dtype, kind=kind,
                outer=outer, rows=rows, cols=cols, ld=ld, rht_seed=int(rng.integers(1 << 62)),
                sr_seed=int(rng.integers(1 << 62)), data_seed=int(rng.integers(1 << 31)),
                inv=bool(rht and rng.random() < 0.7),
                out_dtype="bf16" if rng.random() < 0.5 else "f32")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    k = draw_case(i)
    rows, cols, ld = k["rows"], k["cols"], k["ld"]
    base = workloads.small_case(k["kind"], rows, ld, k["data_seed"])
    if k["dtype"] == "bf16":
        base = workloads.to_bf16_bits(base)
    x = np.ascontiguousarray(base[:, :cols])
    tag = " ".join("%s=%s" % (a, k[a]) for a in ("fmt", "axis", "rounding", "rht", "dtype",
                                                  "kind", "outer", "rows", "cols", "ld"))
    note("random case %d: %s" % (i, tag))
    xd = to_device(base)[:, :cols]
    assert xd.stride(0) == ld
    c, s, ts = fp4.quantize(xd, k["fmt"], k["axis"], k["rounding"], k["rht"], k["rht_seed"],
                            k["sr_seed"], outer=k["outer"])
    torch.cuda.synchronize()
    oc, osc, ots = oracle.quantize(x, k["fmt"], k["axis"], k["rounding"], k["rht"],
                                   k["rht_seed"], k["sr_seed"], outer=k["outer"])
    assert_bytes_equal(to_host(s), osc, "scales " + tag)
    assert_bytes_equal(to_host(c), oc, "codes " + tag)
    if k["outer"]:
        assert_bytes_equal(to_host(ts).view(np.uint32), ots.view(np.uint32), "outer " + tag)
    elif k["fmt"] not in fp4.NO_TENSOR_SCALE:
        assert f32_bits(float(to_host(ts)[0])) == f32_bits(ots), "tensor scale " + tag

    # the output pitch, like the input's, is a whole number of 16-byte units
    odt = torch.float32 if k["out_dtype"] == "f32" else torch.bfloat16
    ostep = 4 if k["out_dtype"] == "f32" else 8
    out = torch.empty((rows, -(-cols // ostep) * ostep), dtype=odt, device=xd.device)[:, :cols]
    fp4.dequantize(c, s, ts, rows, cols, k["fmt"], k["axis"], k["rht"], k["rht_seed"],
                   k["inv"], odt, out=out)
    torch.cuda.synchronize()
    want = oracle.dequantize(oc, osc, ots, rows, cols, k["fmt"], k["axis"], k["rht"],
                             k["rht_seed"], k["inv"], k["out_dtype"])
    got = np.ascontiguousarray(to_host(out))
    if odt == torch.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    assert_bytes_equal(got, want, "dequant inv=%s %s %s" % (k["inv"], k["out_dtype"], tag))
