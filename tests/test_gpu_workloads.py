"""GPU parity at the full sizes of the synthetic workloads, in the same
entry points and launch configuration the benchmark times.  Every output
byte is compared with the oracle (which finishes these in seconds on the
host's cores)."""
import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import assert_bytes_equal, note, quantize_both, to_device, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("key", list(workloads.WORKLOADS))
def test_workload_full_size(key):
    w = workloads.workload(key)
    cache = {}
    for call in w.calls:
        if call.tensor not in cache:
            note("generating %s/%s %s" % (key, call.tensor, w.shape(call.tensor)))
            cache[call.tensor] = w.make(call.tensor)
        x = cache[call.tensor]
        note("workload %s: %s" % (key, call))
        c, s, ts, (oc, osc, ots) = quantize_both(x, call.fmt, call.axis, call.rounding, call.rht,
                                                 call.rht_seed, call.sr_seed, outer=call.outer)
        if key == "single_fp32":
            rows, cols = x.shape
            out = fp4.dequantize(c, s, ts, rows, cols, call.fmt, call.axis, call.rht,
                                 call.rht_seed, call.rht)
            torch.cuda.synchronize()
            want = oracle.dequantize(oc, osc, ots, rows, cols, call.fmt, call.axis, call.rht,
                                     call.rht_seed, call.rht)
            assert_bytes_equal(to_host(out).view(np.uint32), want.view(np.uint32), "dequant")
        del c, s, ts, oc, osc
    cache.clear()
