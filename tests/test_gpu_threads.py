"""Two host threads, each with its own stream and workspace, quantizing at
the same time (single-pass, two-pass column and MX calls): every output is
the oracle's.  The library's host state is a per-process call counter (the
single-pass tags) and per-device caches behind a mutex."""
import threading

import numpy as np
import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle
import workloads
from tests.gpu_util import DEV, assert_bytes_equal, f32_bits, note, to_device, to_host

pytestmark = pytest.mark.gpu

CALLS = [("nvfp4", "row", "sr"), ("nvfp4", "col", "rtne"), ("mxfp4", "row", "rtne"),
         ("ufp4", "row", "rtne")]


def test_two_threads_two_streams():
    xs = [workloads.to_bf16_bits(workloads.small_case("outlier_cols", 1024, 1024, 40 + t))
          for t in range(2)]
    want = [[oracle.quantize(x, f, a, r, True, 3, 7) for (f, a, r) in CALLS] for x in xs]
    xds = [to_device(x) for x in xs]
    got = [[None] * len(CALLS) for _ in range(2)]
    errors = []

    def work(t):
        try:
            s = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(s):
                for rep in range(3):
                    for i, (f, a, r) in enumerate(CALLS):
                        got[t][i] = fp4.quantize(xds[t], f, a, r, True, 3, 7, stream=s)
            s.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(e)

    note("two threads, two streams")
    threads = [threading.Thread(target=work, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    for t in range(2):
        for i, (f, a, r) in enumerate(CALLS):
            c, s, ts = got[t][i]
            oc, osc, ots = want[t][i]
            assert_bytes_equal(to_host(c), oc, "thread %d %s codes" % (t, CALLS[i]))
            assert_bytes_equal(to_host(s), osc, "thread %d %s scales" % (t, CALLS[i]))
            if ots is not None:
                assert f32_bits(float(to_host(ts)[0])) == f32_bits(ots)
