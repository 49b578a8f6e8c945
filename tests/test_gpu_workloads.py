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
from tests.gpu_util import assert_bytes_equal, check_gemm, note, quantize_both, to_device, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _dual_full(x, call):
    """A dual-output call against the oracle's two single-axis quantizations."""
    (cr, sr_, tr), (cc, sc, tc) = fp4.quantize_dual(to_device(x), call.fmt, call.rounding,
                                                    call.rht, call.rht_seed, call.sr_seed,
                                                    outer=call.outer)
    torch.cuda.synchronize()
    for axis, (c, s, t) in (("row", (cr, sr_, tr)), ("col", (cc, sc, tc))):
        oc, osc, ots = oracle.quantize(x, call.fmt, axis, call.rounding, call.rht, call.rht_seed,
                                       call.sr_seed, outer=call.outer)
        assert_bytes_equal(to_host(s), osc, "dual scales " + axis)
        assert_bytes_equal(to_host(c), oc, "dual codes " + axis)
        if call.outer:
            assert_bytes_equal(to_host(t).view(np.uint32), ots.view(np.uint32), "dual outer")
        elif call.fmt not in fp4.NO_TENSOR_SCALE:
            assert to_host(t).view(np.uint32)[0] == np.float32(ots).view(np.uint32)


def _gemm_full(key, w):
    """A GEMM workload: every operand quantization byte-exact at full size,
    then each GEMM in the benchmark's configuration (BF16 out) with 256
    sampled outputs against the oracle's per-element dot products."""
    cache, ops = {}, {}
    for gm in w.gemms:
        for op in (gm.a, gm.b):
            if op in ops:
                continue
            t, axis, rounding, sr_seed = op
            if t not in cache:
                note("generating %s/%s" % (key, t))
                cache[t] = w.make(t)
            note("workload %s: %s %s %s %s rht=%s" % (key, t, w.fmt, axis, rounding, w.rht))
            # quantize_both compares codes and scales byte for byte
            c, s, _ts, (oc, osc, _ots) = quantize_both(cache[t], w.fmt, axis, rounding, w.rht, 0,
                                                       sr_seed)
            ops[op] = (c, s, oc, osc)
    rng = np.random.default_rng(7)
    for gm in w.gemms:
        (ac, asc, oac, oasc), (bc, bsc, obc, obsc) = ops[gm.a], ops[gm.b]
        M, N, K = ac.shape[0], bc.shape[0], 2 * ac.shape[1]
        note("workload %s: %s GEMM %dx%dx%d" % (key, gm.name, M, N, K))
        out = torch.empty((M, N), dtype=torch.bfloat16, device=ac.device)
        fp4.gemm_mx(ac, asc, bc, bsc, out=out)
        torch.cuda.synchronize()
        ms, ns = rng.integers(0, M, 16), rng.integers(0, N, 16)
        sub = out[torch.tensor(ms, device=out.device)][:, torch.tensor(ns, device=out.device)]
        check_gemm(sub, oac[ms], oasc[ms], obc[ns], obsc[ns], 16, 16, K, torch.bfloat16,
                   "%s %s sampled" % (key, gm.name))
        del out


@pytest.mark.parametrize("key", list(workloads.WORKLOADS))
def test_workload_full_size(key):
    w = workloads.workload(key)
    if isinstance(w, workloads.GemmWorkload):
        _gemm_full(key, w)
        return
    cache = {}
    for call in w.calls:
        if call.tensor not in cache:
            note("generating %s/%s %s" % (key, call.tensor, w.shape(call.tensor)))
            cache[call.tensor] = w.make(call.tensor)
        x = cache[call.tensor]
        note("workload %s: %s" % (key, call))
        if call.axis == "both":
            _dual_full(x, call)
            continue
        if call.op == "rht":
            y = fp4.rht(to_device(x), call.axis, call.rht_seed)
            torch.cuda.synchronize()
            want = oracle.rht(x, call.axis, call.rht_seed)
            assert_bytes_equal(to_host(y).view(np.uint32), want.view(np.uint32), "rht")
            continue
        c, s, ts, (oc, osc, ots) = quantize_both(x, call.fmt, call.axis, call.rounding, call.rht,
                                                 call.rht_seed, call.sr_seed, outer=call.outer)
        if key == "single_fp32" or call.op == "dequantize":
            rows, cols = x.shape
            bf16 = call.op == "dequantize" and call.out_dtype == "bf16"
            out = fp4.dequantize(c, s, ts, rows, cols, call.fmt, call.axis, call.rht,
                                 call.rht_seed, call.rht,
                                 torch.bfloat16 if bf16 else torch.float32)
            torch.cuda.synchronize()
            want = oracle.dequantize(oc, osc, ots, rows, cols, call.fmt, call.axis, call.rht,
                                     call.rht_seed, call.rht, "bf16" if bf16 else "f32")
            got = to_host(out)
            if not bf16:
                got, want = got.view(np.uint32), want.view(np.uint32)
            assert_bytes_equal(got, want, "dequant")
        del c, s, ts, oc, osc
    cache.clear()
