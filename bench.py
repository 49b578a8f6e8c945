#!/usr/bin/env python3
"""Benchmark of the fused RHT + FP4 quantize path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input: every
quantize call of the workload (default: the training operands of one linear
layer at hidden 4096, FFN 14336 and 16384 tokens -- X and W along rows, dY
along columns with stochastic rounding and X along columns, 16-point RHT +
NVFP4 with a computed tensor scale; `--workload activation` is the 4096 x
4096 activation, RTNE and SR).  Inputs are resident in device memory before
timing starts.  W untimed warmup steps, then exactly K steps between device
synchronizations, timed with HIP events on the stream the kernels run on.
Prints one JSON line.

`value` is input GB/s over the whole step (bytes of BF16 input of every call
/ step time), warm: the same tensors are quantized every step, so inputs of
up to 256 MB may be partly served from the MALL.  `config.cold_per_call_us`
times each call after reading a 512 MiB buffer, which evicts L2 and MALL
(`cold_input_gbs` is the step rate from those times).  `roofline` covers the
dominant call: its algorithmic bytes (input + codes + scale bytes + 4-byte
tensor scale) over its mean duration, against the 8 TB/s HBM peak.
`cpu_baseline` times the scalar oracle on the host on a bounded sample of
the same workload.  Beside the per-call fractions of the 8 TB/s peak
(single-read algorithmic bytes, bytes as moved with the input counted as
often as the chosen path reads it, counter-measured bytes) the line carries the rate of a plain
device copy (`copy_ceiling_gbs`, the practical ceiling) and, for the
workloads with a fused RHT, the plain / fused / unfused quantize times of
the first operand (the ratio the shrinkage-bias page reports in
"Eficiencia").  The 256x256 FP32 and 8192x28672 workloads add their error
reports (per-block error, signed errors, SQNR, flush-to-zero rate) from the
GPU outputs, checked against the same report on the oracle's outputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "fused RHT+FP4 quantize GB/s (BF16 in) at 1 GPU; % of HBM peak"
KERNEL_SOURCES = ["block_scaled_bit_fp4_amd/csrc/" + f for f in (
    "fp4_quantize.h", "fp4_quantize_nvfp4.hip", "fp4_quantize_mxfp4.hip", "fp4_quantize_ufp4.hip",
    "fp4_quantize_mxfp4_oas.hip", "fp4_quantize_e2m1_cap2.hip", "fp4_quantize_mxfp4_mbs.hip",
    "fp4_quantize_mxfp4_oas16.hip", "fp4_quantize_hif4.hip", "fp4_dequant.hip", "fp4_tiles.h",
    "fp4_device.h")]
MX = ("mxfp4", "mxfp4_oas", "mxfp4_oas16")
NO_TS = MX + ("hif4",)  # formats with no tensor or outer scale


GEMM_SOURCES = ["block_scaled_bit_fp4_amd/csrc/fp4_gemm.hip"]


def kernel_source_hash(workload: str = "") -> str:
    """Hash of the kernel sources a workload's counters depend on (the GEMM
    kernel for the GEMM workload, the quantize and dequantize kernels for
    the others)."""
    h = hashlib.sha256()
    for f in (GEMM_SOURCES if workload == "gemm_mx" else KERNEL_SOURCES):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(rows: int, cols: int, fmt: str, in_bytes: int, outer: bool = False,
                      outputs: int = 1) -> int:
    """Bytes the method must move once: the input, the packed codes, one
    scale byte per block, and for the two-level formats the FP32 tensor
    scale, or one FP32 outer scale per 128 elements (double block); a
    dual-output call reads the input once and writes two sets."""
    n = rows * cols
    if fmt in MX:
        return n * in_bytes + outputs * (n // 2 + n // (16 if fmt == "mxfp4_oas16" else 32))
    if fmt == "hif4":  # a 4-byte scale word per 64 elements, no tensor scale
        return n * in_bytes + outputs * (n // 2 + n // 16)
    return n * in_bytes + outputs * (n // 2 + n // 16 + (4 * (n // 128) if outer else 4))


def call_label(c) -> str:
    if c.op == "rht":
        return "%s rht %s" % (c.tensor, c.axis)
    lab = "%s %s %s %s rht=%s%s" % (c.tensor, c.fmt, c.axis, c.rounding, c.rht,
                                    " outer128" if c.outer else "")
    return lab if c.op == "quantize" else "%s dequantize to %s%s" % (
        lab, c.out_dtype, " (inverse RHT)" if c.rht else "")


def op_bytes(c, rows: int, cols: int, in_bytes: int) -> int:
    """Algorithmic bytes of one call of any operation."""
    n = rows * cols
    if c.op == "rht":
        return n * in_bytes + n * 4
    if c.op == "dequantize":
        q = algorithmic_bytes(rows, cols, c.fmt, 0, c.outer)  # codes, scales, tensor scale
        return q + n * (2 if c.out_dtype == "bf16" else 4)
    return algorithmic_bytes(rows, cols, c.fmt, in_bytes, c.outer, 2 if c.axis == "both" else 1)


def moved_bytes(c, rows: int, cols: int, in_bytes: int, reads=None) -> int:
    """Bytes the chosen algorithm moves: the algorithmic bytes with the input
    counted as often as the path reads it.  `reads` = the library's own
    account of the input bytes a single-axis quantize call reads (once for
    the single pass, in between for the wide single pass, twice after a
    tensor-amax pass); a dual call with a computed tensor scale always takes
    its amax pass."""
    alg = op_bytes(c, rows, cols, in_bytes)
    if reads is not None:
        return alg + reads - rows * cols * in_bytes
    extra = (c.op == "quantize" and c.fmt not in MX + ("hif4",) and not c.outer)
    return alg + (rows * cols * in_bytes if extra else 0)


def traffic_for(workload: str, call_index: int):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    per = t.get("per_call_bytes")
    if not per or call_index >= len(per):
        return None
    return per[call_index]


def traffic_from_counters(workload: str, fetch_csv: str, write_csv: str, copy_mib: int,
                          commands: list) -> dict:
    """Per-call HBM bytes from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE;
    KiB per dispatch) of `bench.py --copy-mib N`: the last dispatches are the
    calls, each followed by a 1 MiB delimiter copy, then one N MiB copy whose
    readings calibrate each counter (known bytes / reported bytes).  One more
    delimiter precedes the first call."""
    import csv

    def segments(path):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        copies = [i for i, r in enumerate(rows) if "copyBuffer" in r["Kernel_Name"]]
        big = copies[-1]
        reported = float(rows[big]["Counter_Value"]) * 1024.0
        delims = [i for i in copies[:-1]]
        return rows, big, reported, delims

    import workloads
    wl = workloads.workload(workload)
    ncalls = len(wl.gemms) if isinstance(wl, workloads.GemmWorkload) else len(wl.calls)
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(workload),
           "copy_mib": copy_mib, "commands": commands}
    per = {}
    for name, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows, big, reported, delims = segments(path)
        factor = (copy_mib << 20) / reported
        # the last ncalls + 1 delimiters bracket the calls' segments
        bounds = delims[-ncalls - 1:]
        starts, ends = [b + 1 for b in bounds[:-1]], bounds[1:]
        vals, names = [], []
        for a, b in zip(starts, ends):
            seg = rows[a:b]
            vals.append(sum(float(r["Counter_Value"]) for r in seg) * 1024.0 * factor)
            names.append([r["Kernel_Name"].replace("(anonymous namespace)::", "")
                          .replace("void ", "").split("(")[0] for r in seg])
        out[name + "_factor"] = round(factor, 5)
        per[name] = vals
        out["per_call_kernels"] = names
    out["per_call_fetch_bytes"] = [int(v) for v in per["fetch"]]
    out["per_call_write_bytes"] = [int(v) for v in per["write"]]
    out["per_call_bytes"] = [int(a + b) for a, b in zip(per["fetch"], per["write"])]
    return out


def cpu_baseline(w, tensors, budget_s=12.0):
    """The oracle, as it is, on the host: whole workload steps repeated until
    ~budget_s of CPU time has passed (at least one step)."""
    import oracle
    reps, t0, nbytes = 0, time.perf_counter(), 0
    while True:
        for call in w.calls:
            x = tensors[call.tensor]
            if call.op == "rht":
                oracle.rht(x, call.axis, call.rht_seed)
            else:
                for axis in (("row", "col") if call.axis == "both" else (call.axis,)):
                    q = oracle.quantize(x, call.fmt, axis, call.rounding, call.rht,
                                        call.rht_seed, call.sr_seed, outer=call.outer)
                    if call.op == "dequantize":
                        oracle.dequantize(q[0], q[1], q[2], x.shape[0], x.shape[1], call.fmt,
                                          axis, call.rht, call.rht_seed, call.rht,
                                          "f32" if call.out_dtype == "f32" else "bf16")
            nbytes += x.size * x.itemsize
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d full step(s) of the workload (%d calls each) in %.1f s" % (
                reps, len(w.calls), dt)}


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_ceiling_gbs(dev, mib=512, reps=10) -> float:
    """Bytes moved (read + write) per second by a plain device-to-device copy
    of `mib` MiB: the practical HBM ceiling the fractions are set beside."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def fused_ratio(x, stream, reps=30):
    """NVFP4 quantize of x (row axis, RTNE, computed tensor scale) timed
    three ways: plain (no RHT), fused (the RHT inside the quantize call) and
    unfused (the standalone RHT to FP32, then the plain quantize of its
    output, which gives the same bytes as the fused call).  The
    shrinkage-bias page ("Eficiencia") reports fused ~1.06-1.07x and unfused
    ~1.4-1.6x the plain quantize on NVIDIA SM90/SM100."""
    import torch
    import block_scaled_bit_fp4_amd as fp4
    rows, cols = x.shape
    cs, ss = fp4.output_shapes(rows, cols, "nvfp4", "row")
    outs = [(torch.empty(cs, dtype=torch.uint8, device=x.device),
             torch.empty(ss, dtype=torch.uint8, device=x.device),
             torch.empty(1, dtype=torch.float32, device=x.device)) for _ in range(2)]
    ws = fp4.new_workspace(rows, cols, fp4.make_params("nvfp4"), x.device)
    y = torch.empty((rows, cols), dtype=torch.float32, device=x.device)

    def q(inp, rht, o):
        fp4.quantize(inp, "nvfp4", "row", "rtne", rht, 0, 0, codes=o[0], scales=o[1],
                     ts_out=o[2], workspace=ws, stream=stream)

    arms = {"plain": lambda: q(x, False, outs[0]),
            "fused": lambda: q(x, True, outs[0]),
            "unfused": lambda: (fp4.rht(x, "row", 0, out=y, stream=stream), q(y, False, outs[1]))}
    us = {}
    for name, fn in arms.items():
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        us[name] = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
    # the unfused arm's codes equal the fused call's
    arms["fused"]()
    torch.cuda.synchronize()
    same = all(bool(torch.equal(a, b)) for a, b in zip(outs[0], outs[1]))
    return {"operand": list(x.shape), "format": "nvfp4 row rtne, computed tensor scale",
            "plain_us": round(us["plain"], 2), "fused_us": round(us["fused"], 2),
            "unfused_us": round(us["unfused"], 2),
            "fused_over_plain": round(us["fused"] / us["plain"], 3),
            "unfused_over_plain": round(us["unfused"] / us["plain"], 3),
            "unfused_bytes_equal_fused": same}


def error_report(x, y, xhat, xhat_rot, d_b, block):
    """Quantization-error figures of one call (torch float64, any device).
    x: the input (original domain); y: what was quantized (x, or its RHT);
    xhat / xhat_rot: the dequantized values in the original / quantized
    domain; d_b: each element's block scale (0 where the block codes zeros),
    all of the logical operand's shape.  Readings of the pages' quantities:
      - signed errors: mean(sign(x) (xhat - x)) and mean(xhat - x) in the
        original domain; the normalized magnitude bias mean(|q| - |v|), v =
        y / d_b and q its level, over elements of blocks with d_b > 0 (the
        shrinkage-bias page, Metodologia 1);
      - gain <xhat, x> / <x, x>; SQNR 10 log10(sum x^2 / sum (xhat - x)^2);
      - flush to zero: share of nonzero y coded as zero;
      - per block (quantized domain): MSE, max |error| and signed magnitude
        mean, each at p50 / p90 / p99 / max, with the worst block."""
    import torch
    x, y, xhat, xhat_rot, d_b = (t.double() for t in (x, y, xhat, xhat_rot, d_b))
    err = xhat - x
    ok = d_b > 0
    v = torch.where(ok, y.abs() / torch.where(ok, d_b, 1.0), 0.0)
    q = torch.where(ok, xhat_rot.abs() / torch.where(ok, d_b, 1.0), 0.0)
    e_rot = xhat_rot - y
    R, W = y.shape
    blk = lambda t: t.reshape(R, W // block, block)
    mse = (blk(e_rot) ** 2).mean(-1).flatten()
    mx = blk(e_rot).abs().amax(-1).flatten()
    smag = (blk(torch.sign(y) * e_rot)).mean(-1).flatten()

    def pct(t):
        qs = torch.quantile(t.float().cpu(), torch.tensor([0.5, 0.9, 0.99]))
        return {"p50": float(qs[0]), "p90": float(qs[1]), "p99": float(qs[2]),
                "max": float(t.max())}
    nz = y != 0
    return {
        "mean_signed_error_magnitude": float((torch.sign(x) * err).mean()),
        "mean_error": float(err.mean()),
        "normalized_magnitude_bias": float((q[ok] - v[ok]).mean()) if bool(ok.any()) else None,
        "gain": float((xhat * x).sum() / (x * x).sum()),
        "sqnr_db": float(10.0 * torch.log10((x * x).sum() / (err * err).sum())),
        "flush_to_zero_rate": float(((xhat_rot == 0) & nz).sum() / max(int(nz.sum()), 1)),
        "per_block_mse": pct(mse), "per_block_max_abs_error": pct(mx),
        "per_block_signed_magnitude_mean": pct(smag),
        "worst_block_mse": {"block": int(mse.argmax()), "row": int(mse.argmax()) // (W // block),
                            "mse": float(mse.max())},
    }


def block_scales(scales, ts, fmt, block, shape):
    """Each element's decoded block scale (torch float64): E4M3 byte times the
    tensor scale (two-level formats), 2^(S - 127) (MX formats)."""
    import torch
    MX_ = ("mxfp4", "mxfp4_oas", "mxfp4_oas16")
    s = scales.to(torch.int64)
    if fmt in MX_:
        d = torch.ldexp(torch.ones_like(s, dtype=torch.float64), s - 127)
    else:
        e4 = scales.view(torch.float8_e4m3fn).double()
        d = torch.where(s == 0, 0.0, e4 * float(ts))
    return d.repeat_interleave(block, dim=1).reshape(shape)


def call_report(x_bits, x_dev, call, codes, scales, ts, oracle_out=None):
    """error_report of one call from the GPU's codes (dequantized by the
    library on the GPU) and, when oracle_out is given, the same report from
    the oracle's codes on the host; the two must agree (the bytes are
    identical; only the order of the float64 sums differs)."""
    import numpy as np
    import torch
    import block_scaled_bit_fp4_amd as fp4
    rows, cols = x_dev.shape
    B = fp4.BLOCK[call.fmt]
    xf = x_dev.float()
    y = fp4.rht(x_dev, "row", call.rht_seed) if call.rht else xf
    xr = fp4.dequantize(codes, scales, ts, rows, cols, call.fmt, "row", call.rht, call.rht_seed,
                        False, torch.float32)
    xh = fp4.dequantize(codes, scales, ts, rows, cols, call.fmt, "row", call.rht, call.rht_seed,
                        True, torch.float32) if call.rht else xr
    tsv = float(ts.item()) if ts is not None else None
    rep = error_report(xf, y, xh, xr, block_scales(scales, tsv, call.fmt, B, (rows, cols)), B)
    if oracle_out is not None:
        import oracle
        oc, osc, ots = oracle_out
        xo = torch.from_numpy(x_bits.astype(np.float32) if x_bits.dtype == np.float32
                              else oracle.bf16_bits_to_f32(x_bits))
        yo = torch.from_numpy(oracle.rht(x_bits, "row", call.rht_seed)) if call.rht else xo
        xro = torch.from_numpy(oracle.dequantize(oc, osc, ots, rows, cols, call.fmt, "row",
                                                 call.rht, call.rht_seed, False))
        xho = torch.from_numpy(oracle.dequantize(oc, osc, ots, rows, cols, call.fmt, "row",
                                                 call.rht, call.rht_seed, True)) \
            if call.rht else xro
        ro = error_report(xo, yo, xho, xro, block_scales(torch.from_numpy(osc), ots, call.fmt, B,
                                                         (rows, cols)), B)
        rep["oracle_check"] = "agrees" if _reports_close(rep, ro) else {"oracle": ro}
    return rep


def _reports_close(a, b, rtol=1e-6):
    if isinstance(a, dict):
        return all(_reports_close(a[k], b[k], rtol) for k in a)
    if isinstance(a, float) and isinstance(b, float):
        return abs(a - b) <= rtol * max(abs(a), abs(b), 1e-30)
    return a == b


# workloads whose error figures the line reports: the 256x256 FP32 tensor
# (per-block error, signed errors) and the 8192x28672 up-projection weight
# (signed bias per format)
REPORTED = ("nvfp4_fp32_256x256", "ufp4_vs_nvfp4_upproj_8192x28672")

FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak
# formats whose GEMM-level quality the GEMM workload reports through
# dequantize + a float32 GEMM (same operands, recipes and seeds)
GEMM_SQNR_FORMATS = ("nvfp4", "ufp4", "e2m1_cap2", "mxfp4", "mxfp4_oas", "mxfp4_mbs")


def gemm_bench(args, w, dev):
    """The GEMM workload: operands quantized once (outside the timed region),
    then each step runs the workload's GEMMs; value = their flops over their
    time.  Also reported: each operand's quantize time (the quantize
    overhead relative to the GEMMs), the output SQNR of every GEMM against a
    float32 product of the BF16 inputs, with and without the RHT (FP4 GEMM;
    and for every format through dequantize and a float32 GEMM), and the
    oracle's GEMM rate on a sample."""
    import numpy as np
    import torch

    import block_scaled_bit_fp4_amd as fp4

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    host = {k: w.make(k) for k in w.tensors}
    x = {k: to_dev(v) for k, v in host.items()}
    stream = torch.cuda.current_stream()

    def quant(op, rht):
        t, axis, rounding, sr_seed = op
        return fp4.quantize(x[t], w.fmt, axis, rounding, rht, 0, sr_seed)

    ops = {}
    for gm in w.gemms:
        for op in (gm.a, gm.b):
            if op not in ops:
                ops[op] = quant(op, w.rht)[:2]
    shapes, outs = [], []
    for gm in w.gemms:
        (ac, _), (bc, _) = ops[gm.a], ops[gm.b]
        M, N, K = ac.shape[0], bc.shape[0], 2 * ac.shape[1]
        shapes.append((M, N, K))
        outs.append(torch.empty((M, N), dtype=torch.bfloat16, device=dev))

    def run(i):
        gm = w.gemms[i]
        (ac, asc), (bc, bsc) = ops[gm.a], ops[gm.b]
        fp4.gemm_mx(ac, asc, bc, bsc, out=outs[i], stream=stream)

    def step():
        for i in range(len(w.gemms)):
            run(i)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    flops = [2.0 * M * N * K for M, N, K in shapes]
    value = sum(flops) / (ms_per_step * 1e-3) / 1e12

    def timed(fn, reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps

    reps = max(5, args.steps // 2)
    per_call = [timed(lambda i=i: run(i), reps) for i in range(len(w.gemms))]
    quant_us = {}
    for op in ops:
        lab = "%s %s %s" % (op[0], op[1], op[2])
        t, axis, rounding, sr_seed = op
        codes, scales = ops[op]
        quant_us[lab] = round(timed(lambda: fp4.quantize(
            x[t], w.fmt, axis, rounding, w.rht, 0, sr_seed, codes=codes, scales=scales,
            stream=stream), reps) * 1e3, 2)

    # output SQNR per path against float32 products of the BF16 inputs
    sqnr = {}
    fmt_sqnr = {f: {} for f in GEMM_SQNR_FORMATS}
    plain = {op: quant(op, False)[:2] for op in ops} if not args.no_reports else {}

    def dequantized(op, fmt, rht):
        # the operand quantized in `fmt` and dequantized exactly to float32
        # by the library (still rotated: both operands of a GEMM carry the
        # same RHT along K, which cancels in the product), as [rows, K]
        t, axis, rounding, sr_seed = op
        c, sc, ts = fp4.quantize(x[t], fmt, axis, rounding, rht, 0, sr_seed)
        R, C = x[t].shape
        v = fp4.dequantize(c, sc, ts, R, C, fmt, axis, rht, 0, False, torch.float32)
        return (v if axis == "row" else v.t()).contiguous()

    def db(c, ref, ref_e):
        err = float(((c.double() - ref.double()) ** 2).sum())
        return round(10.0 * np.log10(ref_e / err), 2) if err > 0 else None

    for gm, (M, N, K) in zip(w.gemms, shapes):
        if args.no_reports:
            break

        def operand(op):
            t, axis = op[0], op[1]
            v = x[t].float()
            return (v if axis == "row" else v.t()).contiguous()
        ref = operand(gm.a) @ operand(gm.b).t().contiguous()
        ref_e = float((ref.double() ** 2).sum())
        res = {}
        for tag, qs in (("rht", ops), ("no_rht", plain)):
            (ac, asc), (bc, bsc) = qs[gm.a], qs[gm.b]
            c = fp4.gemm_mx(ac, asc, bc, bsc, out_dtype=torch.float32)
            res[tag] = db(c, ref, ref_e)
            del c
        sqnr[gm.name] = res
        # every format through dequantize + one float32 GEMM (the formats the
        # scaled MFMA cannot take; MXFP4 again as a check on the FP4 GEMM)
        for f in GEMM_SQNR_FORMATS:
            r = {}
            for tag, rht in (("rht", True), ("no_rht", False)):
                a = dequantized(gm.a, f, rht)
                b = dequantized(gm.b, f, rht)
                c = a @ b.t().contiguous()
                r[tag] = db(c, ref, ref_e)
                del a, b, c
            fmt_sqnr[f][gm.name] = r
        del ref
        torch.cuda.empty_cache()

    if args.copy_mib:
        # Counter runs: each GEMM once, each followed by a 1 MiB delimiter
        # copy, then one copy of known size that calibrates the counters.
        small = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        small2 = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        small2.copy_(small)
        for i in range(len(w.gemms)):
            run(i)
            small2.copy_(small)
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    dom = max(range(len(w.gemms)), key=lambda i: per_call[i])
    achieved = flops[dom] / (per_call[dom] * 1e-3) / 1e12
    line = {
        "metric": "MXFP4 GEMM TFLOP/s (forward, input-gradient and weight-gradient GEMMs of one "
                  "linear layer)",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4", "data": "synthetic",
        "config": {"workload": w.name, "description": w.description,
                   "gemms": [{"name": gm.name, "M": M, "N": N, "K": K}
                             for gm, (M, N, K) in zip(w.gemms, shapes)],
                   "per_call_us": [round(m * 1e3, 2) for m in per_call],
                   "per_call_tflops": [round(f / (m * 1e-3) / 1e12, 1)
                                       for f, m in zip(flops, per_call)],
                   "quantize_us": quant_us,
                   "quantize_over_gemm": round(sum(quant_us.values()) /
                                               (sum(per_call) * 1e3), 4),
                   "output_sqnr_db": sqnr,
                   "output_sqnr_db_by_format": fmt_sqnr},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": FP4_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP4_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic_for(args.workload, dom),
                     "kernel": "call %d (%s GEMM): fp4_gemm_mx" % (dom, w.gemms[dom].name),
                     "mean_us": round(per_call[dom] * 1e3, 2)},
        "cpu_baseline": None if args.no_cpu_baseline else gemm_cpu_baseline(w, host, ops),
    }
    return line


def gemm_cpu_baseline(w, host, ops, budget_s=12.0):
    """The oracle's GEMM on the host: 64 x 64 output blocks of the forward
    GEMM (its full K), repeated for ~budget_s."""
    import oracle
    gm = w.gemms[0]
    (ac, asc), (bc, bsc) = ops[gm.a], ops[gm.b]
    a, sa = ac[:64].cpu().numpy(), asc[:64].cpu().numpy()
    b, sb = bc[:64].cpu().numpy(), bsc[:64].cpu().numpy()
    K = 2 * a.shape[1]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm_mx(a, sa, b, sb, 64, 64, K)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(reps * 2.0 * 64 * 64 * K / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "%d blocks of 64 x 64 outputs of the %s GEMM (K = %d) in %.1f s" % (
                reps, gm.name, K, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="linear_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache per-call timing (512 MiB eviction before each call)")
    ap.add_argument("--no-reports", action="store_true",
                    help="skip the fused-RHT ratio and the error reports (their extra kernels "
                         "would show in a profiler's trace)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run one device-to-device copy of this many MiB "
                         "(a known-size reference for hardware byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two counter runs")
    args = ap.parse_args()
    if args.traffic_from:
        cmd = ("cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {c} -f csv -d <dir> -o run -- python3 "
               "bench.py --workload %s --steps 2 --warmup 1 --no-cpu-baseline --no-cold "
               "--no-reports --copy-mib %d"
               % (args.workload, args.copy_mib or 256))
        t = traffic_from_counters(args.workload, args.traffic_from[0], args.traffic_from[1],
                                  args.copy_mib or 256,
                                  [cmd.format(c="FETCH_SIZE"), cmd.format(c="WRITE_SIZE")])
        path = os.path.join(ROOT, "profiles", "traffic_%s.json" % args.workload)
        with open(path, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library quantizes on one device and has no "
              "multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_bit_fp4_amd as fp4
    import workloads

    w = workloads.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if isinstance(w, workloads.GemmWorkload):
        print(json.dumps(gemm_bench(args, w, dev)), flush=True)
        return
    tensors = {}
    for call in w.calls:
        if call.tensor not in tensors:
            tensors[call.tensor] = w.make(call.tensor)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    dtensors = {k: to_dev(v) for k, v in tensors.items()}
    # preallocated outputs and workspaces, so the timed loop only launches
    stream = torch.cuda.current_stream()
    plans = []
    for call in w.calls:
        x = dtensors[call.tensor]
        rows, cols = x.shape
        dual = call.axis == "both"
        axes = ("row", "col") if dual else (call.axis,)
        p = fp4.make_params(call.fmt, axes[0], call.rounding, call.rht, call.rht_seed,
                            call.sr_seed, outer=call.outer)
        outs = []
        for axis in axes:
            cs, ss = fp4.output_shapes(rows, cols, call.fmt, axis)
            ts_shape = fp4.outer_shape(rows, cols, axis) if call.outer else (1,)
            outs.append((torch.empty(cs, dtype=torch.uint8, device=dev),
                         torch.empty(ss, dtype=torch.uint8, device=dev),
                         torch.empty(ts_shape, dtype=torch.float32, device=dev)))
        nws = (fp4.workspace_bytes_dual if dual else fp4.workspace_bytes)(rows, cols, p)
        reads = (fp4.input_bytes(rows, cols, x.stride(0), x.dtype, p, nws)
                 if call.op == "quantize" and not dual else None)
        pl = dict(call=call, x=x, outs=outs,
                  ws=torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None,
                  alg=op_bytes(call, rows, cols, x.element_size()),
                  moved=moved_bytes(call, rows, cols, x.element_size(), reads),
                  in_bytes=x.numel() * x.element_size())
        if call.op == "dequantize":   # this call's codes, made once outside the timed region
            codes, scales, ts = outs[0]
            fp4.quantize(x, call.fmt, call.axis, call.rounding, call.rht, call.rht_seed,
                         call.sr_seed, codes=codes, scales=scales, ts_out=ts, workspace=pl["ws"],
                         outer=call.outer)
            pl["y"] = torch.empty((rows, cols), device=dev, dtype=torch.bfloat16
                                  if call.out_dtype == "bf16" else torch.float32)
        elif call.op == "rht":
            pl["y"] = torch.empty((rows, cols), device=dev, dtype=torch.float32)
        # quantize and dequantize calls marshalled once: the timed loop makes
        # only the C call (the wrapper's per-call Python work would otherwise
        # leave the GPU idle between calls of a few microseconds)
        if call.op == "quantize" and not dual:
            codes, scales, ts = outs[0]
            pl["prep"] = fp4.prepare_quantize(x, call.fmt, call.axis, call.rounding, call.rht,
                                              call.rht_seed, call.sr_seed, codes, scales, ts,
                                              pl["ws"], stream, outer=call.outer)
        elif call.op == "dequantize":
            codes, scales, ts = outs[0]
            pl["prep"] = fp4.prepare_dequantize(codes, scales, ts, rows, cols, call.fmt,
                                                call.axis, call.rht, call.rht_seed, call.rht,
                                                pl["y"], stream)
        plans.append(pl)

    def run(pl):
        c = pl["call"]
        if "prep" in pl:
            pl["prep"]()
        elif c.op == "rht":
            fp4.rht(pl["x"], c.axis, c.rht_seed, out=pl["y"], stream=stream)
        elif c.op == "dequantize":
            codes, scales, ts = pl["outs"][0]
            rows, cols = pl["x"].shape
            fp4.dequantize(codes, scales, ts, rows, cols, c.fmt, c.axis, c.rht, c.rht_seed,
                           c.rht, pl["y"].dtype, out=pl["y"], stream=stream)
        elif c.axis == "both":
            fp4.quantize_dual(pl["x"], c.fmt, c.rounding, c.rht, c.rht_seed, c.sr_seed,
                              outer=c.outer, out_row=pl["outs"][0], out_col=pl["outs"][1],
                              workspace=pl["ws"], stream=stream)
        else:
            codes, scales, ts = pl["outs"][0]
            fp4.quantize(pl["x"], c.fmt, c.axis, c.rounding, c.rht, c.rht_seed, c.sr_seed,
                         codes=codes, scales=scales, ts_out=ts, workspace=pl["ws"],
                         stream=stream, outer=c.outer)

    def step():
        for pl in plans:
            run(pl)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t_wall = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    ms_per_step = e0.elapsed_time(e1) / args.steps
    in_bytes = sum(pl["in_bytes"] for pl in plans)
    value = in_bytes / (ms_per_step * 1e-3) / 1e9

    # per-call durations (events on the launch stream around each call)
    reps = max(20, args.steps // 2)
    per_call = []
    for i, pl in enumerate(plans):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            run(pl)
            b.record(stream)
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs) / reps
        per_call.append(ms)
    # the practical ceiling: a plain device copy (before the counter section
    # below, whose last copy calibrates the byte counters)
    ceiling = copy_ceiling_gbs(dev)
    # cold caches: before each call, reading a 512 MiB buffer evicts the
    # inputs from L2 and the 256 MB MALL (a read leaves no dirty lines to
    # write back during the call); only the call itself is timed
    cold_per_call = []
    if not args.no_cold:
        scratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        creps = max(10, args.steps // 10)
        for pl in plans:
            tot = 0.0
            for r in range(creps):
                torch.sum(scratch, dim=0, out=sink)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                run(pl)
                b.record(stream)
                b.synchronize()
                tot += a.elapsed_time(b)
            cold_per_call.append(tot / creps)
        del scratch
    # per call: algorithmic (single-read) bytes, bytes as moved (with the
    # amax pass's re-read) and counter-measured HBM bytes, each over the
    # call's mean duration, as fractions of the 8 TB/s peak
    def frac(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    frac_alg = [frac(pl["alg"], m) for pl, m in zip(plans, per_call)]
    frac_moved = [frac(pl["moved"], m) for pl, m in zip(plans, per_call)]
    measured = [traffic_for(args.workload, i) for i in range(len(plans))]
    frac_rocprof = [frac(t, m) if t else None for t, m in zip(measured, per_call)]
    dom = max(range(len(plans)), key=lambda i: per_call[i])
    pl = plans[dom]
    achieved = pl["alg"] / (per_call[dom] * 1e-3) / 1e9
    c = pl["call"]
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(args.workload, dom),
        "kernel": "call %d (%s): %s" % (
            dom, call_label(c), "fp4_rht" if c.op == "rht" else "fp4_dequantize"
            if c.op == "dequantize" else "fp4_quantize, quantize kernel"
            if (c.fmt in MX + ("hif4",) or c.outer) else "fp4_quantize, computed tensor scale: the single-pass "
            "kernel when the operand fits one resident grid, the wide single pass for BF16 rows while "
            "a lane holds half its units, else tensor-amax + quantize kernels"),
        "algorithmic_bytes": pl["alg"], "mean_us": round(per_call[dom] * 1e3, 2)}

    if args.copy_mib:
        # Counter runs: each call once, each followed by a 1 MiB delimiter
        # copy, then one copy of known size that calibrates the counters.
        small = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        small2 = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        small2.copy_(small)
        for pl in plans:
            run(pl)
            small2.copy_(small)
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()

    # beside the timing: the fused-RHT ratio of the first operand, and the
    # error reports of the workloads that ask for them
    c0 = plans[0]["call"]
    fused = None
    if (not args.no_reports and c0.op == "quantize" and c0.fmt == "nvfp4" and c0.rht
            and c0.axis == "row" and plans[0]["x"].dtype == torch.bfloat16):
        fused = fused_ratio(plans[0]["x"], stream)
    reports = None
    if w.name in REPORTED and not args.no_reports:
        import oracle
        reports = {}
        for pl in plans:
            c = pl["call"]
            codes, scales, ts = pl["outs"][0]
            run(pl)
            torch.cuda.synchronize()
            host = tensors[c.tensor]
            ref = oracle.quantize(host, c.fmt, c.axis, c.rounding, c.rht, c.rht_seed, c.sr_seed)
            same = (np.array_equal(codes.cpu().numpy(), ref[0]) and
                    np.array_equal(scales.cpu().numpy(), ref[1]))
            rep = call_report(host, pl["x"], c, codes, scales, None if c.fmt in NO_TS else ts,
                              ref)
            rep["gpu_bytes_equal_oracle"] = bool(same)
            reports[call_label(c)] = rep
            if c.rht:  # the same format without the RHT, for the RHT's change in SQNR
                import dataclasses
                c2 = dataclasses.replace(c, rht=False)
                q2 = fp4.quantize(pl["x"], c.fmt, "row", c.rounding, False, 0, c.sr_seed)
                reports[call_label(c2)] = call_report(host, pl["x"], c2, q2[0], q2[1],
                                                      None if c.fmt in NO_TS else q2[2])
                del q2
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, tensors)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description,
                   "tensors": {k: list(v.shape) for k, v in tensors.items()},
                   "calls": [call_label(c) for c in w.calls],
                   "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4),
                   "per_call_us": [round(m * 1e3, 2) for m in per_call],
                   "frac_alg": frac_alg, "frac_moved": frac_moved,
                   "frac_rocprof": frac_rocprof if any(frac_rocprof) else None,
                   "copy_ceiling_gbs": ceiling,
                   "frac_alg_of_copy_ceiling": [round(f * HBM_PEAK_GBS / ceiling, 4)
                                                for f in frac_alg],
                   "fused_ratio": fused, "reports": reports,
                   "wall_ms_per_step": round(wall_ms, 4),
                   "cold_per_call_us": [round(m * 1e3, 2) for m in cold_per_call] or None,
                   "cold_input_gbs": round(in_bytes / (sum(cold_per_call) * 1e-3) / 1e9, 2)
                   if cold_per_call else None},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
