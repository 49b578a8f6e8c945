"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the quantization method: it only draws
numbers with numpy's PCG64 generator and rounds them to BF16 with torch's CPU
conversion (round to nearest even).  Both the oracle and the HIP library
receive the same bytes from here.

The pages train and evaluate on public corpora and suites (OLMo-2 data,
MMLU, GSM8K, Wikitext-2, C4, ...) and on trained checkpoints; none of those
is used.  These tensors stand in for the statistics of LLM GEMM operands that
the pages discuss instead: heavy-tailed activations with a few outlier
channels, Gaussian weights with rare large entries, heavy-tailed gradients.

Tensors are returned as numpy arrays: FP32 as float32, BF16 as uint16 bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float -> BF16 bit patterns (uint16), RNE via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- tensors
def normal_f32(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cols)) * std).astype(np.float32)


def normal_bf16(rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    return to_bf16_bits(normal_f32(rows, cols, seed, std))


def student_t_bf16(rows: int, cols: int, seed: int, nu: float) -> np.ndarray:
    """Student-t with nu > 2 degrees of freedom, scaled to unit variance."""
    rng = np.random.default_rng(seed)
    t = rng.standard_t(nu, size=(rows, cols)) / math.sqrt(nu / (nu - 2.0))
    return to_bf16_bits(t.astype(np.float32))


def activation_with_outlier_channels(rows: int, cols: int, seed: int, nu: float = 3.0,
                                     frac: float = 1e-3, gain: float = 50.0) -> np.ndarray:
    """Unit-variance Student-t activation with round(frac*cols) distinct
    columns (drawn after the t-draws from the same generator) times gain."""
    rng = np.random.default_rng(seed)
    t = rng.standard_t(nu, size=(rows, cols)) / math.sqrt(nu / (nu - 2.0))
    k = max(1, int(frac * cols))
    chans = rng.choice(cols, size=k, replace=False)
    t[:, chans] *= gain
    return to_bf16_bits(t.astype(np.float32))


def weight_with_spikes(rows: int, cols: int, seed: int, std: float = 0.02,
                       frac: float = 1e-4, spike_sigmas: float = 20.0) -> np.ndarray:
    """N(0, std^2) weight with round(frac*N) distinct entries set to
    +-spike_sigmas*std (sign equiprobable), drawn after the Gaussian."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((rows, cols)) * std
    n = rows * cols
    k = int(round(frac * n))
    pos = rng.choice(n, size=k, replace=False)
    sign = np.where(rng.random(k) < 0.5, -1.0, 1.0)
    w.reshape(-1)[pos] = sign * spike_sigmas * std
    return to_bf16_bits(w.astype(np.float32))


# ---------------------------------------------------------------- workloads
@dataclass
class Call:
    """One quantize call of a workload."""
    tensor: str
    fmt: str
    axis: str = "row"     # "row", "col", or "both" (one dual-output call)
    rounding: str = "rtne"
    rht: bool = False
    rht_seed: int = 0
    sr_seed: int = 0
    outer: bool = False   # two-level formats: outer (MBS: macro) scale per 128 elements
    op: str = "quantize"  # "quantize", "dequantize" (of this call's own codes) or "rht"
    out_dtype: str = "bf16"  # dequantize output


@dataclass
class Workload:
    name: str
    description: str
    tensors: dict = field(default_factory=dict)   # name -> (rows, cols, dtype, maker)
    calls: list = field(default_factory=list)

    def make(self, name: str) -> np.ndarray:
        rows, cols, _dt, maker = self.tensors[name]
        return maker()

    def shape(self, name: str):
        rows, cols, dt, _ = self.tensors[name]
        return rows, cols, dt


def _w_single_fp32() -> Workload:
    w = Workload("nvfp4_fp32_256x256",
                 "256x256 FP32 N(0,1), seed 0: NVFP4 RTNE row axis, no RHT; then dequantize")
    w.tensors["x"] = (256, 256, "f32", lambda: normal_f32(256, 256, 0))
    w.calls = [Call("x", "nvfp4")]
    return w


def _w_activation() -> Workload:
    w = Workload("rht_nvfp4_act_4096x4096",
                 "4096x4096 BF16 Student-t(3) unit variance with 0.1% outlier columns x50: "
                 "16-point RHT + NVFP4, row axis, RTNE and SR (Philox seed 1)")
    w.tensors["x"] = (4096, 4096, "bf16", lambda: activation_with_outlier_channels(4096, 4096, 0))
    w.calls = [Call("x", "nvfp4", "row", "rtne", True, 0, 0),
               Call("x", "nvfp4", "row", "sr", True, 0, 1)]
    return w


def _w_mx_weight() -> Workload:
    w = Workload("mxfp4_weight_8192x8192",
                 "8192x8192 BF16 N(0, 0.02^2): MXFP4 RTNE, row and column axis, RHT off and on")
    w.tensors["w"] = (8192, 8192, "bf16", lambda: normal_bf16(8192, 8192, 0, 0.02))
    w.calls = [Call("w", "mxfp4", ax, "rtne", r, 0, 0)
               for ax in ("row", "col") for r in (False, True)]
    return w


def _w_up_proj() -> Workload:
    w = Workload("ufp4_vs_nvfp4_upproj_8192x28672",
                 "8192x28672 BF16 N(0, 0.02^2) with 0.01% entries at +-20 sigma: "
                 "uniform grid vs NVFP4 vs E2M1 cut at 2, all with RHT, RTNE, row axis")
    w.tensors["w"] = (8192, 28672, "bf16", lambda: weight_with_spikes(8192, 28672, 0))
    w.calls = [Call("w", "ufp4", "row", "rtne", True, 0, 0),
               Call("w", "nvfp4", "row", "rtne", True, 0, 0),
               Call("w", "e2m1_cap2", "row", "rtne", True, 0, 0)]
    return w


def _w_linear_layer() -> Workload:
    w = Workload("nvfp4_rht_linear_h4096_f14336_t16384",
                 "training operands of one linear layer (hidden 4096, FFN 14336, 16384 tokens): "
                 "X and dY Student-t(4) unit variance, W N(0, 0.02^2); NVFP4 + RHT: X and W row "
                 "(forward), dY column with SR and X column (weight gradient)")
    w.tensors["X"] = (16384, 4096, "bf16", lambda: student_t_bf16(16384, 4096, 0, 4.0))
    w.tensors["dY"] = (16384, 14336, "bf16", lambda: student_t_bf16(16384, 14336, 1, 4.0))
    w.tensors["W"] = (14336, 4096, "bf16", lambda: normal_bf16(14336, 4096, 2, 0.02))
    w.calls = [Call("X", "nvfp4", "row", "rtne", True, 0, 0),
               Call("W", "nvfp4", "row", "rtne", True, 0, 0),
               Call("dY", "nvfp4", "col", "sr", True, 0, 1),
               Call("X", "nvfp4", "col", "rtne", True, 0, 0)]
    return w


def _w_activation_outer() -> Workload:
    w = _w_activation()
    w.name = "rht_nvfp4_double_block_act_4096x4096"
    w.description = ("the 4096x4096 activation above, NVFP4 + RHT with double-block scales "
                     "(FP32 outer scale per 128 elements, no tensor amax pass), RTNE and SR")
    for c in w.calls:
        c.outer = True
    return w


def _w_linear_layer_outer() -> Workload:
    w = _w_linear_layer()
    w.name = "nvfp4_rht_double_block_linear_h4096_f14336_t16384"
    w.description = ("the linear-layer operands above with double-block NVFP4 scales (FP32 outer "
                     "scale per 128 elements of each A-row, no tensor amax pass)")
    for c in w.calls:
        c.outer = True
    return w


def _w_mx_weight_oas() -> Workload:
    w = _w_mx_weight()
    w.name = "mxfp4_oas_weight_8192x8192"
    w.description = ("8192x8192 BF16 N(0, 0.02^2): MXFP4 with overflow-aware scales, RTNE, row "
                     "and column axis, RHT off and on")
    for c in w.calls:
        c.fmt = "mxfp4_oas"
    return w


def _w_mx_weight_oas16() -> Workload:
    w = _w_mx_weight()
    w.name = "mxfp4_oas16_weight_8192x8192"
    w.description = ("8192x8192 BF16 N(0, 0.02^2): MXFP4 with overflow-aware scales on 16-element "
                     "blocks (E8M0 per 16), RTNE, row and column axis, RHT off and on")
    for c in w.calls:
        c.fmt = "mxfp4_oas16"
    return w


def _w_hif4_weight() -> Workload:
    w = _w_mx_weight()
    w.name = "hif4_weight_8192x8192"
    w.description = ("8192x8192 BF16 N(0, 0.02^2): HiF4 (E6M2 per 64, E1M0 per 8 and per 4, E1M2 "
                     "elements), RTNE, row and column axis, RHT off and on")
    for c in w.calls:
        c.fmt = "hif4"
    return w


def _w_mx_weight_mbs() -> Workload:
    w = _w_mx_weight()
    w.name = "mxfp4_mbs_weight_8192x8192"
    w.description = ("8192x8192 BF16 N(0, 0.02^2): MXFP4 with static macro-block scaling (macro "
                     "scale per 128, E8M0 per 16), RTNE, row and column axis, RHT off and on")
    for c in w.calls:
        c.fmt = "mxfp4_mbs"
        c.outer = True
    return w


def _w_linear_layer_dual() -> Workload:
    w = _w_linear_layer()
    w.name = "nvfp4_rht_dual_linear_h4096_f14336_t16384"
    w.description = ("the linear-layer operands above; X quantized along rows and columns by one "
                     "dual-output call (same outputs as the separate X row and X column calls)")
    w.calls = [Call("X", "nvfp4", "both", "rtne", True, 0, 0),
               Call("W", "nvfp4", "row", "rtne", True, 0, 0),
               Call("dY", "nvfp4", "col", "sr", True, 0, 1)]
    return w


def _w_training_operands() -> Workload:
    w = _w_linear_layer()
    w.name = "nvfp4_rht_all_gemm_operands_h4096_f14336_t16384"
    w.description = ("every quantized operand of the three GEMMs of one linear layer (forward, "
                     "input gradient, weight gradient): X, W and dY each along rows and columns "
                     "by dual-output calls; NVFP4 + RHT, SR on dY")
    w.calls = [Call("X", "nvfp4", "both", "rtne", True, 0, 0),
               Call("W", "nvfp4", "both", "rtne", True, 0, 0),
               Call("dY", "nvfp4", "both", "sr", True, 0, 1)]
    return w


def _w_dequant() -> Workload:
    w = _w_linear_layer()
    w.name = "nvfp4_rht_dequant_and_rht_h4096_t16384"
    w.description = ("the 16384x4096 linear-layer activation X: NVFP4 + RHT codes (quantized once, "
                     "outside the timed region) dequantized with the inverse RHT to BF16 along "
                     "rows and along columns, double-block codes dequantized to FP32, and the "
                     "standalone forward RHT along rows (FP32 out); value counts the BF16 bytes "
                     "of X per call")
    w.tensors = {"X": w.tensors["X"]}
    w.calls = [Call("X", "nvfp4", "row", "rtne", True, 0, 0, op="dequantize"),
               Call("X", "nvfp4", "col", "rtne", True, 0, 0, op="dequantize"),
               Call("X", "nvfp4", "row", "rtne", True, 0, 0, outer=True, op="dequantize",
                    out_dtype="f32"),
               Call("X", "nvfp4", "row", op="rht")]
    return w


@dataclass
class Gemm:
    """One GEMM C = A · Bᵀ of MXFP4 operands quantized along K: each operand
    is (tensor, axis, rounding, sr_seed) of a quantize call whose A is the
    GEMM operand (axis "col" quantizes the transpose)."""
    name: str
    a: tuple
    b: tuple


@dataclass
class GemmWorkload:
    name: str
    description: str
    fmt: str
    rht: bool
    tensors: dict = field(default_factory=dict)
    gemms: list = field(default_factory=list)

    def make(self, name: str) -> np.ndarray:
        rows, cols, _dt, maker = self.tensors[name]
        return maker()


def _w_gemm_mx() -> GemmWorkload:
    lin = _w_linear_layer()
    w = GemmWorkload("mxfp4_rht_training_gemms_h4096_f14336_t16384",
                     "the three GEMMs of one linear layer (hidden 4096, FFN 14336, 16384 tokens) "
                     "on MXFP4 + RHT operands quantized along each GEMM's K (SR on dY): forward "
                     "Y = X Wᵀ, input gradient dX = dY W, weight gradient dW = dYᵀ X; BF16 out",
                     "mxfp4", True)
    w.tensors = dict(lin.tensors)
    w.gemms = [Gemm("fprop", ("X", "row", "rtne", 0), ("W", "row", "rtne", 0)),
               Gemm("dgrad", ("dY", "row", "sr", 1), ("W", "col", "rtne", 0)),
               Gemm("wgrad", ("dY", "col", "sr", 1), ("X", "col", "rtne", 0))]
    return w


WORKLOADS = {
    "single_fp32": _w_single_fp32,
    "activation": _w_activation,
    "mx_weight": _w_mx_weight,
    "up_proj": _w_up_proj,
    "linear_layer": _w_linear_layer,
    "activation_outer": _w_activation_outer,
    "linear_layer_outer": _w_linear_layer_outer,
    "mx_weight_oas": _w_mx_weight_oas,
    "mx_weight_mbs": _w_mx_weight_mbs,
    "mx_weight_oas16": _w_mx_weight_oas16,
    "hif4_weight": _w_hif4_weight,
    "linear_layer_dual": _w_linear_layer_dual,
    "training_operands": _w_training_operands,
    "dequant": _w_dequant,
    "gemm_mx": _w_gemm_mx,
}


def workload(key: str) -> Workload:
    return WORKLOADS[key]()


# ------------------------------------------------------- small random cases
def small_case(kind: str, rows: int, cols: int, seed: int) -> np.ndarray:
    """Small FP32 tensors with structure that stresses edge cases."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        a = rng.standard_normal((rows, cols))
    elif kind == "t3":
        a = rng.standard_t(3, size=(rows, cols))
    elif kind == "outlier_cols":
        a = rng.standard_normal((rows, cols))
        a[:, rng.choice(cols, size=max(1, cols // 64), replace=False)] *= 100.0
    elif kind == "wide_range":
        # magnitudes spread over ~60 binades, random signs
        a = np.exp2(rng.uniform(-40, 20, size=(rows, cols))) * rng.choice([-1.0, 1.0], (rows, cols))
    elif kind == "tiny":
        # values around the FP32/BF16 subnormal range
        a = np.exp2(rng.uniform(-140, -110, size=(rows, cols))) * rng.choice([-1.0, 1.0], (rows, cols))
    elif kind == "zeros_mixed":
        a = rng.standard_normal((rows, cols))
        a[rng.random((rows, cols)) < 0.3] = 0.0
        a[:, : min(cols, 32)] = 0.0
        a[0, 0] = -0.0
    elif kind == "grid_ties":
        # multiples of 1/8 in a narrow range: many exact ties after scaling
        a = rng.integers(-48, 49, size=(rows, cols)) / 8.0
    elif kind == "constant":
        a = np.full((rows, cols), 0.7)
    else:
        raise KeyError(kind)
    return a.astype(np.float32)


SMALL_KINDS = ("normal", "t3", "outlier_cols", "wide_range", "tiny", "zeros_mixed",
               "grid_ties", "constant")
