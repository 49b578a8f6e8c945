"""Scalar CPU oracle for fused RHT + block-scaled FP4 quantize / dequantize.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the HIP library in ``block_scaled_bit_fp4_amd``; the C sources
here are compiled with gcc into their own shared object.

Pages cited in the C sources (summaries on gist.science):
  [UFP4]  es/paper/2606.20381  shrinkage bias and the uniform E1M2 grid
  [NGPT]  it/paper/2605.06067  normalized transformers under NVFP4
  [TJ2]   it/paper/2510.27527  TetraJet-v2 NVFP4 training
  [MXFP4] fr/paper/2603.08713  MXFP4 error reduction (OAS, MBS)
  [HIF]   es/paper/2602.12635  HiFloat formats on Ascend NPUs

Tensors cross this module as numpy arrays: BF16 is carried as ``uint16`` bit
patterns, FP32 as ``float32``.  Every function returns fresh arrays.

Parity status of each function is pinned by ``tests/test_oracle_*.py``:
E2M1 / uniform RTNE and SR rounding, E4M3 and E8M0 encodes, the RHT, the
Philox generator, the closed-form shrinkage table, round trips and the
column/row transpose invariant.  The per-block error figures and signed
biases on the synthetic workloads are reports, not pins (parity unpinned:
the pages print no values for them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_HDR = os.path.join(_HERE, "fp4_oracle.h")
_SO = os.path.join(_HERE, "libfp4_oracle.so")
_lock = threading.Lock()
_lib = None

FORMATS = {"nvfp4": 0, "mxfp4": 1, "ufp4": 2, "mxfp4_oas": 3, "e2m1_cap2": 4, "mxfp4_mbs": 5,
           "mxfp4_oas16": 6, "hif4": 7}
AXES = {"row": 0, "col": 1}
ROUNDINGS = {"rtne": 0, "sr": 1}
GRIDS = {"e2m1": 0, "uniform": 1, "e2m1_cap2": 2}
BLOCK = {"nvfp4": 16, "mxfp4": 32, "ufp4": 16, "mxfp4_oas": 32, "e2m1_cap2": 16,
         "mxfp4_mbs": 16, "mxfp4_oas16": 16, "hif4": 64}
# scale bytes per block: one, but four for HiF4 (E6M2 byte, 8 + 16 E1M0 bits)
SCALE_BYTES = {f: (4 if f == "hif4" else 1) for f in BLOCK}
ALWAYS_OUTER = ("mxfp4_mbs",)  # formats that only exist with 128-element outer scales
TS_MODES = {"compute": 0, "given": 1, "outer128": 2}
OUTER = 128  # outer block of the double-block mode
MX = ("mxfp4", "mxfp4_oas", "mxfp4_oas16")
NO_TENSOR_SCALE = MX + ("hif4",)  # every scale per block
E2M1_LEVELS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
UNIFORM_LEVELS = (0.0, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0)


class Params(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("axis", ctypes.c_int32),
        ("rounding", ctypes.c_int32),
        ("rht", ctypes.c_int32),
        ("ts_mode", ctypes.c_int32),
        ("rht_seed", ctypes.c_uint64),
        ("sr_seed", ctypes.c_uint64),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (seconds).  Returns the library path."""
    with _lock:
        fresh = os.path.exists(_SO) and os.path.getmtime(_SO) >= max(
            os.path.getmtime(_SRC), os.path.getmtime(_HDR))
        if force or not fresh:
            tmp = _SO + ".tmp%d" % os.getpid()
            cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                   "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                   _SRC, "-o", tmp, "-lm"]
            subprocess.run(cmd, check=True)
            os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f32p = ctypes.POINTER(ctypes.c_float)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.fp4r_philox4x32_10.argtypes = [ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.POINTER(ctypes.c_uint32),
                                         ctypes.POINTER(ctypes.c_uint32)]
        L.fp4r_rht_signs.argtypes = [ctypes.c_uint64]
        L.fp4r_rht_signs.restype = ctypes.c_uint16
        L.fp4r_sr_u16.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.fp4r_sr_u16.restype = ctypes.c_uint32
        L.fp4r_rht16.argtypes = [f32p, ctypes.c_uint16, ctypes.c_int, f32p]
        L.fp4r_e4m3_encode.argtypes = [ctypes.c_float]
        L.fp4r_e4m3_encode.restype = ctypes.c_uint8
        L.fp4r_e6m2_encode_n.argtypes = [f32p, i64, u8p]
        L.fp4r_e6m2_decode.argtypes = [ctypes.c_uint8]
        L.fp4r_e6m2_decode.restype = ctypes.c_float
        L.fp4r_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.fp4r_e4m3_decode.restype = ctypes.c_float
        L.fp4r_e8m0_exponent.argtypes = [ctypes.c_float]
        L.fp4r_e8m0_exponent.restype = ctypes.c_int
        L.fp4r_round8.argtypes = [ctypes.c_float]
        L.fp4r_round8.restype = ctypes.c_float
        L.fp4r_mbs_macro_scale.argtypes = [ctypes.c_float]
        L.fp4r_mbs_macro_scale.restype = ctypes.c_float
        L.fp4r_e8m0_exponent_oas.argtypes = [ctypes.c_float]
        L.fp4r_e8m0_exponent_oas.restype = ctypes.c_int
        L.fp4r_round_rtne.argtypes = [ctypes.c_float, ctypes.c_int]
        L.fp4r_round_rtne.restype = ctypes.c_int
        L.fp4r_round_sr.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_uint32]
        L.fp4r_round_sr.restype = ctypes.c_int
        L.fp4r_level.argtypes = [ctypes.c_int, ctypes.c_int]
        L.fp4r_level.restype = ctypes.c_float
        L.fp4r_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64,
                                    ctypes.POINTER(Params), u8p, u8p, f32p]
        L.fp4r_quantize.restype = ctypes.c_int
        L.fp4r_dequantize.argtypes = [u8p, u8p, f32p, i64, i64, ctypes.POINTER(Params),
                                      ctypes.c_int, vp, ctypes.c_int, i64]
        L.fp4r_dequantize.restype = ctypes.c_int
        L.fp4r_rht.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int,
                               ctypes.c_uint64, ctypes.c_int, f32p]
        L.fp4r_rht.restype = ctypes.c_int
        L.fp4r_quantize_block.argtypes = [f32p, ctypes.POINTER(Params), ctypes.c_uint8,
                                          ctypes.c_float, i64, i64, i64, u8p]
        L.fp4r_e4m3_encode_n.argtypes = [f32p, i64, u8p]
        L.fp4r_round_n.argtypes = [f32p, i64, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_uint32), u8p]
        L.fp4r_sr_u16_n.argtypes = [ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64), i64,
                                    ctypes.POINTER(ctypes.c_uint32)]
        L.fp4r_f32_to_bf16_n.argtypes = [f32p, i64, ctypes.POINTER(ctypes.c_uint16)]
        L.fp4r_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def make_params(fmt="nvfp4", axis="row", rounding="rtne", rht=False, rht_seed=0,
                sr_seed=0, ts_mode="compute") -> Params:
    return Params(FORMATS[fmt], BLOCK[fmt], AXES[axis], ROUNDINGS[rounding], int(bool(rht)),
                  TS_MODES[ts_mode], int(rht_seed) & (2**64 - 1),
                  int(sr_seed) & (2**64 - 1))


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return 0
    if x.dtype == np.float32:
        return 1
    raise TypeError("oracle takes BF16 bits (uint16) or float32, got %s" % x.dtype)


# ---------------------------------------------------------------- primitives
def philox(key: int, ctr) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().fp4r_philox4x32_10(key & 0xFFFFFFFF, (key >> 32) & 0xFFFFFFFF,
                             _ptr(c, ctypes.c_uint32), _ptr(out, ctypes.c_uint32))
    return out


def rht_signs(seed: int) -> int:
    return int(lib().fp4r_rht_signs(seed))


def sr_u16(seed: int, idx) -> np.ndarray:
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.uint64).ravel())
    out = np.zeros(idx.size, dtype=np.uint32)
    lib().fp4r_sr_u16_n(seed, _ptr(idx, ctypes.c_uint64), idx.size, _ptr(out, ctypes.c_uint32))
    return out


def rht16(a, seed: int = 0, inverse: bool = False, signs: int | None = None) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32).ravel())
    assert a.size == 16
    s = rht_signs(seed) if signs is None else signs
    out = np.zeros(16, dtype=np.float32)
    lib().fp4r_rht16(_ptr(a, ctypes.c_float), s, int(inverse), _ptr(out, ctypes.c_float))
    return out


def e4m3_encode(r) -> np.ndarray:
    r = np.ascontiguousarray(np.asarray(r, dtype=np.float32).ravel())
    out = np.zeros(r.size, dtype=np.uint8)
    lib().fp4r_e4m3_encode_n(_ptr(r, ctypes.c_float), r.size, _ptr(out, ctypes.c_uint8))
    return out


def e6m2_encode(r) -> np.ndarray:
    r = np.ascontiguousarray(np.asarray(r, dtype=np.float32).ravel())
    out = np.zeros(r.size, dtype=np.uint8)
    lib().fp4r_e6m2_encode_n(_ptr(r, ctypes.c_float), r.size, _ptr(out, ctypes.c_uint8))
    return out


def e6m2_decode(b: int) -> float:
    return float(lib().fp4r_e6m2_decode(b))


def e4m3_decode(b: int) -> float:
    return float(lib().fp4r_e4m3_decode(b))


def e8m0_exponent(amax: float) -> int:
    return int(lib().fp4r_e8m0_exponent(amax))


def e8m0_exponent_oas(amax: float) -> int:
    return int(lib().fp4r_e8m0_exponent_oas(amax))


def round_grid(m, grid="e2m1", rounding="rtne", u16=None) -> np.ndarray:
    m = np.ascontiguousarray(np.asarray(m, dtype=np.float32).ravel())
    if u16 is None:
        u16 = np.zeros(m.size, dtype=np.uint32)
    u16 = np.ascontiguousarray(np.broadcast_to(np.asarray(u16, dtype=np.uint32), m.shape))
    out = np.zeros(m.size, dtype=np.uint8)
    lib().fp4r_round_n(_ptr(m, ctypes.c_float), m.size, GRIDS[grid], ROUNDINGS[rounding],
                       _ptr(u16, ctypes.c_uint32), _ptr(out, ctypes.c_uint8))
    return out


def f32_to_bf16(v) -> np.ndarray:
    """The conversion behind dequantize's BF16 output, on an array of float32
    values; returns BF16 bit patterns (uint16)."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32).ravel())
    out = np.zeros(v.size, dtype=np.uint16)
    lib().fp4r_f32_to_bf16_n(_ptr(v, ctypes.c_float), v.size, _ptr(out, ctypes.c_uint16))
    return out


def max_threads() -> int:
    return int(lib().fp4r_max_threads())


# ------------------------------------------------------------------- tensors
def quantize(x: np.ndarray, fmt="nvfp4", axis="row", rounding="rtne", rht=False,
             rht_seed=0, sr_seed=0, tensor_scale: float | None = None, outer=False):
    """Quantize a 2-D array; returns (codes, scales, tensor_scale).

    codes: uint8 [rows_A, W/2]; scales: uint8 [rows_A, W/B]; tensor_scale is a
    float for NVFP4/UFP4 (computed, or the given one) and None for MXFP4.
    Passing ``tensor_scale`` selects the given-scale mode; ``outer=True`` the
    double-block mode, where tensor_scale is a float32 [rows_A, W/128] array
    of outer scales."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    outer = outer or fmt in ALWAYS_OUTER
    mode = "outer128" if outer else ("given" if tensor_scale is not None else "compute")
    p = make_params(fmt, axis, rounding, rht, rht_seed, sr_seed, mode)
    ra, w = (rows, cols) if axis == "row" else (cols, rows)
    codes = np.zeros((ra, w // 2), dtype=np.uint8)
    scales = np.zeros((ra, w // BLOCK[fmt] * SCALE_BYTES[fmt]), dtype=np.uint8)
    if outer:
        ts = np.zeros((ra, max(w // OUTER, 1)), dtype=np.float32)
    else:
        ts = np.array([tensor_scale if tensor_scale is not None else 0.0], dtype=np.float32)
    rc = lib().fp4r_quantize(x.ctypes.data, _dtype_code(x), rows, cols, cols, ctypes.byref(p),
                             _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                             _ptr(ts, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    if fmt in NO_TENSOR_SCALE:
        return codes, scales, None
    return codes, scales, (ts[:, : w // OUTER] if outer else float(ts[0]))


def round8(x: float) -> float:
    """A binary32 value rounded to 8 fraction bits (ties to even)."""
    return float(lib().fp4r_round8(float(x)))


def mbs_macro_scale(amax: float) -> float:
    """MBS-Static macro scale of a 128-element piece: round8(amax / 6)."""
    return float(lib().fp4r_mbs_macro_scale(float(amax)))


def dequantize(codes, scales, tensor_scale, rows, cols, fmt="nvfp4", axis="row", rht=False,
               rht_seed=0, inverse_rht=False, out_dtype="f32") -> np.ndarray:
    """Rebuild x.  tensor_scale: a float, or the [rows_A, W/128] outer-scale
    array of the double-block mode."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    outer = isinstance(tensor_scale, np.ndarray) and tensor_scale.ndim == 2
    p = make_params(fmt, axis, "rtne", rht, rht_seed, 0, "outer128" if outer else "given")
    if outer:
        ts = np.ascontiguousarray(tensor_scale, dtype=np.float32)
    else:
        ts = np.array([tensor_scale if tensor_scale is not None else 0.0], dtype=np.float32)
    out = np.zeros((rows, cols), dtype=np.float32 if out_dtype == "f32" else np.uint16)
    rc = lib().fp4r_dequantize(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                               _ptr(ts, ctypes.c_float), rows, cols, ctypes.byref(p),
                               int(inverse_rht), out.ctypes.data,
                               1 if out_dtype == "f32" else 0, cols)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def rht(x: np.ndarray, axis="row", seed=0, inverse=False) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    y = np.zeros((rows, cols), dtype=np.float32)
    rc = lib().fp4r_rht(x.ctypes.data, _dtype_code(x), rows, cols, cols, AXES[axis], seed,
                        int(inverse), _ptr(y, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def quantize_block(y, fmt, rounding, scale_byte, tensor_scale, row_a, col_a0, W, sr_seed=0):
    """Codes (one per byte) of one block of transformed values with a forced scale byte."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32).ravel())
    assert y.size == BLOCK[fmt]
    p = make_params(fmt, "row", rounding, False, 0, sr_seed, "given")
    out = np.zeros(y.size, dtype=np.uint8)
    lib().fp4r_quantize_block(_ptr(y, ctypes.c_float), ctypes.byref(p), scale_byte,
                              tensor_scale or 0.0, row_a, col_a0, W, _ptr(out, ctypes.c_uint8))
    return out


def gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, fmt="mxfp4") -> np.ndarray:
    """C = A · Bᵀ of two MXFP4 operands quantized along K, in float64: each
    operand rebuilt element by element by ``dequantize`` (sign * L[k] *
    2^(S - 127), exact), then one float64 matrix product.  The plain
    definition of the GEMM the [UFP4] page's single-GEMM diagnostics and the
    [MXFP4] page's GEMM kernels consume ("Diagnosticos de Cuantizacion y
    GEMM"; "4. Resultats Experimentaux")."""
    a = dequantize(a_codes, a_scales, None, M, K, fmt, "row").astype(np.float64)
    b = dequantize(b_codes, b_scales, None, N, K, fmt, "row").astype(np.float64)
    return a @ b.T


# ------------------------------------------------------------ unpack helpers
def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[R, W/2] packed bytes -> [R, W] 4-bit codes (even column = low nibble)."""
    lo = codes & 0x0F
    hi = codes >> 4
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
