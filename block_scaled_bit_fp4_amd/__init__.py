"""MI355X (gfx950) fused RHT + block-scaled FP4 quantize / dequantize.

A thin ctypes binding over ``libfp4.so`` (the C ABI in ``include/fp4.h``).
This module only marshals arguments: it allocates outputs as torch device
tensors, passes raw pointers, sizes and the current HIP stream, and raises on
a non-zero status.  Every step of the computation runs in the HIP kernels;
there is no CPU fallback, and importing the library fails loudly when
``libfp4.so`` has not been built (``python -m block_scaled_bit_fp4_amd.build``).

Formats: ``"nvfp4"`` (E2M1, 16-element blocks, E4M3 scale, FP32 tensor
scale), ``"mxfp4"`` (E2M1, 32-element blocks, E8M0 scale), ``"ufp4"``
(uniform 0..7 grid, 16-element blocks, E4M3 scale, FP32 tensor scale),
``"mxfp4_oas"`` (MXFP4 with overflow-aware E8M0 scales), ``"e2m1_cap2"``
(E2M1 cut at magnitude 2, NVFP4's scaling with the block amax mapped to 2),
``"mxfp4_mbs"`` (static macro-block scaling: a macro scale with an 8-bit
mantissa per 128 elements over 16-element E8M0 blocks; always returns the
macro-scale array as its third result, as ``outer=True`` does),
``"mxfp4_oas16"`` (overflow-aware E8M0 scales on 16-element blocks), ``"hif4"``
(HiF4: an E6M2 scale per 64 elements refined by one-bit E1M0 factors per 8
and per 4 elements, E1M2 elements; four scale bytes per block).
The two-level formats (NVFP4, the uniform grid, the cut E2M1) also take
double-block scales (``outer=True``): one FP32 outer scale per 128 elements
of each row of the quantized operand instead of the tensor scale.

``stream`` (every call): None launches on torch's current stream; a
``torch.cuda.Stream`` launches on it, and whatever the call allocates
(outputs, the workspace, an uploaded tensor scale) is allocated with that
stream current, so torch's caching allocator does not reuse those blocks
while the kernels are queued; a raw ``hipStream_t`` handle (an int) is
accepted only when every such buffer is passed in.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp4.so")

FORMATS = {"nvfp4": 0, "mxfp4": 1, "ufp4": 2, "mxfp4_oas": 3, "e2m1_cap2": 4, "mxfp4_mbs": 5,
           "mxfp4_oas16": 6, "hif4": 7}
BLOCK = {"nvfp4": 16, "mxfp4": 32, "ufp4": 16, "mxfp4_oas": 32, "e2m1_cap2": 16,
         "mxfp4_mbs": 16, "mxfp4_oas16": 16, "hif4": 64}
# scale bytes per block: one, but four for HiF4 (E6M2 byte and 8 + 16 E1M0 bits)
SCALE_BYTES = {f: (4 if f == "hif4" else 1) for f in BLOCK}
ALWAYS_OUTER = ("mxfp4_mbs",)  # formats that exist only with 128-element macro scales
MX = ("mxfp4", "mxfp4_oas", "mxfp4_oas16")
NO_TENSOR_SCALE = MX + ("hif4",)  # every scale per block: no tensor or outer scale
OUTER = 128  # elements per outer scale (double-block mode)
TS_COMPUTE, TS_GIVEN, TS_OUTER128 = 0, 1, 2
AXES = {"row": 0, "col": 1}
ROUNDINGS = {"rtne": 0, "sr": 1}
DTYPES = {torch.bfloat16: 0, torch.float32: 1}

FP4_OK = 0
STATUS = {0: "FP4_OK", -1: "FP4_ERR_NULL", -2: "FP4_ERR_FORMAT", -3: "FP4_ERR_SHAPE",
          -4: "FP4_ERR_ALIGN", -5: "FP4_ERR_DTYPE", -6: "FP4_ERR_WORKSPACE",
          -7: "FP4_ERR_DEVICE"}

# every symbol include/fp4.h declares
EXPORTS = ("fp4_workspace_bytes", "fp4_quantize", "fp4_dequantize", "fp4_rht",
           "fp4_rht_signs", "fp4_status_str", "fp4_workspace_bytes_dual", "fp4_quantize_dual",
           "fp4_gemm_mx", "fp4_quantize_noalloc", "fp4_quantize_input_bytes")


class FP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().fp4_status_str(status).decode()
        super().__init__("%s: %s (%s)" % (where, STATUS.get(status, status), msg))


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


_lib = None


def load():
    """The ctypes handle of libfp4.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp4.so is not built: run python -m block_scaled_bit_fp4_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER(Params)
        L.fp4_workspace_bytes.argtypes = [i64, i64, P]
        L.fp4_workspace_bytes.restype = sz
        L.fp4_quantize.argtypes = [vp, i32, i64, i64, i64, P, vp, vp, vp, vp, sz, vp]
        L.fp4_quantize.restype = i32
        L.fp4_quantize_noalloc.argtypes = [vp, i32, i64, i64, i64, P, vp, vp, vp, vp]
        L.fp4_quantize_noalloc.restype = i32
        L.fp4_quantize_input_bytes.argtypes = [i32, i64, i64, i64, P, sz,
                                               ctypes.POINTER(ctypes.c_int64)]
        L.fp4_quantize_input_bytes.restype = i32
        L.fp4_workspace_bytes_dual.argtypes = [i64, i64, P]
        L.fp4_workspace_bytes_dual.restype = sz
        L.fp4_quantize_dual.argtypes = [vp, i32, i64, i64, i64, P, vp, vp, vp, vp, vp, vp, vp,
                                        sz, vp]
        L.fp4_quantize_dual.restype = i32
        L.fp4_dequantize.argtypes = [vp, vp, vp, i64, i64, P, i32, vp, i32, i64, vp]
        L.fp4_dequantize.restype = i32
        L.fp4_rht.argtypes = [vp, i32, i64, i64, i64, i32, ctypes.c_uint64, i32, vp, vp]
        L.fp4_rht.restype = i32
        L.fp4_gemm_mx.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, i64, vp]
        L.fp4_gemm_mx.restype = i32
        L.fp4_rht_signs.argtypes = [ctypes.c_uint64]
        L.fp4_rht_signs.restype = ctypes.c_uint16
        L.fp4_status_str.argtypes = [i32]
        L.fp4_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_params(fmt="nvfp4", axis="row", rounding="rtne", rht=False, rht_seed=0, sr_seed=0,
                ts_given=False, outer=False) -> Params:
    mode = TS_OUTER128 if outer else (TS_GIVEN if ts_given else TS_COMPUTE)
    return Params(FORMATS[fmt], BLOCK[fmt], AXES[axis], ROUNDINGS[rounding], int(bool(rht)),
                  mode, int(rht_seed) & (2**64 - 1), int(sr_seed) & (2**64 - 1))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class _Alloc:
    """Where a call's own buffers (outputs, workspace, an uploaded tensor
    scale) come from.  They are allocated with ``stream`` current, so the
    caching allocator ties each block to the stream the kernels run on and
    does not hand it to other work while they are queued.  With a raw stream
    handle the binding cannot do that, so such a call must bring every buffer
    itself."""

    def __init__(self, stream):
        self.raw = stream is not None and not isinstance(stream, torch.cuda.Stream)
        self.ctx = (torch.cuda.stream(stream) if isinstance(stream, torch.cuda.Stream)
                    else contextlib.nullcontext())

    def __enter__(self):
        self.ctx.__enter__()
        return self

    def __exit__(self, *exc):
        return self.ctx.__exit__(*exc)

    def _check(self, what):
        if self.raw:
            raise ValueError("%s would be allocated for a launch on a raw stream handle: pass a "
                             "torch.cuda.Stream, or preallocate it" % what)

    def empty(self, shape, dtype, device, what):
        self._check(what)
        return torch.empty(shape, dtype=dtype, device=device)

    def scalar(self, v, device, what):
        self._check(what)
        return torch.tensor([float(v)], dtype=torch.float32, device=device)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_2d(x: torch.Tensor, name: str):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("%s must be a 2-D tensor with unit column stride" % name)
    if not x.is_cuda:
        raise ValueError("%s must be a device tensor" % name)


def rht_signs(seed: int) -> int:
    return int(load().fp4_rht_signs(int(seed) & (2**64 - 1)))


def workspace_bytes(rows: int, cols: int, params: Params) -> int:
    return int(load().fp4_workspace_bytes(rows, cols, ctypes.byref(params)))


def workspace_bytes_dual(rows: int, cols: int, params: Params) -> int:
    return int(load().fp4_workspace_bytes_dual(rows, cols, ctypes.byref(params)))


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def new_workspace(rows: int, cols: int, params: Params, device) -> Optional[torch.Tensor]:
    """A workspace for repeated quantize calls (None if none is needed); its
    contents need no initialization."""
    n = workspace_bytes(rows, cols, params)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def output_shapes(rows: int, cols: int, fmt: str, axis: str):
    ra, w = (rows, cols) if axis == "row" else (cols, rows)
    return (ra, w // 2), (ra, w // BLOCK[fmt] * SCALE_BYTES[fmt])


def outer_shape(rows: int, cols: int, axis: str):
    """Shape of the outer-scale array of the double-block mode."""
    ra, w = (rows, cols) if axis == "row" else (cols, rows)
    return (ra, w // OUTER)


def quantize(x: torch.Tensor, fmt: str = "nvfp4", axis: str = "row", rounding: str = "rtne",
             rht: bool = False, rht_seed: int = 0, sr_seed: int = 0,
             tensor_scale=None, codes: Optional[torch.Tensor] = None,
             scales: Optional[torch.Tensor] = None, ts_out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None, stream=None, outer: bool = False):
    """Quantize a BF16/FP32 device matrix.  Returns (codes, scales, tensor_scale).

    ``tensor_scale``: None computes the two-level tensor scale from the data;
    a float or one-element float32 device tensor supplies it.  The returned
    tensor scale is a one-element float32 device tensor (None for the MX
    formats).  ``outer=True`` selects double-block scales: the third result
    is then the float32 outer-scale array of shape ``outer_shape()``."""
    _check_2d(x, "x")
    if x.dtype not in DTYPES:
        raise TypeError("x must be bfloat16 or float32")
    rows, cols = x.shape
    outer = (bool(outer) or fmt in ALWAYS_OUTER) and fmt not in NO_TENSOR_SCALE
    given = tensor_scale is not None and not outer
    p = make_params(fmt, axis, rounding, rht, rht_seed, sr_seed, given, outer)
    cshape, sshape = output_shapes(rows, cols, fmt, axis)
    dev = x.device
    with _Alloc(stream) as al:
        if codes is None:
            codes = al.empty(cshape, torch.uint8, dev, "codes")
        if scales is None:
            scales = al.empty(sshape, torch.uint8, dev, "scales")
        ts = None
        if outer:
            ts = ts_out if ts_out is not None else al.empty(
                outer_shape(rows, cols, axis), torch.float32, dev, "the outer-scale array")
        elif fmt not in NO_TENSOR_SCALE:
            if given:
                ts = tensor_scale if torch.is_tensor(tensor_scale) else al.scalar(
                    tensor_scale, dev, "the given tensor scale")
            else:
                ts = ts_out if ts_out is not None else al.empty(1, torch.float32, dev,
                                                                "the tensor scale")
        nws = workspace_bytes(rows, cols, p)
        if nws and workspace is None:
            workspace = al.empty(nws, torch.uint8, dev, "the workspace")
        st = load().fp4_quantize(x.data_ptr(), DTYPES[x.dtype], rows, cols, x.stride(0),
                                 ctypes.byref(p), codes.data_ptr(), scales.data_ptr(), _ptr(ts),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream))
    if st != FP4_OK:
        raise FP4Error(st, "fp4_quantize")
    return codes, scales, ts


class Prepared:
    """One library call with its arguments marshalled once (pointers, sizes,
    parameters, stream); calling it makes only the C call.  It holds the
    tensors it points to, so they stay alive as long as it does."""

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self._name, self._keep = fn, args, name, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != FP4_OK:
            raise FP4Error(st, self._name)


def prepare_quantize(x: torch.Tensor, fmt: str, axis: str, rounding: str, rht: bool,
                     rht_seed: int, sr_seed: int, codes: torch.Tensor, scales: torch.Tensor,
                     ts_out: Optional[torch.Tensor], workspace: Optional[torch.Tensor],
                     stream=None, outer: bool = False) -> Prepared:
    """``quantize`` into the given buffers (nothing is allocated), with a
    computed tensor scale (or outer scales, or none for the MX formats and
    HiF4), as a prepared call for repeated launches."""
    _check_2d(x, "x")
    if x.dtype not in DTYPES:
        raise TypeError("x must be bfloat16 or float32")
    rows, cols = x.shape
    outer = (bool(outer) or fmt in ALWAYS_OUTER) and fmt not in NO_TENSOR_SCALE
    p = make_params(fmt, axis, rounding, rht, rht_seed, sr_seed, False, outer)
    if fmt in NO_TENSOR_SCALE:
        ts_out = None
    elif ts_out is None:
        raise ValueError("a two-level format needs ts_out")
    if workspace_bytes(rows, cols, p) and workspace is None:
        raise ValueError("a computed tensor scale needs a workspace")
    args = (x.data_ptr(), DTYPES[x.dtype], rows, cols, x.stride(0), ctypes.byref(p),
            codes.data_ptr(), scales.data_ptr(), _ptr(ts_out), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    return Prepared(load().fp4_quantize, args, "fp4_quantize",
                    (x, codes, scales, ts_out, workspace, p, stream))


def prepare_dequantize(codes: torch.Tensor, scales: torch.Tensor, tensor_scale, rows: int,
                       cols: int, fmt: str, axis: str, rht: bool, rht_seed: int,
                       inverse_rht: bool, out: torch.Tensor, stream=None) -> Prepared:
    """``dequantize`` into ``out`` as a prepared call for repeated launches."""
    if out.dtype not in DTYPES:
        raise TypeError("out must be bfloat16 or float32")
    outer = torch.is_tensor(tensor_scale) and tensor_scale.dim() == 2
    p = make_params(fmt, axis, "rtne", rht, rht_seed, 0, not outer, outer)
    args = (codes.data_ptr(), scales.data_ptr(), _ptr(tensor_scale), rows, cols,
            ctypes.byref(p), int(bool(inverse_rht)), out.data_ptr(), DTYPES[out.dtype],
            out.stride(0), _stream(stream))
    return Prepared(load().fp4_dequantize, args, "fp4_dequantize",
                    (codes, scales, tensor_scale, out, p, stream))


def input_bytes(rows: int, cols: int, ld: int, dtype: torch.dtype, params: Params,
                ws_bytes: int) -> int:
    """Bytes of x that fp4_quantize reads with these arguments on the current
    device, outside graph capture (once, or twice with a tensor-maximum pass,
    or in between for the wide single pass); no launch."""
    if dtype not in DTYPES:
        raise TypeError("x must be bfloat16 or float32")
    out = ctypes.c_int64(0)
    st = load().fp4_quantize_input_bytes(DTYPES[dtype], rows, cols, ld, ctypes.byref(params),
                                         ws_bytes, ctypes.byref(out))
    if st != FP4_OK:
        raise FP4Error(st, "fp4_quantize_input_bytes")
    return int(out.value)


def quantize_noalloc(x: torch.Tensor, fmt: str = "nvfp4", axis: str = "row",
                     rounding: str = "rtne", rht: bool = False, rht_seed: int = 0,
                     sr_seed: int = 0, tensor_scale=None, codes: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None,
                     ts_out: Optional[torch.Tensor] = None, stream=None, outer: bool = False):
    """``quantize`` through the allocation-free entry point: the library
    takes no workspace and allocates nothing (its records live in a fixed
    per-device array, shared by every such call on the device, so calls
    that overlap in time on one device race).  Outputs not passed in are
    allocated here, as ``quantize`` does; a caller that must not allocate
    passes all of them (and a device tensor as a given tensor scale)."""
    _check_2d(x, "x")
    if x.dtype not in DTYPES:
        raise TypeError("x must be bfloat16 or float32")
    rows, cols = x.shape
    outer = (bool(outer) or fmt in ALWAYS_OUTER) and fmt not in NO_TENSOR_SCALE
    given = tensor_scale is not None and not outer
    p = make_params(fmt, axis, rounding, rht, rht_seed, sr_seed, given, outer)
    cshape, sshape = output_shapes(rows, cols, fmt, axis)
    dev = x.device
    with _Alloc(stream) as al:
        if codes is None:
            codes = al.empty(cshape, torch.uint8, dev, "codes")
        if scales is None:
            scales = al.empty(sshape, torch.uint8, dev, "scales")
        ts = None
        if outer:
            ts = ts_out if ts_out is not None else al.empty(
                outer_shape(rows, cols, axis), torch.float32, dev, "the outer-scale array")
        elif fmt not in NO_TENSOR_SCALE:
            if given:
                ts = tensor_scale if torch.is_tensor(tensor_scale) else al.scalar(
                    tensor_scale, dev, "the given tensor scale")
            else:
                ts = ts_out if ts_out is not None else al.empty(1, torch.float32, dev,
                                                                "the tensor scale")
        st = load().fp4_quantize_noalloc(x.data_ptr(), DTYPES[x.dtype], rows, cols,
                                         x.stride(0), ctypes.byref(p), codes.data_ptr(),
                                         scales.data_ptr(), _ptr(ts), _stream(stream))
    if st != FP4_OK:
        raise FP4Error(st, "fp4_quantize_noalloc")
    return codes, scales, ts


def quantize_dual(x: torch.Tensor, fmt: str = "nvfp4", rounding: str = "rtne", rht: bool = False,
                  rht_seed: int = 0, sr_seed: int = 0, tensor_scale=None, outer: bool = False,
                  out_row=None, out_col=None, workspace: Optional[torch.Tensor] = None,
                  stream=None):
    """Row-axis and column-axis quantization of x in one call.  Returns
    ((codes, scales, ts) of the row axis, (codes, scales, ts) of the column
    axis), each as ``quantize`` would.  ``tensor_scale``: None (computed), or
    a pair (row, column) of given scales.  ``out_row`` / ``out_col``:
    optional preallocated (codes, scales, ts) triples."""
    _check_2d(x, "x")
    if x.dtype not in DTYPES:
        raise TypeError("x must be bfloat16 or float32")
    rows, cols = x.shape
    outer = (bool(outer) or fmt in ALWAYS_OUTER) and fmt not in NO_TENSOR_SCALE
    given = tensor_scale is not None and not outer
    p = make_params(fmt, "row", rounding, rht, rht_seed, sr_seed, given, outer)
    dev = x.device
    outs = []
    with _Alloc(stream) as al:
        for axis, pre in (("row", out_row), ("col", out_col)):
            if pre is not None:
                outs.append(tuple(pre))
                continue
            cshape, sshape = output_shapes(rows, cols, fmt, axis)
            ts = None
            if outer:
                ts = al.empty(outer_shape(rows, cols, axis), torch.float32, dev,
                              "the outer-scale array")
            elif fmt not in NO_TENSOR_SCALE:
                if given:
                    v = tensor_scale[0 if axis == "row" else 1]
                    ts = v if torch.is_tensor(v) else al.scalar(v, dev, "the given tensor scale")
                else:
                    ts = al.empty(1, torch.float32, dev, "the tensor scale")
            outs.append((al.empty(cshape, torch.uint8, dev, "codes"),
                         al.empty(sshape, torch.uint8, dev, "scales"), ts))
        nws = workspace_bytes_dual(rows, cols, p)
        if nws and workspace is None:
            workspace = al.empty(nws, torch.uint8, dev, "the workspace")
        (cr, sr_, tr), (cc, sc, tc) = outs
        st = load().fp4_quantize_dual(x.data_ptr(), DTYPES[x.dtype], rows, cols, x.stride(0),
                                      ctypes.byref(p), cr.data_ptr(), sr_.data_ptr(), _ptr(tr),
                                      cc.data_ptr(), sc.data_ptr(), _ptr(tc), _ptr(workspace),
                                      _nbytes(workspace), _stream(stream))
    if st != FP4_OK:
        raise FP4Error(st, "fp4_quantize_dual")
    return outs[0], outs[1]


def dequantize(codes: torch.Tensor, scales: torch.Tensor, tensor_scale, rows: int, cols: int,
               fmt: str = "nvfp4", axis: str = "row", rht: bool = False, rht_seed: int = 0,
               inverse_rht: bool = False, out_dtype=torch.float32,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Rebuild a rows x cols matrix (x's layout) from codes and scales.  A 2-D
    ``tensor_scale`` is the outer-scale array of the double-block mode."""
    outer = torch.is_tensor(tensor_scale) and tensor_scale.dim() == 2
    p = make_params(fmt, axis, "rtne", rht, rht_seed, 0, not outer, outer)
    with _Alloc(stream) as al:
        if out is None:
            out = al.empty((rows, cols), out_dtype, codes.device, "out")
    if out.dtype not in DTYPES:
        raise TypeError("out must be bfloat16 or float32")
    st = load().fp4_dequantize(codes.data_ptr(), scales.data_ptr(), _ptr(tensor_scale), rows,
                               cols, ctypes.byref(p), int(bool(inverse_rht)), out.data_ptr(),
                               DTYPES[out.dtype], out.stride(0), _stream(stream))
    if st != FP4_OK:
        raise FP4Error(st, "fp4_dequantize")
    return out


def gemm_mx(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
            b_scales: torch.Tensor, out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """C = A · Bᵀ of two MXFP4 operands quantized along K (``quantize(...,
    "mxfp4", "row")`` outputs: codes [rows, K/2], scales [rows, K/32]).
    Returns the M x N float32 or bfloat16 product."""
    M, kh = a_codes.shape
    N, kh2 = b_codes.shape
    if kh != kh2:
        raise ValueError("A and B must have the same K")
    K = 2 * kh
    with _Alloc(stream) as al:
        if out is None:
            out = al.empty((M, N), out_dtype, a_codes.device, "out")
    if out.dtype not in DTYPES:
        raise TypeError("out must be bfloat16 or float32")
    st = load().fp4_gemm_mx(a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(),
                            b_scales.data_ptr(), M, N, K, out.data_ptr(), DTYPES[out.dtype],
                            out.stride(0), _stream(stream))
    if st != FP4_OK:
        raise FP4Error(st, "fp4_gemm_mx")
    return out


def rht(x: torch.Tensor, axis: str = "row", seed: int = 0, inverse: bool = False,
        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Standalone 16-point RHT (or its inverse) along an axis; FP32 output."""
    _check_2d(x, "x")
    rows, cols = x.shape
    with _Alloc(stream) as al:
        if out is None:
            out = al.empty((rows, cols), torch.float32, x.device, "out")
    st = load().fp4_rht(x.data_ptr(), DTYPES[x.dtype], rows, cols, x.stride(0), AXES[axis],
                        int(seed) & (2**64 - 1), int(bool(inverse)), out.data_ptr(),
                        _stream(stream))
    if st != FP4_OK:
        raise FP4Error(st, "fp4_rht")
    return out
