"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/fp4.h declares, and rejects bad arguments on the host before any
HIP call.  No valid (computing) call is made here."""
import ctypes
import os
import re

import pytest
import torch

import block_scaled_bit_fp4_amd as fp4
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "fp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fp4.LIB_PATH):
        from block_scaled_bit_fp4_amd import build
        build.build()
    return fp4.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(fp4.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(-7, 1):
        assert lib.fp4_status_str(code)
    assert lib.fp4_status_str(0) == b"ok"


def test_rht_signs_agree_with_oracle(lib):
    for seed in (0, 1, 2, 77, 2**32 + 5, 2**64 - 1):
        assert fp4.rht_signs(seed) == oracle.rht_signs(seed)


def test_workspace_bytes(lib):
    # 1024 partial maxima (two-pass) or 1025 16-byte tagged slots (single pass)
    assert fp4.workspace_bytes(64, 64, fp4.make_params("nvfp4")) == 1025 * 16
    assert fp4.workspace_bytes(64, 64, fp4.make_params("ufp4")) > 0
    assert fp4.workspace_bytes(64, 64, fp4.make_params("mxfp4")) == 0
    assert fp4.workspace_bytes(64, 64, fp4.make_params("nvfp4", ts_given=True)) == 0
    assert fp4.workspace_bytes(64, 128, fp4.make_params("nvfp4", outer=True)) == 0
    assert fp4.workspace_bytes(64, 64, fp4.make_params("mxfp4_oas")) == 0
    assert fp4.workspace_bytes(64, 64, fp4.make_params("mxfp4_oas16")) == 0


# Fake device pointers: validation must reject these calls before touching them.
A = 1 << 20          # 16-byte aligned
MIS = (1 << 20) + 4  # misaligned


def _q(lib, p, x=A, dt=0, rows=64, cols=64, ld=64, codes=A, scales=A, ts=A, ws=A, nws=4096):
    return lib.fp4_quantize(x, dt, rows, cols, ld, ctypes.byref(p) if p is not None else None,
                            codes, scales, ts, ws, nws, None)


def test_quantize_validation(lib):
    P = fp4.make_params
    bad = fp4.Params(*[getattr(P("nvfp4"), f) for f, _ in fp4.Params._fields_])
    assert _q(lib, None) == -1
    bad.block = 32
    assert _q(lib, bad) == -2                                   # NVFP4 needs 16
    bad = P("mxfp4"); bad.block = 16
    assert _q(lib, bad) == -2
    bad = P("nvfp4"); bad.format = 7
    assert _q(lib, bad) == -2
    bad = P("nvfp4"); bad.axis = 2
    assert _q(lib, bad) == -2
    bad = P("nvfp4"); bad.rounding = 3
    assert _q(lib, bad) == -2
    bad = P("nvfp4"); bad.ts_mode = 5
    assert _q(lib, bad) == -2
    bad = P("mxfp4_oas"); bad.block = 16
    assert _q(lib, bad) == -2
    bad = P("hif4"); bad.block = 16                               # HiF4 blocks are 64
    assert _q(lib, bad) == -2
    assert _q(lib, P("hif4"), cols=96, ld=96) == -3               # W % 64
    assert fp4.workspace_bytes(64, 64, P("hif4")) == 0
    assert fp4.output_shapes(64, 128, "hif4", "row") == ((64, 64), (64, 8))
    bad = P("mxfp4_oas16"); bad.block = 32                        # OAS16 is E8M0 per 16
    assert _q(lib, bad) == -2
    assert _q(lib, P("mxfp4_oas16"), cols=40, ld=40) == -3       # W % 16
    bad = P("e2m1_cap2"); bad.block = 32
    assert _q(lib, bad) == -2
    assert _q(lib, P("mxfp4_mbs")) == -2                         # MBS needs its macro scales
    assert _q(lib, P("mxfp4_mbs", ts_given=True)) == -2
    bad = P("nvfp4"); bad.format = 42
    assert _q(lib, bad) == -2
    assert _q(lib, P("nvfp4", outer=True), cols=144, ld=144) == -3   # W % 128
    assert _q(lib, P("ufp4", outer=True, axis="col"), rows=96) == -3
    assert _q(lib, P("nvfp4", outer=True), cols=128, ld=128, ts=0) == -1
    assert _q(lib, P("nvfp4"), dt=9) == -5
    assert _q(lib, P("nvfp4"), cols=24, ld=24) == -3            # W % 16
    assert _q(lib, P("mxfp4"), cols=48, ld=48) == -3            # W % 32
    assert _q(lib, P("nvfp4", axis="col"), rows=24) == -3       # W = rows
    assert _q(lib, P("nvfp4"), ld=32) == -3                     # ld < cols
    assert _q(lib, P("nvfp4"), rows=-1) == -3
    assert _q(lib, P("nvfp4"), x=0) == -1
    assert _q(lib, P("nvfp4"), codes=0) == -1
    assert _q(lib, P("nvfp4"), scales=0) == -1
    assert _q(lib, P("nvfp4"), ts=0) == -1                      # two-level needs ts
    assert _q(lib, P("nvfp4"), x=MIS) == -4
    assert _q(lib, P("nvfp4"), codes=MIS) == -4
    assert _q(lib, P("nvfp4"), cols=16, ld=20) == -4            # 40-byte rows (bf16)
    assert _q(lib, P("nvfp4"), ws=0) == -6
    assert _q(lib, P("nvfp4"), nws=16) == -6
    assert _q(lib, P("nvfp4"), ws=MIS) == -4


def test_dequantize_and_rht_validation(lib):
    P = fp4.make_params
    dq = lambda p, **k: lib.fp4_dequantize(k.get("codes", A), k.get("scales", A), k.get("ts", A),
                                           k.get("rows", 64), k.get("cols", 64),
                                           ctypes.byref(p), k.get("inv", 0), k.get("out", A),
                                           k.get("odt", 1), k.get("ld", 64), None)
    assert dq(P("nvfp4"), odt=4) == -5
    assert dq(P("nvfp4"), inv=1) == -2                           # inverse without rht
    assert dq(P("nvfp4"), cols=40, ld=40) == -3
    assert dq(P("nvfp4"), codes=0) == -1
    assert dq(P("nvfp4"), ts=0) == -1
    assert dq(P("nvfp4"), out=MIS) == -4
    assert dq(P("nvfp4"), rows=0) == 0                           # empty: nothing to do
    r = lambda **k: lib.fp4_rht(k.get("x", A), k.get("dt", 0), k.get("rows", 64),
                                k.get("cols", 64), k.get("ld", 64), k.get("axis", 0), 0,
                                k.get("inv", 0), k.get("y", A), None)
    assert r(dt=3) == -5
    assert r(axis=4) == -2
    assert r(cols=40, ld=40) == -3
    assert r(axis=1, rows=40) == -3
    assert r(x=0) == -1
    assert r(y=MIS) == -4
    assert r(rows=0) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fp4, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fp4, "_lib", None)
    with pytest.raises(RuntimeError):
        fp4.load()


def test_dual_validation(lib):
    P = fp4.make_params
    def dq(p, **k):
        return lib.fp4_quantize_dual(k.get("x", A), k.get("dt", 0), k.get("rows", 128),
                                     k.get("cols", 128), k.get("ld", 128),
                                     ctypes.byref(p) if p is not None else None,
                                     k.get("cr", A), k.get("sr", A), k.get("tr", A),
                                     k.get("cc", A), k.get("sc", A), k.get("tc", A),
                                     k.get("ws", A), k.get("nws", 8192), None)
    # both axes' partial maxima, and room for the single-pass slot exchange
    assert fp4.workspace_bytes_dual(128, 128, P("nvfp4")) >= 2 * 4 * 1024
    assert fp4.workspace_bytes_dual(128, 128, P("nvfp4")) >= fp4.workspace_bytes(128, 128, P("nvfp4"))
    assert fp4.workspace_bytes_dual(128, 128, P("nvfp4", outer=True)) == 0
    assert dq(None) == -1
    assert dq(P("nvfp4"), dt=7) == -5
    assert dq(P("nvfp4"), rows=120) == -3          # column axis: W = rows % 16
    assert dq(P("nvfp4"), cols=120, ld=120) == -3  # row axis
    assert dq(P("nvfp4", outer=True), rows=144) == -3
    assert dq(P("nvfp4"), tr=0) == -1
    assert dq(P("nvfp4"), tc=0) == -1
    assert dq(P("nvfp4"), cc=MIS) == -4
    assert dq(P("nvfp4"), sc=0) == -1
    assert dq(P("nvfp4"), nws=4096) == -6           # needs two partial arrays
    assert dq(P("nvfp4"), ws=0) == -6


def test_noalloc_validation(lib):
    """The allocation-free entry point checks its arguments on the host, as
    fp4_quantize does, before any HIP call (there is no GPU here)."""
    P = fp4.make_params

    def nq(p, x=A, dt=0, rows=64, cols=64, ld=64, codes=A, scales=A, ts=A):
        return lib.fp4_quantize_noalloc(x, dt, rows, cols, ld,
                                        ctypes.byref(p) if p is not None else None,
                                        codes, scales, ts, None)
    assert nq(None) == -1
    bad = P("nvfp4"); bad.block = 32
    assert nq(bad) == -2
    assert nq(P("nvfp4"), dt=9) == -5
    assert nq(P("nvfp4"), cols=24, ld=24) == -3
    assert nq(P("nvfp4"), x=0) == -1
    assert nq(P("nvfp4"), ts=0) == -1
    assert nq(P("nvfp4"), codes=MIS) == -4
    assert nq(P("mxfp4_mbs")) == -2
    # the scratch array holds every workspace the library asks for
    for shape in ((64, 64), (16384, 14336)):
        for fmt in ("nvfp4", "ufp4", "e2m1_cap2"):
            assert fp4.workspace_bytes(*shape, P(fmt)) <= 16640


def test_input_bytes_query(lib):
    """fp4_quantize_input_bytes: host checks, and the modes that read x once
    on any device (no tensor maximum to find first)."""
    P = fp4.make_params
    out = ctypes.c_int64(-1)
    q = lambda p, dt=0, rows=64, cols=64, ld=64, nws=4096, o=ctypes.byref(out): \
        lib.fp4_quantize_input_bytes(dt, rows, cols, ld,
                                     ctypes.byref(p) if p is not None else None, nws, o)
    assert q(None) == -1
    assert q(P("nvfp4"), o=None) == -1
    bad = P("nvfp4"); bad.block = 32
    assert q(bad) == -2
    assert q(P("nvfp4"), dt=4) == -5
    assert q(P("nvfp4"), cols=24, ld=24) == -3
    assert q(P("nvfp4"), ld=32) == -3
    assert q(P("nvfp4"), nws=16) == -6
    assert q(P("nvfp4"), rows=0) == 0 and out.value == 0
    # a workspace too small for the slot exchange: amax pass + quantize pass
    assert q(P("nvfp4", rht=True)) == 0 and out.value == 2 * 64 * 64 * 2
    assert q(P("nvfp4", axis="col"), dt=1) == 0 and out.value == 2 * 64 * 64 * 4
    for p in (P("mxfp4"), P("mxfp4_oas"), P("hif4"), P("nvfp4", ts_given=True)):
        cols = 128
        assert q(p, cols=cols, ld=cols, nws=0) == 0 and out.value == 64 * cols * 2, p.format
    assert q(P("nvfp4", outer=True), cols=128, ld=128, nws=0) == 0 and out.value == 64 * 128 * 2
    assert fp4.input_bytes(64, 128, 128, torch.bfloat16, P("mxfp4_mbs", outer=True), 0) == \
        64 * 128 * 2
