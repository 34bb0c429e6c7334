"""C-ABI checks that need no GPU: the library loads, exports every function
include/prox.h declares, and rejects invalid arguments with the documented
status before launching anything (the pointers below are never touched)."""
import ctypes
import os
import re
import subprocess

import pytest

import free_sparse_swiglu_stage1_amd as P
from free_sparse_swiglu_stage1_amd import prox as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prox.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(prox_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return P.load_library()


def test_header_declares_binding_symbols():
    assert declared_functions() == sorted(B.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\bT (prox_[a-z0-9_]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert lib.prox_status_string(s).decode().startswith("PROX_")
    assert b"unknown" in lib.prox_status_string(7)
    assert P.version().startswith("prox-gfx950")


@pytest.mark.parametrize("d,F,keep,sp,want", [
    (4096, 14336, 0.5, 0.7, (2048, 4301)), (4096, 11008, 0.5, 0.9, (2048, 1101)),
    (8192, 28672, 0.4, 0.7, (3277, 8602)), (512, 1376, 0.5, 0.5, (256, 688)),
    (4096, 11008, 0.5, 0.0, (2048, 11008)), (4096, 14336, 1.0, 1.0, (4096, 0)),
    (64, 16, 1e-6, 0.5, (1, 8)),
])
def test_counts(d, F, keep, sp, want):
    assert P.counts(d, F, keep, sp) == want


@pytest.mark.parametrize("keep,sp", [(float("nan"), 0.5), (0.0, 0.5), (-0.1, 0.5), (1.01, 0.5),
                                     (0.5, float("nan")), (0.5, -0.01), (0.5, 1.5)])
def test_counts_reject_bad_fractions(keep, sp):
    with pytest.raises(P.ProxError) as e:
        P.counts(4096, 14336, keep, sp)
    assert e.value.status == B.ERR_INVALID_ARG


@pytest.mark.parametrize("d,F,mode,status", [
    (4096, 14336, "int8_row", 0), (8192, 28672, "int4_g128", 0), (4100, 14336, "int8_row", B.ERR_UNSUPPORTED),
    (4096, 14330, "int8_row", B.ERR_UNSUPPORTED), (4104, 14336, "int4_g128", B.ERR_UNSUPPORTED),
    (32768, 14336, "int8_row", B.ERR_UNSUPPORTED), (4096, 131072, "int8_row", B.ERR_UNSUPPORTED),
    (4096, 65536, "int8_row", B.ERR_UNSUPPORTED), (4096, 65520, "int8_row", 0),
])
def test_proxy_sizes(d, F, mode, status):
    if status == 0:
        cb, sb = P.proxy_sizes(d, F, mode)
        if mode == "int8_row":
            assert (cb, sb) == (2 * d * F, 8 * F)
        else:
            assert (cb, sb) == (d * F, 4 * (d // 128) * 2 * F)
    else:
        with pytest.raises(P.ProxError) as e:
            P.proxy_sizes(d, F, mode)
        assert e.value.status == status


def test_workspace_size_limits():
    assert P.workspace_size(4096, 14336, 1) > 0
    assert P.workspace_size(4096, 14336, 16) > P.workspace_size(4096, 14336, 1)
    for bad_b, st in ((0, B.ERR_INVALID_ARG), (17, B.ERR_UNSUPPORTED)):
        with pytest.raises(P.ProxError) as e:
            P.workspace_size(4096, 14336, bad_b)
        assert e.value.status == st
    with pytest.raises(P.ProxError) as e:
        P.workspace_size(8192, 28672, 5, "int4_g128")
    assert e.value.status == B.ERR_UNSUPPORTED


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced: validation fails first


def _w(d=4096, F=14336, dtype=B.BF16, gu=FAKE, dt=FAKE + 4096, wformat=B.W_NATIVE, gsc=None, dsc=None):
    return B._CWeights(d, F, dtype, gu, dt, wformat, gsc, dsc)


def _p(d=4096, F=14336, mode=B.Q_INT8_ROW, codes=FAKE + 8192, scales=FAKE + 12288):
    return B._CProxy(mode, d, F, codes, scales)


def _fwd(lib, x=FAKE + 16384, batch=1, w=None, p=None, keep=0.5, sp=0.7, out=FAKE + 20480, sel=None,
         ws=FAKE + 32768, ws_bytes=1 << 40):
    w = w or _w()
    p = p or _p()
    return lib.prox_ffn_forward(ctypes.c_void_p(x), batch, ctypes.byref(w), ctypes.byref(p), keep, sp,
                                ctypes.c_void_p(out), ctypes.c_void_p(sel) if sel else None,
                                ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), B.ERR_INVALID_ARG),
    (dict(x=FAKE + 8), B.ERR_INVALID_ARG),                 # misaligned
    (dict(out=0), B.ERR_INVALID_ARG),
    (dict(out=FAKE + 16384), B.ERR_INVALID_ARG),           # aliases x
    (dict(ws=0), B.ERR_INVALID_ARG),
    (dict(sel=FAKE + 4), B.ERR_INVALID_ARG),
    (dict(batch=0), B.ERR_INVALID_ARG),
    (dict(batch=17), B.ERR_UNSUPPORTED),
    (dict(keep=float("nan")), B.ERR_INVALID_ARG),
    (dict(keep=0.0), B.ERR_INVALID_ARG),
    (dict(sp=1.0001), B.ERR_INVALID_ARG),
    (dict(sp=float("nan")), B.ERR_INVALID_ARG),
    (dict(ws_bytes=1024), B.ERR_WORKSPACE),
    (dict(w=_w(dtype=7)), B.ERR_UNSUPPORTED),
    (dict(w=_w(d=4100)), B.ERR_UNSUPPORTED),
    (dict(w=_w(gu=0)), B.ERR_INVALID_ARG),
    (dict(p=_p(d=2048)), B.ERR_INVALID_ARG),               # proxy shape != weights shape
    (dict(p=_p(mode=5)), B.ERR_UNSUPPORTED),
    (dict(p=_p(codes=FAKE + 1)), B.ERR_INVALID_ARG),
    (dict(p=_p(mode=B.Q_INT4_G128), batch=8), B.ERR_UNSUPPORTED),
    (dict(w=_w(wformat=7)), B.ERR_UNSUPPORTED),
    (dict(w=_w(wformat=B.W_FP8_E4M3)), B.ERR_INVALID_ARG),                       # FP8 without scales
    (dict(w=_w(wformat=B.W_FP8_E4M3, gsc=FAKE + 40960, dsc=FAKE + 8)), B.ERR_INVALID_ARG),  # misaligned
    (dict(w=_w(d=4104, wformat=B.W_FP8_E4M3, gsc=FAKE + 40960, dsc=FAKE + 45056),
          p=_p(d=4104)), B.ERR_UNSUPPORTED),                                     # FP8 needs d % 16 == 0
])
def test_forward_rejects_before_launch(lib, kw, status):
    assert _fwd(lib, **kw) == status


def test_other_entry_points_reject(lib):
    w, p = _w(), _p()
    v = ctypes.c_void_p
    assert lib.prox_stage2_exact(v(FAKE), 1, ctypes.byref(w), v(FAKE + 64), 14337, v(FAKE + 128), v(FAKE + 256),
                                 1 << 40, None) == B.ERR_INVALID_ARG  # k > F
    assert lib.prox_stage2_exact(v(FAKE), 1, ctypes.byref(w), None, 5, v(FAKE + 128), v(FAKE + 256),
                                 1 << 40, None) == B.ERR_INVALID_ARG  # k > 0 without a mask
    assert lib.prox_topk(v(FAKE), 0, 0, v(FAKE), None, 0, None) == B.ERR_INVALID_ARG
    assert lib.prox_topk(v(FAKE), 100, 101, v(FAKE), None, 0, None) == B.ERR_INVALID_ARG
    assert lib.prox_topk(v(FAKE), 70000, 5, v(FAKE), None, 0, None) == B.ERR_INVALID_ARG
    assert lib.prox_topk(v(FAKE), 65536, 5, v(FAKE), None, 0, None) == B.ERR_INVALID_ARG
    assert lib.prox_stage1_select(v(FAKE), 1, ctypes.byref(w), ctypes.byref(p), 0.5, 0.0, v(FAKE + 64), None,
                                  v(FAKE + 256), 1 << 40, None) == B.ERR_INVALID_ARG  # k == F: no Stage 1
    assert lib.prox_rmsnorm(v(FAKE), 1, 4096, 9, 1e-5, v(FAKE), None) == B.ERR_UNSUPPORTED
    assert lib.prox_rmsnorm(v(FAKE), 1, 4096, B.BF16, float("nan"), v(FAKE), None) == B.ERR_INVALID_ARG
    for d in (16392, 1001, 4100, 4, 65536):  # beyond the row the kernel holds, or not whole 16-byte vectors
        assert lib.prox_rmsnorm(v(FAKE), 1, d, B.BF16, 1e-5, v(FAKE), None) == B.ERR_UNSUPPORTED
        assert lib.prox_rmsnorm(v(FAKE), 2, d, B.F32, 1e-5, v(FAKE), None) == B.ERR_UNSUPPORTED
    assert lib.prox_pack_weights(v(FAKE), v(FAKE), v(0), 4096, 14336, B.BF16, v(FAKE), v(FAKE),
                                 None) == B.ERR_INVALID_ARG
    assert lib.prox_quantize_proxy(ctypes.byref(w), 3, v(FAKE), v(FAKE), None) == B.ERR_UNSUPPORTED
    for act, sig in ((7, 0), (0, 9), (-1, 0)):  # unknown options are refused before any launch
        opt = B._COptions(act, sig)
        assert lib.prox_ffn_forward_ex(v(FAKE), 1, ctypes.byref(w), ctypes.byref(p), 0.5, 0.7, ctypes.byref(opt), None,
                                       v(FAKE + 20480), None, v(FAKE + 32768), 1 << 40, None) == B.ERR_UNSUPPORTED
        assert lib.prox_stage2_exact_ex(v(FAKE), 1, ctypes.byref(w), v(FAKE + 64), 5, ctypes.byref(opt),
                                        v(FAKE + 128), v(FAKE + 256), 1 << 40, None) == B.ERR_UNSUPPORTED
    # the no-alloc forward refuses, on the host, a layer its static array cannot hold
    assert lib.prox_ffn_forward_noalloc(v(FAKE), 16, ctypes.byref(_w(8192, 28672)), ctypes.byref(_p(8192, 28672)),
                                        0.5, 0.7, None, v(FAKE + 20480), None, None) == B.ERR_SCRATCH_LIMIT
    assert lib.prox_ffn_forward_noalloc(v(FAKE), 1, None, ctypes.byref(_p()), 0.5, 0.7, None, v(FAKE + 20480),
                                        None, None) == B.ERR_INVALID_ARG
    assert lib.prox_ffn_forward_noalloc(v(FAKE), 1, ctypes.byref(_w(4100)), ctypes.byref(_p(4100)), 0.5, 0.7, None,
                                        v(FAKE + 20480), None, None) == B.ERR_UNSUPPORTED
    sink = v(FAKE + 64)
    assert lib.prox_read_probe(None, 1024, sink, None) == B.ERR_INVALID_ARG
    assert lib.prox_read_probe(v(FAKE), 1000, sink, None) == B.ERR_INVALID_ARG  # not whole 16-byte vectors
    assert lib.prox_read_probe(v(FAKE), 0, sink, None) == B.ERR_INVALID_ARG
    assert lib.prox_read_probe(v(FAKE), 1024, None, None) == B.ERR_INVALID_ARG
    opt = B._COptions(0, 0, 0, 2)  # an unknown flag
    assert lib.prox_ffn_forward_ex(v(FAKE), 1, ctypes.byref(w), ctypes.byref(p), 0.5, 0.7, ctypes.byref(opt), None,
                                   v(FAKE + 20480), None, v(FAKE + 32768), 1 << 40, None) == B.ERR_UNSUPPORTED
    opt = B._COptions(0, 0, -1)  # a negative wait limit
    assert lib.prox_ffn_forward_ex(v(FAKE), 1, ctypes.byref(w), ctypes.byref(p), 0.5, 0.7, ctypes.byref(opt), None,
                                   v(FAKE + 20480), None, v(FAKE + 32768), 1 << 40, None) == B.ERR_INVALID_ARG
    assert lib.prox_stage2_exact_ex(v(FAKE), 1, ctypes.byref(w), v(FAKE + 64), 5, ctypes.byref(opt),
                                    v(FAKE + 128), v(FAKE + 256), 1 << 40, None) == B.ERR_INVALID_ARG
    n = ctypes.c_uint32()
    assert lib.prox_workspace_check(None, 1 << 20, ctypes.byref(n), None) == B.ERR_INVALID_ARG
    assert lib.prox_workspace_check(v(FAKE), 1 << 20, None, None) == B.ERR_INVALID_ARG
    assert lib.prox_workspace_check(v(FAKE), 4096, ctypes.byref(n), None) == B.ERR_WORKSPACE
    opt = B._COptions(0, 1)  # a proxy signal needs the proxy
    assert lib.prox_ffn_forward_ex(v(FAKE), 1, ctypes.byref(w), None, 0.5, 0.7, ctypes.byref(opt), None,
                                   v(FAKE + 20480), None, v(FAKE + 32768), 1 << 40, None) == B.ERR_INVALID_ARG
    f8 = (v(FAKE), v(FAKE + 64), v(FAKE + 128), v(FAKE + 192))
    assert lib.prox_pack_weights_fp8(v(FAKE), v(FAKE), v(FAKE), 4104, 14336, B.BF16, *f8, None) == B.ERR_UNSUPPORTED
    assert lib.prox_pack_weights_fp8(v(FAKE), v(FAKE), v(FAKE), 4096, 14336, 5, *f8, None) == B.ERR_UNSUPPORTED
    assert lib.prox_pack_weights_fp8(v(FAKE), v(FAKE), v(FAKE), 4096, 14336, B.BF16, v(FAKE), None, v(FAKE),
                                     v(FAKE), None) == B.ERR_INVALID_ARG
    ws = (B._CWeights * 2)(w, _w(F=11008))
    ps = (B._CProxy * 2)(p, _p(F=11008))
    assert lib.prox_chain_forward(v(FAKE), 1, ws, ps, 2, 1e-5, 0.5, 0.7, v(FAKE + 256), 1 << 40,
                                  None) == B.ERR_INVALID_ARG  # layers differ in shape
    assert lib.prox_chain_forward(v(FAKE), 1, ws, ps, 1, 1e-5, 0.5, 0.7, v(FAKE + 256), 64,
                                  None) == B.ERR_WORKSPACE


def test_binding_fails_loudly_without_library(tmp_path):
    # the binding has no fallback: a missing library is an error, never a silent CPU path
    import importlib
    mod = importlib.import_module("free_sparse_swiglu_stage1_amd.prox")
    saved = mod._lib
    mod._lib = None
    try:
        with pytest.raises(RuntimeError):
            mod.load_library(str(tmp_path / "nope.so"))
    finally:
        mod._lib = saved
