"""Prox CPU oracle (ctypes shim over ``prox_oracle.c``).

TEST INFRASTRUCTURE: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path
(the HIP library and its Python binding) never does, and shares no code
with it.

Every step follows the Prox pages' description of the method (original
abstract; technical summary: Problem Statement, Stage 1: Lightweight Proxy
Construction, Stage 2: Exact Sparse Computation); the readings taken where
the pages are silent are stated in ``prox_oracle.c`` beside each step.
Arithmetic is binary64 except the quantizer, which is binary32 with
round-to-nearest-even.

Inputs are NumPy arrays: float32 values, or bfloat16 bit patterns as
uint16 (widened here, exactly, to binary32 / binary64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "prox_oracle.c")
_LIB = os.path.join(_HERE, "libprox_oracle.so")

MODE_INT8_ROW = 0
MODE_INT4_G128 = 1
_MODES = {"int8_row": MODE_INT8_ROW, "int4_g128": MODE_INT4_G128}
ACTS = {"silu": 0, "gelu_tanh": 1}
# selection signals: the proxy intermediate state (Prox), one proxy branch,
# or the exact intermediate state (dense exact gate/up: the "oracle" mask)
SIGNALS = {"s": 0, "h": 1, "u": 2, "exact_s": 3}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (binary64 loops, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                               "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_LIB_SAN = os.path.join(_HERE, "libprox_oracle_san.so")
_CLANG = "/opt/rocm/llvm/bin/clang"


def build_sanitized() -> str:
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (clang, whose sanitizer runtime also serves the HIP library's sanitized
    host build), for the host-sanitizer test run.  Same arithmetic flags."""
    tmp = _LIB_SAN + ".tmp%d" % os.getpid()
    subprocess.check_call([_CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-std=c11", "-ffp-contract=off", "-fopenmp",
                           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm", "-L/opt/rocm/llvm/lib",
                           "-Wl,-rpath,/opt/rocm/llvm/lib"])
    os.replace(tmp, _LIB_SAN)
    return _LIB_SAN


def use_library(path=None) -> None:
    """Point the shim at another build of ``prox_oracle.c`` (None = the default).

    Used only by the mutation test, which compiles copies of the oracle with
    a planted mistake to show that the pins catch it."""
    global _lib
    _lib = None
    if path is not None:
        _bind(ctypes.CDLL(path))


def _load():
    if _lib is None:
        alt = os.environ.get("PROX_ORACLE_LIB")  # another build of prox_oracle.c (the sanitized one)
        if alt:
            _bind(ctypes.CDLL(alt))
        else:
            build(force=False)
            _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    global _lib
    P = ctypes.c_void_p
    I = ctypes.c_int64
    D = ctypes.c_double
    lib.oracle_silu.argtypes = [D]
    lib.oracle_silu.restype = D
    lib.oracle_gelu_tanh.argtypes = [D]
    lib.oracle_gelu_tanh.restype = D
    lib.oracle_input_count.argtypes = [D, I]
    lib.oracle_input_count.restype = I
    lib.oracle_channel_count.argtypes = [D, I]
    lib.oracle_channel_count.restype = I
    lib.oracle_quantize_int8_row.argtypes = [P, I, I, P, P]
    lib.oracle_quantize_int4_g128.argtypes = [P, I, I, P, P]
    lib.oracle_topk_ascending.argtypes = [P, I, I, P, P]
    lib.oracle_input_select.argtypes = [P, I, I, I, P]
    lib.oracle_proxy.argtypes = [P, I, I, I, ctypes.c_int, P, P, P, P, ctypes.c_int, ctypes.c_int, P, P, P]
    lib.oracle_ffn_masked.argtypes = [P, I, I, I, P, P, P, P, I, ctypes.c_int, P, P]
    lib.oracle_rmsnorm.argtypes = [P, I, I, D, P]
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_decode.restype = D
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode.restype = ctypes.c_int
    lib.oracle_quantize_fp8_row.argtypes = [P, I, I, P, P]
    lib.oracle_dequant_fp8_f32.argtypes = [P, P, I, I, P]
    lib.oracle_ffn_masked_fp8.argtypes = [P, I, I, I, P, P, P, P, P, P, P, I, ctypes.c_int, P, P]
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_get_threads.restype = ctypes.c_int
    _lib = lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def as_f32(a: np.ndarray) -> np.ndarray:
    """binary32 values of an input tensor; uint16 is read as bfloat16 bits."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float32)


def as_f64(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(as_f32(a), dtype=np.float64)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


# ---------------------------------------------------------------- steps

def gelu_tanh(z: float) -> float:
    return _load().oracle_gelu_tanh(float(z))


def silu(z: float) -> float:
    return float(_load().oracle_silu(float(z)))


def input_count(keep: float, d: int) -> int:
    """k_in for an input-keep fraction (given as the binary32 value the API receives)."""
    return int(_load().oracle_input_count(float(np.float32(keep)), int(d)))


def channel_count(sparsity: float, F: int) -> int:
    """k for an FFN-sparsity fraction (binary32 value, as the API receives it)."""
    return int(_load().oracle_channel_count(float(np.float32(sparsity)), int(F)))


def quantize(w: np.ndarray, mode: str):
    """Proxy quantization of one [F][d] weight matrix.

    Returns (codes int8 [F][d], scales float32 [F] or [F][d/128])."""
    w = as_f32(w)
    F, d = w.shape
    q = np.empty((F, d), dtype=np.int8)
    lib = _load()
    if _MODES[mode] == MODE_INT8_ROW:
        sc = np.empty((F,), dtype=np.float32)
        lib.oracle_quantize_int8_row(_p(w), F, d, _p(q), _p(sc))
    else:
        assert d % 128 == 0
        sc = np.empty((F, d // 128), dtype=np.float32)
        lib.oracle_quantize_int4_g128(_p(w), F, d, _p(q), _p(sc))
    return q, sc


def e4m3_decode(c: int) -> float:
    """Value of one OCP E4M3 code (NaN for S.1111.111)."""
    return _load().oracle_e4m3_decode(int(c))


def e4m3_encode(v: float) -> int:
    """Nearest OCP E4M3 code to a binary32 value (ties to even, saturating at 448)."""
    return _load().oracle_e4m3_encode(float(np.float32(v)))


def quantize_fp8(w: np.ndarray):
    """FP8 (E4M3) copy of one weight matrix, one binary32 scale per row.

    Returns (codes uint8 [R][C], scales float32 [R])."""
    w = as_f32(w)
    R, C = w.shape
    q = np.empty((R, C), dtype=np.uint8)
    sc = np.empty((R,), dtype=np.float32)
    _load().oracle_quantize_fp8_row(_p(w), R, C, _p(q), _p(sc))
    return q, sc


def dequant_fp8_f32(q: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """fl32(scale * decode(code)) per element: the binary32 weights an FP8 matrix stands for."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sc = np.ascontiguousarray(sc, dtype=np.float32)
    R, C = q.shape
    w = np.empty((R, C), dtype=np.float32)
    _load().oracle_dequant_fp8_f32(_p(q), _p(sc), R, C, _p(w))
    return w


def ffn_masked_fp8(x: np.ndarray, fp8, sel: np.ndarray, act: str = "silu"):
    """Stage-2 exact SwiGLU on FP8 weights, fp8 = (qg, sg, qu, su, qd, sd) from
    ``quantize_fp8`` of W_gate, W_up [F][d] and W_down [d][F].

    Returns (y [B][d] binary64, s [B][k])."""
    x = np.atleast_2d(as_f64(x))
    B, d = x.shape
    qg, sg, qu, su, qd, sd = [np.ascontiguousarray(a) for a in fp8]
    F = qg.shape[0]
    assert qg.shape == (F, d) and qu.shape == (F, d) and qd.shape == (d, F)
    assert qg.dtype == np.uint8 and sg.dtype == np.float32 and sd.shape == (d,)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    k = sel.size
    y = np.empty((B, d))
    s = np.empty((B, k))
    _load().oracle_ffn_masked_fp8(_p(x), B, d, F, _p(qg), _p(sg), _p(qu), _p(su), _p(qd), _p(sd), _p(sel), k,
                                  ACTS[act], _p(s), _p(y))
    return y, s


def topk_ascending(v: np.ndarray, k: int):
    """First k indices of v under (|v| desc, index asc), ascending; and the k-th magnitude."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty((max(k, 0),), dtype=np.int64)
    kth = ctypes.c_double(0.0)
    _load().oracle_topk_ascending(_p(v), v.size, int(k), _p(out), ctypes.byref(kth))
    return out, kth.value


def input_select(x: np.ndarray, k_in: int) -> np.ndarray:
    """Stage-1 sparse input: per token, the k_in largest-magnitude entries kept."""
    x = np.atleast_2d(as_f64(x))
    B, d = x.shape
    xh = np.empty_like(x)
    _load().oracle_input_select(_p(x), B, d, int(k_in), _p(xh))
    return xh


def proxy(xhat: np.ndarray, qg, scg, qu, scu, mode: str, act: str = "silu", signal: str = "s"):
    """Proxy gate/up activations and the channel salience score for a proxy
    signal ("s": |act(g~) u~|, "h": |act(g~)|, "u": |u~|), summed over tokens.

    Returns (g~ [B][F], u~ [B][F], score [F])."""
    xhat = np.ascontiguousarray(np.atleast_2d(xhat), dtype=np.float64)
    B, d = xhat.shape
    F = qg.shape[0]
    qg = np.ascontiguousarray(qg, dtype=np.int8)
    qu = np.ascontiguousarray(qu, dtype=np.int8)
    scg = np.ascontiguousarray(scg, dtype=np.float32)
    scu = np.ascontiguousarray(scu, dtype=np.float32)
    gt = np.empty((B, F))
    ut = np.empty((B, F))
    score = np.empty((F,))
    _load().oracle_proxy(_p(xhat), B, d, F, _MODES[mode], _p(qg), _p(scg), _p(qu), _p(scu),
                         ACTS[act], SIGNALS[signal], _p(gt), _p(ut), _p(score))
    return gt, ut, score


def ffn_masked(x: np.ndarray, wg, wu, wd, sel: np.ndarray, act: str = "silu"):
    """Stage-2 exact SwiGLU FFN on the channels in ``sel`` (ascending).

    Returns (y [B][d] binary64, s [B][k])."""
    x = np.atleast_2d(as_f64(x))
    B, d = x.shape
    wg, wu, wd = as_f32(wg), as_f32(wu), as_f32(wd)
    F = wg.shape[0]
    assert wg.shape == (F, d) and wu.shape == (F, d) and wd.shape == (d, F)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    k = sel.size
    y = np.empty((B, d))
    s = np.empty((B, k))
    _load().oracle_ffn_masked(_p(x), B, d, F, _p(wg), _p(wu), _p(wd), _p(sel), k, ACTS[act], _p(s), _p(y))
    return y, s


def ffn_dense(x, wg, wu, wd, act: str = "silu"):
    """Dense SwiGLU (or GeGLU) FFN: the masked FFN with every channel selected."""
    F = np.asarray(wg).shape[0]
    return ffn_masked(x, wg, wu, wd, np.arange(F, dtype=np.int64), act)


def exact_scores(x, wg, wu, wd, act: str = "silu", fp8=None):
    """The exact-state signal, score_j = sum_b |s_{b,j}| with s the exact
    intermediate state of every channel (dense x, the exact weights)."""
    F = (np.asarray(wg) if fp8 is None else fp8[0]).shape[0]
    allc = np.arange(F, dtype=np.int64)
    _, s = ffn_masked(x, wg, wu, wd, allc, act) if fp8 is None else ffn_masked_fp8(x, fp8, allc, act)
    return np.abs(s).sum(axis=0)


def rmsnorm(h: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    h = np.atleast_2d(as_f64(h))
    B, d = h.shape
    r = np.empty_like(h)
    _load().oracle_rmsnorm(_p(h), B, d, float(eps), _p(r))
    return r


# --------------------------------------------------------- whole forward

def prox_forward(x, wg, wu, wd, proxy_q, input_keep: float, ffn_sparsity: float, mode: str, fp8=None,
                 act: str = "silu", signal: str = "s"):
    """The Prox forward, step by step.

    proxy_q = (codes_gate, scales_gate, codes_up, scales_up) from ``quantize``.
    Stage 1: sparse x -> proxy g~, u~ -> salience -> top-k mask (shared by
    gate, up and down).  Stage 2: exact masked SwiGLU with dense x; with
    ``fp8`` = (qg, sg, qu, su, qd, sd), on those FP8 weights instead of
    wg, wu, wd (which may then be None).  ``act`` is the gate activation
    (silu, or gelu_tanh for GeGLU FFNs); ``signal`` the selection signal:
    "s" (Prox), "h" or "u" (one proxy branch), or "exact_s" (the exact
    intermediate state of every channel, no proxy: the ideal mask).
    Returns a dict with k_in, k, xhat, score, sel, T (k-th score), y, s."""
    x = np.atleast_2d(x)
    B, d = x.shape
    F = (np.asarray(wg) if fp8 is None else fp8[0]).shape[0]
    k_in = input_count(input_keep, d)
    k = channel_count(ffn_sparsity, F)
    xhat = input_select(x, k_in)
    if signal == "exact_s":
        gt = ut = None
        score = exact_scores(x, wg, wu, wd, act, fp8)
    else:
        qg, scg, qu, scu = proxy_q
        gt, ut, score = proxy(xhat, qg, scg, qu, scu, mode, act, signal)
    sel, T = topk_ascending(score, k)
    y, s = ffn_masked(x, wg, wu, wd, sel, act) if fp8 is None else ffn_masked_fp8(x, fp8, sel, act)
    return dict(k_in=k_in, k=k, xhat=xhat, g_proxy=gt, u_proxy=ut, score=score, sel=sel, T=T, y=y, s=s)


# ------------------------------------------------- sparsity allocation
# The pages (technical summary, Sparsity Allocation): Stage 2 sparsity is
# anchored near 70%; Stage 1 keeps at least 30% of the inputs; a cost model
# picks both to meet a target effective sparsity at the least normalized
# cost, counting the proxy's overhead.  Reading: the normalized cost of a
# layer is (t1(keep) + t2(kappa)) / t_dense with t1, t2 the measured Stage-1
# and Stage-2 times, each linear in its fraction (keep = kept inputs, kappa =
# 1 - sparsity = kept channels); the effective sparsity is 1 - that cost.  A
# target is a cost budget; it is split by holding Stage-2 sparsity at the
# anchor and solving for keep, then -- when keep would leave [min_keep, 1] --
# holding keep at that bound and solving for the sparsity instead.

def effective_sparsity(model, keep: float, sparsity: float) -> float:
    """model = (a1, b1, a2, b2, dense): t1 = a1 + b1 keep, t2 = a2 + b2 (1 - sparsity)."""
    a1, b1, a2, b2, dense = model
    return 1.0 - (a1 + b1 * keep + a2 + b2 * (1.0 - sparsity)) / dense


def allocate_sparsity(model, target: float, anchor: float = 0.7, min_keep: float = 0.3):
    """(keep, sparsity) meeting the target effective sparsity, or None when even
    dropping every channel at the least keep misses it."""
    a1, b1, a2, b2, dense = model
    budget = (1.0 - target) * dense          # time the layer may take
    if b1 > 0:  # hold the anchor, solve for keep
        keep = (budget - a1 - a2 - b2 * (1.0 - anchor)) / b1
        if min_keep <= keep <= 1.0:
            return keep, anchor
        keep = 1.0 if keep > 1.0 else min_keep
    else:       # keep costs nothing: keep every input
        keep = 1.0
    kappa = (budget - a1 - b1 * keep - a2) / b2
    if kappa < 0.0:
        return None
    return keep, 1.0 - min(kappa, 1.0)


def ambiguous_set(score: np.ndarray, T: float, rel: float = 1e-4) -> np.ndarray:
    """Channels whose score lies within ``rel`` (relative) of the k-th score."""
    score = np.asarray(score, dtype=np.float64)
    return np.nonzero(np.abs(score - T) <= rel * T)[0]


def mask_admissible(sel_gpu: np.ndarray, sel_ref: np.ndarray, score: np.ndarray, T: float,
                    k: int, rel: float = 1e-4):
    """Acceptance rule for a mask: exactly k distinct channels; every reference
    channel outside the near-tie window is selected; nothing outside
    reference-or-window is selected.  Returns (ok, message)."""
    sel_gpu = np.asarray(sel_gpu, dtype=np.int64)
    if sel_gpu.size != k:
        return False, "size %d != k %d" % (sel_gpu.size, k)
    if np.unique(sel_gpu).size != k:
        return False, "duplicate channels"
    A = set(ambiguous_set(score, T, rel).tolist())
    ref = set(np.asarray(sel_ref).tolist())
    got = set(sel_gpu.tolist())
    missing = [j for j in ref - A if j not in got]
    extra = [j for j in got if j not in ref and j not in A]
    if missing or extra:
        return False, "missing %s extra %s (window %d)" % (missing[:8], extra[:8], len(A))
    return True, "ok (window %d, differ %d)" % (len(A), len(ref ^ got))
