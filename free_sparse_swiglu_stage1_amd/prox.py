"""Python binding of the Prox HIP library (include/prox.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  PyTorch provides device memory and the current HIP stream.
If ``libprox.so`` is missing or fails to load, every call raises
``ProxError`` -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PROX_LIB names another build of the library (the host-sanitized one)
LIB_PATH = os.environ.get("PROX_LIB") or os.path.join(_HERE, "libprox.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH_LIMIT = 0, -1, -2, -3, -4, -5
STATIC_SCRATCH_BYTES = 64 << 20  # PROX_STATIC_SCRATCH_BYTES
F32, BF16 = 0, 1
Q_INT8_ROW, Q_INT4_G128 = 0, 1
W_NATIVE, W_FP8_E4M3 = 0, 1
FLAG_SINGLE_LAUNCH = 1
ACTIVATIONS = {"silu": 0, "gelu_tanh": 1}
SIGNALS = {"s": 0, "h": 1, "u": 2, "exact_s": 3}
MODES = {"int8_row": Q_INT8_ROW, "int4_g128": Q_INT4_G128}

SYMBOLS = (
    "prox_status_string", "prox_version", "prox_counts", "prox_pack_weights", "prox_pack_weights_fp8",
    "prox_proxy_sizes",
    "prox_quantize_proxy", "prox_workspace_size", "prox_workspace_init", "prox_ffn_forward", "prox_ffn_forward_residual",
    "prox_ffn_forward_timed", "prox_stage1_select", "prox_topk", "prox_stage2_exact", "prox_rmsnorm", "prox_chain_forward",
    "prox_ffn_forward_ex", "prox_stage2_exact_ex", "prox_effective_sparsity", "prox_allocate_sparsity",
    "prox_workspace_check", "prox_ffn_forward_noalloc", "prox_read_probe",
)


class ProxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.prox_status_string(status).decode() if _lib is not None else str(status)
        super().__init__("%s: %s" % (where, msg))


class _CWeights(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int64), ("d_ff", ctypes.c_int64), ("dtype", ctypes.c_int),
                ("w_gu", ctypes.c_void_p), ("w_down_t", ctypes.c_void_p), ("wformat", ctypes.c_int),
                ("gu_scales", ctypes.c_void_p), ("down_scales", ctypes.c_void_p)]


class _COptions(ctypes.Structure):
    _fields_ = [("activation", ctypes.c_int), ("signal", ctypes.c_int), ("wait_limit_ticks", ctypes.c_int64),
                ("flags", ctypes.c_int32)]


class _CCostModel(ctypes.Structure):
    _fields_ = [("stage1_fixed_us", ctypes.c_double), ("stage1_per_keep_us", ctypes.c_double),
                ("stage2_fixed_us", ctypes.c_double), ("stage2_per_kept_us", ctypes.c_double),
                ("dense_us", ctypes.c_double)]


class _CProxy(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("d_model", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libprox.so and declare its C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("Prox HIP library not built: %s is missing "
                           "(run `python -m free_sparse_swiglu_stage1_amd.build`)" % path)
    lib = ctypes.CDLL(path)
    P, I64, F, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    PS = ctypes.POINTER(ctypes.c_size_t)
    PI = ctypes.POINTER(ctypes.c_int64)
    PW = ctypes.POINTER(_CWeights)
    PP = ctypes.POINTER(_CProxy)
    PO = ctypes.POINTER(_COptions)
    PM = ctypes.POINTER(_CCostModel)
    D = ctypes.c_double
    PD = ctypes.POINTER(ctypes.c_double)
    sig = {
        "prox_status_string": ([I32], ctypes.c_char_p),
        "prox_version": ([], ctypes.c_char_p),
        "prox_counts": ([I64, I64, F, F, PI, PI], I32),
        "prox_pack_weights": ([P, P, P, I64, I64, I32, P, P, P], I32),
        "prox_pack_weights_fp8": ([P, P, P, I64, I64, I32, P, P, P, P, P], I32),
        "prox_proxy_sizes": ([I64, I64, I32, PS, PS], I32),
        "prox_quantize_proxy": ([PW, I32, P, P, P], I32),
        "prox_workspace_size": ([I64, I64, I64, I32, PS], I32),
        "prox_workspace_init": ([P, ctypes.c_size_t, P], I32),
        "prox_workspace_check": ([P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint32), P], I32),
        "prox_ffn_forward": ([P, I64, PW, PP, F, F, P, P, P, ctypes.c_size_t, P], I32),
        "prox_ffn_forward_residual": ([P, I64, PW, PP, F, F, P, P, P, P, ctypes.c_size_t, P], I32),
        "prox_ffn_forward_timed": ([P, I64, PW, PP, F, F, P, P, P, ctypes.c_size_t, P, P], I32),
        "prox_stage1_select": ([P, I64, PW, PP, F, F, P, P, P, ctypes.c_size_t, P], I32),
        "prox_topk": ([P, I64, I64, P, P, ctypes.c_size_t, P], I32),
        "prox_stage2_exact": ([P, I64, PW, P, I64, P, P, ctypes.c_size_t, P], I32),
        "prox_rmsnorm": ([P, I64, I64, I32, F, P, P], I32),
        "prox_chain_forward": ([P, I64, PW, PP, I64, F, F, F, P, ctypes.c_size_t, P], I32),
        "prox_ffn_forward_ex": ([P, I64, PW, PP, F, F, PO, P, P, P, P, ctypes.c_size_t, P], I32),
        "prox_stage2_exact_ex": ([P, I64, PW, P, I64, PO, P, P, ctypes.c_size_t, P], I32),
        "prox_effective_sparsity": ([PM, D, D, PD], I32),
        "prox_allocate_sparsity": ([PM, D, D, D, PD, PD], I32),
        "prox_ffn_forward_noalloc": ([P, I64, PW, PP, F, F, P, P, P, P], I32),
        "prox_read_probe": ([P, ctypes.c_size_t, P, P], I32),
    }
    for name in SYMBOLS:
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = sig[name]
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != OK:
        raise ProxError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError("Prox supports float32 and bfloat16 tensors, got %s" % dt)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# -------------------------------------------------------------------- data

@dataclass
class Weights:
    """Exact weights in the library's channel-major layout: in the activation
    dtype, or FP8 E4M3 codes (uint8) with per-row scales."""
    w_gu: torch.Tensor        # [F][2][d]
    w_down_t: torch.Tensor    # [F][d]
    d_model: int
    d_ff: int
    act_dtype: torch.dtype = None            # x / out dtype (default: the weights' dtype)
    gu_scales: torch.Tensor = None           # FP8: fp32 [F][2]
    down_scales: torch.Tensor = None         # FP8: fp32 [d]

    @property
    def fp8(self) -> bool:
        return self.gu_scales is not None

    def c(self) -> _CWeights:
        dt = self.act_dtype if self.act_dtype is not None else self.w_gu.dtype
        if self.fp8:
            return _CWeights(self.d_model, self.d_ff, _dtype_code(dt), self.w_gu.data_ptr(), self.w_down_t.data_ptr(),
                             W_FP8_E4M3, self.gu_scales.data_ptr(), self.down_scales.data_ptr())
        return _CWeights(self.d_model, self.d_ff, _dtype_code(dt), self.w_gu.data_ptr(), self.w_down_t.data_ptr(),
                         W_NATIVE, None, None)


@dataclass
class Proxy:
    """Quantized proxy of W_gate / W_up (opaque layout, see include/prox.h)."""
    codes: torch.Tensor       # uint8
    scales: torch.Tensor      # float32
    mode: int
    d_model: int
    d_ff: int

    def c(self) -> _CProxy:
        return _CProxy(self.mode, self.d_model, self.d_ff, self.codes.data_ptr(), self.scales.data_ptr())


# --------------------------------------------------------------- functions

def version() -> str:
    return load_library().prox_version().decode()


def counts(d: int, F: int, input_keep: float, ffn_sparsity: float):
    lib = load_library()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.prox_counts(d, F, input_keep, ffn_sparsity, ctypes.byref(a), ctypes.byref(b)), "prox_counts")
    return a.value, b.value


def pack_weights(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor) -> Weights:
    """nn.Linear weights (gate [F][d], up [F][d], down [d][F]) -> channel-major layout."""
    lib = load_library()
    F, d = w_gate.shape
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _dev(t, n)
    assert w_up.shape == (F, d) and w_down.shape == (d, F)
    w_gu = torch.empty((F, 2, d), dtype=w_gate.dtype, device=w_gate.device)
    w_dt = torch.empty((F, d), dtype=w_gate.dtype, device=w_gate.device)
    _check(lib.prox_pack_weights(_ptr(w_gate), _ptr(w_up), _ptr(w_down), d, F, _dtype_code(w_gate.dtype),
                                 _ptr(w_gu), _ptr(w_dt), _stream(w_gate.device)), "prox_pack_weights")
    return Weights(w_gu, w_dt, d, F)


def pack_weights_fp8(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor) -> Weights:
    """nn.Linear weights -> FP8 E4M3 codes in the channel-major layout, one fp32
    scale per output row; activations keep w_gate's dtype."""
    lib = load_library()
    F, d = w_gate.shape
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _dev(t, n)
    assert w_up.shape == (F, d) and w_down.shape == (d, F)
    dev = w_gate.device
    w_gu = torch.empty((F, 2, d), dtype=torch.uint8, device=dev)
    w_dt = torch.empty((F, d), dtype=torch.uint8, device=dev)
    gsc = torch.empty((F, 2), dtype=torch.float32, device=dev)
    dsc = torch.empty((d,), dtype=torch.float32, device=dev)
    _check(lib.prox_pack_weights_fp8(_ptr(w_gate), _ptr(w_up), _ptr(w_down), d, F, _dtype_code(w_gate.dtype),
                                     _ptr(w_gu), _ptr(gsc), _ptr(w_dt), _ptr(dsc), _stream(dev)),
           "prox_pack_weights_fp8")
    return Weights(w_gu, w_dt, d, F, act_dtype=w_gate.dtype, gu_scales=gsc, down_scales=dsc)


def effective_sparsity(model, input_keep: float, ffn_sparsity: float) -> float:
    """model = (stage1_fixed_us, stage1_per_keep_us, stage2_fixed_us, stage2_per_kept_us, dense_us)."""
    lib = load_library()
    e = ctypes.c_double()
    _check(lib.prox_effective_sparsity(ctypes.byref(_CCostModel(*model)), input_keep, ffn_sparsity, ctypes.byref(e)),
           "prox_effective_sparsity")
    return e.value


def allocate_sparsity(model, target_effective: float, s2_anchor: float = 0.7, min_keep: float = 0.3):
    """(input_keep, ffn_sparsity) for a target effective sparsity (see include/prox.h); None if unreachable."""
    lib = load_library()
    k, s = ctypes.c_double(), ctypes.c_double()
    st = lib.prox_allocate_sparsity(ctypes.byref(_CCostModel(*model)), target_effective, s2_anchor, min_keep,
                                    ctypes.byref(k), ctypes.byref(s))
    if st == ERR_UNSUPPORTED:
        return None
    _check(st, "prox_allocate_sparsity")
    return k.value, s.value


def proxy_sizes(d: int, F: int, mode: str):
    lib = load_library()
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.prox_proxy_sizes(d, F, MODES[mode], ctypes.byref(a), ctypes.byref(b)), "prox_proxy_sizes")
    return a.value, b.value


def quantize_proxy(w: Weights, mode: str = "int8_row") -> Proxy:
    lib = load_library()
    cb, sb = proxy_sizes(w.d_model, w.d_ff, mode)
    dev = w.w_gu.device
    codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    scales = torch.empty(sb // 4, dtype=torch.float32, device=dev)
    cw = w.c()
    _check(lib.prox_quantize_proxy(ctypes.byref(cw), MODES[mode], _ptr(codes), _ptr(scales), _stream(dev)),
           "prox_quantize_proxy")
    return Proxy(codes, scales, MODES[mode], w.d_model, w.d_ff)


def workspace_size(d: int, F: int, batch: int, mode: str = "int8_row") -> int:
    lib = load_library()
    n = ctypes.c_size_t()
    _check(lib.prox_workspace_size(d, F, batch, MODES[mode], ctypes.byref(n)), "prox_workspace_size")
    return n.value


def workspace_init(ws: torch.Tensor) -> torch.Tensor:
    """Zero a workspace's ticket counters (once per allocation, before first use)."""
    lib = load_library()
    _check(lib.prox_workspace_init(_ptr(ws), ws.numel(), _stream(ws.device)), "prox_workspace_init")
    return ws


def workspace_check(ws: torch.Tensor) -> int:
    """Synchronize ws's stream and read its counters: raises ProxError if a
    ticket or arrival counter is left nonzero; returns the number of bounded
    waits that gave up (their results are still exact)."""
    lib = load_library()
    n = ctypes.c_uint32()
    _check(lib.prox_workspace_check(_ptr(ws), ws.numel(), ctypes.byref(n), _stream(ws.device)), "prox_workspace_check")
    return n.value


def alloc_workspace(d: int, F: int, batch: int, mode: str = "int8_row", device="cuda", extra: int = 0):
    ws = torch.empty(workspace_size(d, F, batch, mode) + extra, dtype=torch.uint8, device=device)
    return workspace_init(ws)


def _mode_name(p: Proxy) -> str:
    return "int4_g128" if p.mode == Q_INT4_G128 else "int8_row"


def ffn_forward(x: torch.Tensor, w: Weights, p: Proxy, input_keep: float, ffn_sparsity: float,
                out: torch.Tensor = None, sel_out: torch.Tensor = None, workspace: torch.Tensor = None,
                residual: torch.Tensor = None, activation: str = "silu", signal: str = "s",
                wait_limit_ticks: int = 0, single_launch: bool = False) -> torch.Tensor:
    """The Prox FFN forward on x[B][d]; returns out[B][d] (out = residual + y if residual is given).

    activation: "silu" (SwiGLU) or "gelu_tanh" (GeGLU); signal: the channel
    selection signal, "s" (Prox), "h" / "u" (one proxy branch) or "exact_s"
    (the exact state, no proxy; p may then be None).  wait_limit_ticks: the
    bound of cross-workgroup waits in 10 ns ticks (0: default).  single_launch:
    both stages in one launch where the shape allows it (slower on MI355X;
    see PROX_FLAG_SINGLE_LAUNCH)."""
    lib = load_library()
    _dev(x, "x")
    B = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(w.d_model, w.d_ff, B, _mode_name(p) if p is not None else "int8_row", x.device)
    cw = w.c()
    if activation != "silu" or signal != "s" or wait_limit_ticks or single_launch:
        opt = _COptions(ACTIVATIONS[activation], SIGNALS[signal], wait_limit_ticks,
                        FLAG_SINGLE_LAUNCH if single_launch else 0)
        st = lib.prox_ffn_forward_ex(_ptr(x), B, ctypes.byref(cw), ctypes.byref(p.c()) if p is not None else None,
                                     input_keep, ffn_sparsity, ctypes.byref(opt), _ptr(residual), _ptr(out),
                                     _ptr(sel_out), _ptr(workspace), workspace.numel(), _stream(x.device))
        _check(st, "prox_ffn_forward_ex")
        return out
    cp = p.c()
    if residual is None:
        st = lib.prox_ffn_forward(_ptr(x), B, ctypes.byref(cw), ctypes.byref(cp), input_keep, ffn_sparsity,
                                  _ptr(out), _ptr(sel_out), _ptr(workspace), workspace.numel(), _stream(x.device))
    else:
        st = lib.prox_ffn_forward_residual(_ptr(x), B, ctypes.byref(cw), ctypes.byref(cp), input_keep,
                                           ffn_sparsity, _ptr(residual), _ptr(out), _ptr(sel_out),
                                           _ptr(workspace), workspace.numel(), _stream(x.device))
    _check(st, "prox_ffn_forward")
    return out


def ffn_forward_noalloc(x: torch.Tensor, w: Weights, p: Proxy, input_keep: float, ffn_sparsity: float,
                        out: torch.Tensor, sel_out: torch.Tensor = None, residual: torch.Tensor = None) -> torch.Tensor:
    """ffn_forward on the library's own per-device workspace array: no device
    memory is allocated by the library (out and sel_out are the caller's).
    Calls that may overlap in time on one device race."""
    lib = load_library()
    _dev(x, "x")
    st = lib.prox_ffn_forward_noalloc(_ptr(x), x.shape[0], ctypes.byref(w.c()), ctypes.byref(p.c()), input_keep,
                                      ffn_sparsity, _ptr(residual), _ptr(out), _ptr(sel_out), _stream(x.device))
    _check(st, "prox_ffn_forward_noalloc")
    return out


def read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """XOR of every 32-bit word of buf (its bytes a multiple of 16) into
    sink[0] (int32, device): one stream read of buf, for timing."""
    lib = load_library()
    _dev(buf, "buf")
    _check(lib.prox_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf.device)),
           "prox_read_probe")


STEP_NAMES = ("xselect", "proxy", "topk", "gateup", "down")


def ffn_forward_timed(x: torch.Tensor, w: Weights, p: Proxy, input_keep: float, ffn_sparsity: float,
                      events, out: torch.Tensor = None, workspace: torch.Tensor = None) -> torch.Tensor:
    """prox_ffn_forward recording six torch.cuda.Event(enable_timing=True) around its steps."""
    lib = load_library()
    _dev(x, "x")
    B = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(w.d_model, w.d_ff, B, _mode_name(p), x.device)
    for e in events:  # torch creates the HIP event lazily on first record
        if e.cuda_event == 0:
            e.record()
    handles = (ctypes.c_void_p * 6)(*[e.cuda_event for e in events])
    cw, cp = w.c(), p.c()
    _check(lib.prox_ffn_forward_timed(_ptr(x), B, ctypes.byref(cw), ctypes.byref(cp), input_keep, ffn_sparsity,
                                      _ptr(out), None, _ptr(workspace), workspace.numel(), _stream(x.device),
                                      handles), "prox_ffn_forward_timed")
    return out


def stage1_select(x: torch.Tensor, w: Weights, p: Proxy, input_keep: float, ffn_sparsity: float,
                  with_scores: bool = False, workspace: torch.Tensor = None, sel_out: torch.Tensor = None):
    """Stage 1 alone: returns sel_idx (int32 [k], ascending) and, optionally, scores [F]."""
    lib = load_library()
    _dev(x, "x")
    B = x.shape[0]
    _, k = counts(w.d_model, w.d_ff, input_keep, ffn_sparsity)
    sel = sel_out if sel_out is not None else torch.empty(max(k, 1), dtype=torch.int32, device=x.device)
    scores = torch.empty(w.d_ff, dtype=torch.float32, device=x.device) if with_scores else None
    if workspace is None:
        workspace = alloc_workspace(w.d_model, w.d_ff, B, _mode_name(p), x.device)
    cw, cp = w.c(), p.c()
    _check(lib.prox_stage1_select(_ptr(x), B, ctypes.byref(cw), ctypes.byref(cp), input_keep, ffn_sparsity,
                                  _ptr(sel), _ptr(scores), _ptr(workspace), workspace.numel(),
                                  _stream(x.device)), "prox_stage1_select")
    sel = sel[:k]
    return (sel, scores) if with_scores else sel


def topk(scores: torch.Tensor, k: int) -> torch.Tensor:
    lib = load_library()
    _dev(scores, "scores")
    sel = torch.empty(max(k, 1), dtype=torch.int32, device=scores.device)
    _check(lib.prox_topk(_ptr(scores), scores.numel(), k, _ptr(sel), None, 0, _stream(scores.device)), "prox_topk")
    return sel[:k]


def stage2_exact(x: torch.Tensor, w: Weights, sel: torch.Tensor, out: torch.Tensor = None,
                 workspace: torch.Tensor = None, activation: str = "silu",
                 wait_limit_ticks: int = 0) -> torch.Tensor:
    lib = load_library()
    _dev(x, "x")
    B = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(w.d_model, w.d_ff, B, "int8_row", x.device)
    cw = w.c()
    sel = sel.to(torch.int32).contiguous() if sel.numel() else sel
    if activation != "silu" or wait_limit_ticks:
        opt = _COptions(ACTIVATIONS[activation], 0, wait_limit_ticks)
        _check(lib.prox_stage2_exact_ex(_ptr(x), B, ctypes.byref(cw), _ptr(sel) if sel.numel() else None,
                                        sel.numel(), ctypes.byref(opt), _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream(x.device)), "prox_stage2_exact_ex")
        return out
    _check(lib.prox_stage2_exact(_ptr(x), B, ctypes.byref(cw), _ptr(sel) if sel.numel() else None, sel.numel(),
                                 _ptr(out), _ptr(workspace), workspace.numel(), _stream(x.device)),
           "prox_stage2_exact")
    return out


def rmsnorm(h: torch.Tensor, eps: float = 1e-5, out: torch.Tensor = None) -> torch.Tensor:
    lib = load_library()
    _dev(h, "h")
    if out is None:
        out = torch.empty_like(h)
    _check(lib.prox_rmsnorm(_ptr(h), h.shape[0], h.shape[1], _dtype_code(h.dtype), eps, _ptr(out),
                            _stream(h.device)), "prox_rmsnorm")
    return out


def chain_workspace_size(d: int, F: int, batch: int, mode: str = "int8_row") -> int:
    return workspace_size(d, F, batch, mode) + 256 + batch * d * 4


def chain_forward(h: torch.Tensor, layers, proxies, input_keep: float, ffn_sparsity: float, eps: float = 1e-5,
                  workspace: torch.Tensor = None) -> torch.Tensor:
    """In place: for each layer, h <- h + FFN_l(RMSNorm(h)).  Returns h."""
    lib = load_library()
    _dev(h, "h")
    B = h.shape[0]
    L = len(layers)
    cws = (_CWeights * L)(*[w.c() for w in layers])
    cps = (_CProxy * L)(*[p.c() for p in proxies])
    if workspace is None:
        workspace = workspace_init(torch.empty(chain_workspace_size(layers[0].d_model, layers[0].d_ff, B,
                                                                    _mode_name(proxies[0])),
                                               dtype=torch.uint8, device=h.device))
    _check(lib.prox_chain_forward(_ptr(h), B, cws, cps, L, eps, input_keep, ffn_sparsity, _ptr(workspace),
                                  workspace.numel(), _stream(h.device)), "prox_chain_forward")
    return h
