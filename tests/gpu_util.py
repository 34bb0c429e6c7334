"""Helpers for the GPU parity tests: seeded layers on the device, unpacking of
the library's proxy layout (as documented in include/prox.h), and the
acceptance rules (mask within the near-tie window; per-token max-norm
relative output error against the oracle's Stage 2 on the GPU's own mask)."""
import sys

import numpy as np
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P

TOL = {"bf16": 1e-2, "f32": 1e-5}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def from_dev(t: torch.Tensor) -> np.ndarray:
    """float64 values of a device tensor (bf16 widened exactly)."""
    if t.dtype == torch.bfloat16:
        return oracle.as_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def unpack_proxy(p: P.Proxy):
    """Library proxy buffers -> (q_gate [F][d], sc_gate, q_up [F][d], sc_up) in the oracle's format."""
    d, F = p.d_model, p.d_ff
    codes = p.codes.cpu().numpy()
    scales = p.scales.cpu().numpy()
    if p.mode == P.MODES["int8_row"]:
        c = codes.view(np.int8).reshape(d, 2, F)
        s = scales.reshape(2, F)
        return c[:, 0, :].T.copy(), s[0].copy(), c[:, 1, :].T.copy(), s[1].copy()
    c = codes.reshape(d, 2, F // 2)
    s = scales.reshape(d // 128, 2, F)
    out = []
    for h in range(2):
        q = np.empty((d, F), dtype=np.int8)
        q[:, 0::2] = (c[:, h, :] & 0xF).astype(np.int8) - 8
        q[:, 1::2] = (c[:, h, :] >> 4).astype(np.int8) - 8
        out += [q.T.copy(), s[:, h, :].T.copy()]
    return out[0], out[1], out[2], out[3]


class Layer:
    """One seeded SwiGLU FFN layer on host (synth arrays) and device (packed).
    drop_host() frees the host arrays once the oracle no longer needs them."""

    def __init__(self, d, F, std, dtype, seed=0, layer=0, pattern=None):
        self.d, self.F, self.dtype = d, F, dtype
        self.wg, self.wu, self.wd = synth.make_weights(d, F, std, dtype, seed=seed, layer=layer)
        if pattern == "dup":  # channel j + F/2 repeats channel j: every proxy score occurs twice
            self.wg[F // 2:] = self.wg[:F // 2]
            self.wu[F // 2:] = self.wu[:F // 2]
        elif pattern == "zeros":  # 80% of the gate rows are zero: those channels score exactly 0
            rng = np.random.default_rng(seed)
            self.wg[rng.permutation(F)[: (4 * F) // 5]] = 0
        self.w = P.pack_weights(to_dev(self.wg), to_dev(self.wu), to_dev(self.wd))
        self._proxy = {}
        self._oproxy = {}

    def proxy(self, mode):
        if mode not in self._proxy:
            self._proxy[mode] = P.quantize_proxy(self.w, mode)
        return self._proxy[mode]

    def drop_host(self):
        self.wg = self.wu = self.wd = None
        self._oproxy = {}

    def oracle_proxy(self, mode):
        if mode not in self._oproxy:
            qg, scg = oracle.quantize(self.wg, mode)
            qu, scu = oracle.quantize(self.wu, mode)
            self._oproxy[mode] = (qg, scg, qu, scu)
        return self._oproxy[mode]


def out_error(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """max over tokens of max_m |y_gpu - y_ref| / max_m |y_ref|."""
    errs = []
    for b in range(y_ref.shape[0]):
        den = np.abs(y_ref[b]).max()
        num = np.abs(y_gpu[b] - y_ref[b]).max()
        errs.append(num / den if den > 0 else num)
    return float(max(errs))


def run_and_check(layer: Layer, x_host: np.ndarray, mode: str, keep: float, sp: float, residual=None,
                  label="", **fwd):
    """Run the GPU forward (keyword options `fwd` passed on to ffn_forward) and
    apply both acceptance rules.  Returns a dict of diagnostics."""
    B = x_host.shape[0]
    x = to_dev(x_host)
    k_in, k = P.counts(layer.d, layer.F, keep, sp)
    sel_t = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    res_t = to_dev(residual) if residual is not None else None
    ws = P.alloc_workspace(layer.d, layer.F, B, mode)
    out = P.ffn_forward(x, layer.w, layer.proxy(mode), keep, sp, sel_out=sel_t, residual=res_t, workspace=ws, **fwd)
    # counters back at zero, and no bounded wait gave up
    assert P.workspace_check(ws) == 0, "%s: a bounded wait gave up" % label
    torch.cuda.synchronize()
    y_gpu = from_dev(out)
    sel_gpu = sel_t[:k].cpu().numpy().astype(np.int64)
    ref = oracle.prox_forward(x_host, layer.wg, layer.wu, layer.wd, layer.oracle_proxy(mode), keep, sp, mode)
    assert ref["k"] == k and ref["k_in"] == k_in
    ok, msg = oracle.mask_admissible(sel_gpu, ref["sel"], ref["score"], ref["T"], k)
    assert ok, "%s mask: %s" % (label, msg)
    assert np.all(np.diff(sel_gpu) > 0) if k > 1 else True
    y_ref, _ = oracle.ffn_masked(x_host, layer.wg, layer.wu, layer.wd, sel_gpu)
    y_own = ref["y"]
    if residual is not None:
        r = oracle.as_f64(residual)
        y_ref = y_ref + r
        y_own = y_own + r
    err = out_error(y_gpu, y_ref) if k > 0 or residual is not None else float(np.abs(y_gpu).max())
    err_own = out_error(y_gpu, y_own) if k > 0 else err
    log("%s k_in=%d k=%d mask %s err=%.3g err_vs_oracle_mask=%.3g" % (label, k_in, k, msg, err, err_own))
    assert err <= TOL[layer.dtype], "%s output error %.3g > %.3g" % (label, err, TOL[layer.dtype])
    return dict(err=err, err_own=err_own, sel=sel_gpu, y=y_gpu, ref=ref, out=out)
