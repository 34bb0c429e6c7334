"""The single-token bf16 Stage 2 on whole-channel streams (stage2_rows_kernel,
d_model 4096 and 8192): parity on given masks against the oracle's masked
FFN across the ways the selected channels fall on the workgroups (fewer
channels than workgroups, one more or one fewer than a multiple, every
channel), the dense forward with the mask output, GeGLU, mask entries out of
range (clamped, as every Stage 2 does), determinism, and its bounded waits
forced to give up at both widths (the result must not change)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, TOL, from_dev, log, out_error, run_and_check, to_dev

pytestmark = pytest.mark.gpu

_layers = {}


def layer(d, F):
    if (d, F) not in _layers:
        _layers.clear()
        _layers[(d, F)] = Layer(d, F, 0.02, "bf16", seed=31)
    return _layers[(d, F)]


def _check_mask(L, x, sel, act="silu", **kw):
    out = P.stage2_exact(to_dev(x), L.w, torch.from_numpy(sel).to("cuda"), activation=act, **kw)
    torch.cuda.synchronize()
    y_ref, _ = oracle.ffn_masked(x, L.wg, L.wu, L.wd, np.clip(sel, 0, L.F - 1).astype(np.int64), act)
    err = out_error(from_dev(out), y_ref)
    assert err <= TOL["bf16"], (len(sel), err)
    return out, err


@pytest.mark.parametrize("d,F", [(4096, 64), (4096, 1040), (4096, 16400), (8192, 2064), (8192, 9008)])
def test_given_masks(d, F):
    L = layer(d, F)
    x = synth.make_x(1, d, "bf16", seed=32)
    rng = np.random.default_rng(33)
    G = 256
    for k in sorted({1, 37, min(F, G - 1), min(F, G), min(F, G + 1), min(F, 3 * G - 1), F // 3, F}):
        sel = np.sort(rng.choice(F, size=k, replace=False)).astype(np.int32)
        _, err = _check_mask(L, x, sel)
        log("rows %dx%d k=%d err %.3g" % (d, F, k, err))


def test_dense_forward_writes_every_channel():
    L = layer(4096, 2048)
    x = synth.make_x(1, 4096, "bf16", seed=34)
    sel = torch.full((2048,), -1, dtype=torch.int32, device="cuda")
    out = P.ffn_forward(to_dev(x), L.w, L.proxy("int8_row"), 0.5, 0.0, sel_out=sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), np.arange(2048))
    y_ref = oracle.ffn_dense(x, L.wg, L.wu, L.wd)[0]
    assert out_error(from_dev(out), y_ref) <= TOL["bf16"]


def test_gelu_and_clamped_entries():
    L = layer(4096, 2048)
    x = synth.make_x(1, 4096, "bf16", seed=35)
    sel = np.sort(np.random.default_rng(36).choice(2048, size=600, replace=False)).astype(np.int32)
    _check_mask(L, x, sel, act="gelu_tanh")
    # entries outside [0, F) read the nearest valid row; the result equals that of the clamped mask
    bad = sel.copy()
    bad[0], bad[-1] = -5, 2048 + 7
    o_bad = P.stage2_exact(to_dev(x), L.w, torch.from_numpy(bad).cuda())
    o_clamped = P.stage2_exact(to_dev(x), L.w, torch.from_numpy(np.clip(bad, 0, 2047).astype(np.int32)).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o_bad.view(torch.int16), o_clamped.view(torch.int16))


def test_deterministic_across_calls():
    L = layer(8192, 2064)
    x = to_dev(synth.make_x(1, 8192, "bf16", seed=37))
    sel = torch.from_numpy(np.sort(np.random.default_rng(38).choice(2064, 700, replace=False)).astype(np.int32)).cuda()
    ws = P.alloc_workspace(8192, 2064, 1)
    outs = [P.stage2_exact(x, L.w, sel, workspace=ws).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert P.workspace_check(ws) == 0


@pytest.mark.parametrize("d,F,k", [(4096, 14336, 4301), (8192, 4096, 1229)])
def test_forced_give_up_is_exact(d, F, k):
    """A one-tick bound makes the slice workgroups' waits give up; each then
    recomputes every partial itself, and the output must not change."""
    L = layer(d, F)
    x = to_dev(synth.make_x(1, d, "bf16", seed=39))
    sel = torch.from_numpy(np.sort(np.random.default_rng(40).choice(F, k, replace=False)).astype(np.int32)).cuda()
    ws = P.alloc_workspace(d, F, 1)
    ref = P.stage2_exact(x, L.w, sel, workspace=ws).clone()
    assert P.workspace_check(ws) == 0
    for _ in range(2):
        out = P.stage2_exact(x, L.w, sel, workspace=ws, wait_limit_ticks=1)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    n_fb = P.workspace_check(ws)
    log("rows %dx%d forced: %d waits gave up" % (d, F, n_fb))
    assert n_fb > 0
    again = P.stage2_exact(x, L.w, sel, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), ref.view(torch.int16))
