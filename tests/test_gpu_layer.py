"""The single-launch layer (opt-in, PROX_FLAG_SINGLE_LAUNCH): both stages of
one bf16 token (bf16 weights, int8 proxy, d_model 4096 or 8192, d_ff <= 16384)
in one launch of one workgroup per CU.

Parity against the oracle by the two acceptance rules on the workloads it
serves, edge cases of both selections (ties in |x| and in the scores, the
smallest and largest k, k_in down to a handful), ragged channel blocks,
every selection signal and activation, the residual in place,
determinism, clean counters, and a forced give-up of
its grid-barrier waits (reported as an error, output NaN; the kernels still
exit normally)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, TOL, from_dev, log, out_error, run_and_check, to_dev

pytestmark = pytest.mark.gpu

SL = {"single_launch": True}

_layers = {}


def layer(d, F, std=0.02, seed=0, pattern=None):
    key = (d, F, std, seed, pattern)
    if key not in _layers:
        if len(_layers) > 3:
            _layers.clear()
        _layers[key] = Layer(d, F, std, "bf16", seed=seed, pattern=pattern)
    return _layers[key]


def test_8b_shape_both_paths():
    """The benchmark layer through one launch and through separate stages:
    both admissible against the oracle, masks equal up to near-ties."""
    L = layer(4096, 14336)
    x = synth.make_x(1, 4096, "bf16", seed=0)
    r1 = run_and_check(L, x, "int8_row", 0.5, 0.7, label="layer 8b", **SL)
    xt = to_dev(x)
    k = r1["ref"]["k"]
    sel2 = torch.empty(k, dtype=torch.int32, device="cuda")
    o2 = P.ffn_forward(xt, L.w, L.proxy("int8_row"), 0.5, 0.7, sel_out=sel2)
    s2 = sel2.cpu().numpy().astype(np.int64)
    ok, msg = oracle.mask_admissible(s2, r1["ref"]["sel"], r1["ref"]["score"], r1["ref"]["T"], k)
    assert ok, msg
    log("one launch vs separate stages: masks differ in %d channels, outputs max diff %.3g"
        % (len(set(s2.tolist()) ^ set(r1["sel"].tolist())), float(np.abs(from_dev(o2) - r1["y"]).max())))


@pytest.mark.parametrize("sp", [0.5, 0.7, 0.9])
def test_7b_shape(sp):
    run_and_check(layer(4096, 11008), synth.make_x(1, 4096, "bf16", seed=1), "int8_row", 0.5, sp,
                  label="layer 7b sp=%g" % sp, **SL)


def test_deterministic_and_clean():
    L = layer(4096, 14336)
    x = to_dev(synth.make_x(1, 4096, "bf16", seed=5))
    ws = P.alloc_workspace(4096, 14336, 1)
    outs = []
    for _ in range(3):
        sel = torch.empty(4301, dtype=torch.int32, device="cuda")
        outs.append((P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, 0.7, sel_out=sel, workspace=ws, **SL).clone(), sel))
        assert P.workspace_check(ws) == 0
    for o, s in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(s, outs[0][1])
    # the mask output is optional and changes nothing
    o = P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, 0.7, workspace=ws, **SL)
    assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))


@pytest.mark.parametrize("pattern", ["dup", "zeros"])
def test_score_ties(pattern):
    # dup: every proxy score occurs twice; zeros: 80% of the channels score exactly 0
    L = layer(4096, 2048, std=0.03, seed=2, pattern=pattern)
    for sp in (0.5, 0.9):
        run_and_check(L, synth.make_x(1, 4096, "bf16", seed=3), "int8_row", 0.5, sp,
                      label="layer ties %s sp=%g" % (pattern, sp), **SL)


def test_input_magnitude_ties():
    L = layer(4096, 2048, std=0.03, seed=4)
    x = synth.make_x(1, 4096, "bf16", seed=6)
    x[0, ::3] = x[0, 7]  # a third of the inputs share one magnitude, some with either sign
    x[0, 1::6] = x[0, 7] ^ 0x8000
    for keep in (0.3, 0.5, 0.8):
        run_and_check(L, x, "int8_row", keep, 0.6, label="layer |x| ties keep=%g" % keep, **SL)


@pytest.mark.parametrize("keep,sp", [(0.5, 1.0 - 1.5 / 2048), (0.5, 1.0 / 2048), (1.0, 0.7), (0.02, 0.7),
                                     (0.001, 0.5)])
def test_extreme_counts(keep, sp):
    # k = 1, k = F - 1, every input kept, and a few dozen or a handful of kept inputs
    L = layer(4096, 2048, std=0.03, seed=8)
    run_and_check(L, synth.make_x(1, 4096, "bf16", seed=9), "int8_row", keep, sp,
                  label="layer keep=%g sp=%g" % (keep, sp), **SL)


@pytest.mark.parametrize("d,F", [(4096, 4112), (4096, 16384), (8192, 2064), (8192, 16384)])
def test_ragged_and_large(d, F):
    # d_ff not a multiple of the 1024-channel proxy block; the largest d_ff; d_model 8192
    run_and_check(layer(d, F, std=0.02, seed=10), synth.make_x(1, d, "bf16", seed=11), "int8_row", 0.45, 0.65,
                  label="layer %dx%d" % (d, F), **SL)


@pytest.mark.parametrize("act,signal", [("silu", "h"), ("silu", "u"), ("gelu_tanh", "s"), ("gelu_tanh", "h")])
def test_signals_and_activations(act, signal):
    L = layer(4096, 2048, std=0.03, seed=12)
    x = synth.make_x(1, 4096, "bf16", seed=13)
    xt = to_dev(x)
    k = P.counts(4096, 2048, 0.5, 0.7)[1]
    sel = torch.empty(k, dtype=torch.int32, device="cuda")
    out = P.ffn_forward(xt, L.w, L.proxy("int8_row"), 0.5, 0.7, sel_out=sel, activation=act, signal=signal, **SL)
    torch.cuda.synchronize()
    ref = oracle.prox_forward(x, L.wg, L.wu, L.wd, L.oracle_proxy("int8_row"), 0.5, 0.7, "int8_row", act=act,
                              signal=signal)
    s = sel.cpu().numpy().astype(np.int64)
    ok, msg = oracle.mask_admissible(s, ref["sel"], ref["score"], ref["T"], k)
    assert ok, msg
    y_ref, _ = oracle.ffn_masked(x, L.wg, L.wu, L.wd, s, act)
    err = out_error(from_dev(out), y_ref)
    log("layer %s/%s mask %s err %.3g" % (act, signal, msg, err))
    assert err <= TOL["bf16"]


def test_residual_in_place():
    L = layer(4096, 2048, std=0.03, seed=14)
    x = to_dev(synth.make_x(1, 4096, "bf16", seed=15))
    r = synth.make_x(1, 4096, "bf16", seed=16)
    rt = to_dev(r)
    ref = P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, 0.7, residual=to_dev(r), **SL)
    out = P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, 0.7, residual=rt, out=rt, **SL)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    run_and_check(L, synth.make_x(1, 4096, "bf16", seed=15), "int8_row", 0.5, 0.7, residual=r, label="layer res", **SL)


def test_forced_barrier_give_up_is_reported():
    """Grid-barrier waits bounded to one tick give up: the call's output is
    NaN and the workspace check reports the failure; after a zero fill the
    workspace serves a normal call again."""
    L = layer(4096, 2048, std=0.03, seed=19)
    x = to_dev(synth.make_x(1, 4096, "bf16", seed=20))
    ws = P.alloc_workspace(4096, 2048, 1)
    good = P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, 0.7, workspace=ws, **SL)
    assert P.workspace_check(ws) == 0
    bad = P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, 0.7, workspace=ws, wait_limit_ticks=1, **SL)
    with pytest.raises(P.ProxError):
        P.workspace_check(ws)
    n_nan = int(torch.isnan(bad.float()).sum().item())
    log("forced give-up: %d of 4096 outputs NaN" % n_nan)
    assert n_nan > 0
    P.workspace_init(ws)
    again = P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, 0.7, workspace=ws, **SL)
    assert P.workspace_check(ws) == 0
    assert torch.equal(again.view(torch.int16), good.view(torch.int16))
