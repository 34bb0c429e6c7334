"""Sparsity allocation on the device it plans for (technical summary, Sparsity
Allocation: Stage-2 sparsity anchored near 70%, Stage 1 keeping at least 30%
of the inputs, a cost model choosing both for a target effective sparsity).

On the 8B-shape layer: Stage 1 is timed live at four input-keep fractions
and Stage 2 at five kept-channel fractions, a straight line is fitted to
each, the dense layer is timed as the unit, and prox_allocate_sparsity
plans (input_keep, ffn_sparsity) for target effective sparsities.  Each plan
must keep at least the 30% floor, equal the oracle's planner on the same
fitted model, meet its target under the model, and its forward must pass
both acceptance rules against the oracle; the planned layer is timed and
the measured effective sparsity reported beside the predicted one."""
import numpy as np
import pytest
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, log, run_and_check, to_dev

pytestmark = pytest.mark.gpu

D, F = 4096, 14336
MIN_KEEP, ANCHOR = 0.3, 0.7


def _live_us(fn, n=40, warm=5):
    for i in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / n


def test_cost_model_fitted_on_device_plans_admissible_layers():
    L = Layer(D, F, 0.02, "bf16", seed=0)
    x_host = synth.make_x(1, D, "bf16", seed=0)
    x = to_dev(x_host)
    w, p = L.w, L.proxy("int8_row")
    ws = P.alloc_workspace(D, F, 1, "int8_row")
    out = torch.empty_like(x)
    sel = torch.empty(F, dtype=torch.int32, device="cuda")

    keeps = [0.3, 0.5, 0.7, 1.0]
    t1 = [_live_us(lambda kp=kp: P.stage1_select(x, w, p, kp, ANCHOR, workspace=ws, sel_out=sel)) for kp in keeps]
    kappas = [0.1, 0.3, 0.5, 0.7, 0.9]
    rng = np.random.default_rng(7)
    t2 = []
    for kap in kappas:
        sk = torch.from_numpy(np.sort(rng.choice(F, int(round(kap * F)), replace=False)).astype(np.int32)).cuda()
        t2.append(_live_us(lambda sk=sk: P.stage2_exact(x, w, sk, out=out, workspace=ws)))
    t_dense = _live_us(lambda: P.ffn_forward(x, w, p, 0.5, 0.0, out=out, workspace=ws))
    b1, a1 = np.polyfit(keeps, t1, 1)
    b2, a2 = np.polyfit(kappas, t2, 1)
    model = (max(a1, 0.0), max(b1, 0.0), max(a2, 0.0), b2, t_dense)
    log("stage 1 us %s, stage 2 us %s, dense %.2f us; model t1 = %.2f + %.2f keep, t2 = %.2f + %.2f kappa"
        % ([round(v, 2) for v in t1], [round(v, 2) for v in t2], t_dense, model[0], model[1], model[2], model[3]))
    # Stage 2 grows with the kept channels, close to a line (its rows are the bulk of its bytes)
    assert b2 > 0
    fit2 = np.polyval([b2, a2], kappas)
    assert np.max(np.abs(fit2 - t2) / np.asarray(t2)) < 0.2, "stage 2 is far from linear in the kept fraction"
    assert t_dense > 0

    planned = 0
    for target in (0.3, 0.4):
        plan = P.allocate_sparsity(model, target, ANCHOR, MIN_KEEP)
        ref = oracle.allocate_sparsity(model, target, ANCHOR, MIN_KEEP)
        if plan is None:
            assert ref is None
            log("target %.2f: out of reach on this device" % target)
            continue
        keep, sp = plan
        assert ref is not None and abs(ref[0] - keep) < 1e-9 and abs(ref[1] - sp) < 1e-9
        assert keep >= MIN_KEEP - 1e-12 and keep <= 1.0 and 0.0 <= sp <= 1.0
        assert abs(P.effective_sparsity(model, keep, sp) - target) < 1e-9
        # the planned layer is an admissible Prox forward
        run_and_check(L, x_host, "int8_row", keep, sp, label="planned target %.2f keep %.3f sp %.3f"
                      % (target, keep, sp))
        t_plan = _live_us(lambda: P.ffn_forward(x, w, p, keep, sp, out=out, workspace=ws))
        log("target %.2f: keep %.3f, sparsity %.3f; predicted %.2f us, measured %.2f us, measured effective "
            "sparsity %.3f" % (target, keep, sp, (1.0 - target) * t_dense, t_plan, 1.0 - t_plan / t_dense))
        assert t_plan < t_dense
        planned += 1
    assert planned > 0, "no target was reachable"
