"""Stage 2's bounded waits, forced to give up from the host.

The single-token Stage 2 hands s values and split partials between its
workgroups through bounded waits.  A wait that gives up must not change the
result: the workgroup computes what it waited for itself.  Here the host
sets the bound to one tick (10 ns), so nearly every wait gives up, and the
output must equal, bitwise, the run with the default bound; the workspace
counters must be back at zero afterwards and the give-ups counted.  Every
kernel exits normally: nothing here stalls or faults the device."""
import numpy as np
import pytest
import torch

import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, TOL, from_dev, log, out_error, to_dev

import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,F,std,sp,dt", [(4096, 14336, 0.02, 0.7, "bf16"), (1000, 1040, 0.05, 0.3, "bf16"),
                                           (512, 1376, 0.02, 0.5, "f32")])
def test_forced_wait_give_up_is_exact(d, F, std, sp, dt):
    L = Layer(d, F, std, dt, seed=3)
    x_host = synth.make_x(1, d, dt, seed=3)
    x = to_dev(x_host)
    mode = "int8_row"
    ws = P.alloc_workspace(d, F, 1, mode)
    _, k = P.counts(d, F, 0.5, sp)
    sel = torch.empty(k, dtype=torch.int32, device="cuda")
    # the default two-launch path, whose Stage 2 hands work over through bounded waits
    ref = P.ffn_forward(x, L.w, L.proxy(mode), 0.5, sp, sel_out=sel, workspace=ws)
    assert P.workspace_check(ws) == 0
    for rep in range(2):  # twice: the first forced run must leave the workspace clean for the next
        out = P.ffn_forward(x, L.w, L.proxy(mode), 0.5, sp, workspace=ws, wait_limit_ticks=1)
        n_fb = P.workspace_check(ws)
        log("d=%d F=%d k=%d forced run %d: %d waits gave up" % (d, F, k, rep, n_fb))
        assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8))
    assert n_fb > 0, "no wait gave up: the fallback path was not exercised"
    # Stage 2 alone on the same mask, forced, and again with the default bound
    o2 = P.stage2_exact(x, L.w, sel, workspace=ws, wait_limit_ticks=1)
    assert torch.equal(o2.view(torch.uint8), ref.view(torch.uint8))
    o3 = P.stage2_exact(x, L.w, sel, workspace=ws)
    assert torch.equal(o3.view(torch.uint8), ref.view(torch.uint8))
    assert P.workspace_check(ws) >= n_fb
    # and the result is the oracle's masked FFN on that mask
    sel_np = sel.cpu().numpy().astype(np.int64)
    y_ref, _ = oracle.ffn_masked(x_host, L.wg, L.wu, L.wd, sel_np)
    assert out_error(from_dev(o2), y_ref) <= TOL[dt]


def test_workspace_check_flags_dirty_counters():
    """A counter left nonzero (as after a call stopped part-way) is reported."""
    ws = P.alloc_workspace(512, 1376, 1, "int8_row")
    assert P.workspace_check(ws) == 0
    ws[4096 * 4 + 1] = 1  # one byte of a Stage-2 arrival line
    with pytest.raises(P.ProxError):
        P.workspace_check(ws)
    P.workspace_init(ws)
    assert P.workspace_check(ws) == 0
