"""prox_ffn_forward_noalloc: the forward on the library's static per-device
workspace, for callers that cannot allocate device memory.

Checked against the entry point with a caller-provided workspace
(prox_ffn_forward / prox_ffn_forward_residual), bitwise on the output and
the mask, over calls in a row on one device: the 8B-shape layer, then a
smaller layer with a residual, then a batch of four, then an int4-proxy
layer of 16416 channels (its top-k a second launch), then the first layer
again (the array keeps the previous call's contents; the counters must be
back at zero for each next call).  The outputs also meet the oracle's
acceptance rules.  No device memory is taken by the calls once the array is
loaded.  A layer too large for the array is refused on the host.  Forwards
captured in a HIP graph and replayed give the eager output bitwise."""
import numpy as np
import pytest
import torch

import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, log, run_and_check, to_dev

pytestmark = pytest.mark.gpu


def _pair(L, x_host, keep, sp, residual=None, mode="int8_row"):
    """The no-alloc call and the workspace call on the same inputs; both
    outputs and masks must be bitwise equal.  Returns the change in free
    device memory across a second no-alloc call on the same inputs (the
    first may load kernels into the device for the first time)."""
    B = x_host.shape[0]
    x = to_dev(x_host)
    k = P.counts(L.d, L.F, keep, sp)[1]
    res = to_dev(residual) if residual is not None else None
    out_a = torch.empty_like(x)
    sel_a = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    P.ffn_forward_noalloc(x, L.w, L.proxy(mode), keep, sp, out_a, sel_out=sel_a, residual=res)
    ws = P.alloc_workspace(L.d, L.F, B, mode)
    sel_b = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    out_b = P.ffn_forward(x, L.w, L.proxy(mode), keep, sp, sel_out=sel_b, residual=res, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.uint8), out_b.view(torch.uint8)), "outputs differ"
    assert torch.equal(sel_a, sel_b), "masks differ"
    free0 = torch.cuda.mem_get_info()[0]
    P.ffn_forward_noalloc(x, L.w, L.proxy(mode), keep, sp, out_a, sel_out=sel_a, residual=res)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert torch.equal(out_a.view(torch.uint8), out_b.view(torch.uint8)), "outputs differ on the repeat"
    return free1 - free0


def test_noalloc_matches_workspace_calls():
    big = Layer(4096, 14336, 0.02, "bf16", seed=0)
    small = Layer(1024, 2048, 0.05, "bf16", seed=1)
    x_big = synth.make_x(1, 4096, "bf16", seed=0)
    x_small = synth.make_x(1, 1024, "bf16", seed=2)
    r_small = synth.make_x(1, 1024, "bf16", seed=3)
    x_b4 = synth.make_x(4, 1024, "bf16", seed=4)
    wide = Layer(1024, 16416, 0.02, "bf16", seed=5)  # int4 beyond 16384 channels: scores, then the top-k launch
    x_wide = synth.make_x(1, 1024, "bf16", seed=6)
    d0 = _pair(big, x_big, 0.5, 0.7)                 # first call on the device: the array is set up
    d1 = _pair(small, x_small, 0.5, 0.7, r_small)    # a smaller layer, with a residual
    d2 = _pair(small, x_b4, 0.5, 0.6)                # a batch of four
    d4 = _pair(wide, x_wide, 0.5, 0.7, mode="int4_g128")
    d3 = _pair(big, x_big, 0.5, 0.7)                 # the first layer again
    log("free device memory change across repeated no-alloc calls: %d, %d, %d, %d, %d bytes" % (d0, d1, d2, d4, d3))
    assert d0 == 0 and d1 == 0 and d2 == 0 and d4 == 0 and d3 == 0
    # and that result (bitwise the same on both entry points) meets the oracle's acceptance rules
    run_and_check(small, x_small, "int8_row", 0.5, 0.7, residual=r_small, label="small layer with residual")


def test_noalloc_refuses_layers_beyond_the_array():
    size = P.workspace_size(8192, 28672, 16, "int8_row")
    assert size > P.STATIC_SCRATCH_BYTES
    w = P.Weights(torch.empty(0, dtype=torch.bfloat16, device="cuda"), torch.empty(0, dtype=torch.bfloat16, device="cuda"),
                  8192, 28672)
    p = P.Proxy(torch.empty(0, device="cuda"), torch.empty(0, device="cuda"), 0, 8192, 28672)
    x = torch.zeros(16, 8192, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P.ProxError) as e:
        P.ffn_forward_noalloc(x, w, p, 0.5, 0.7, torch.empty_like(x))
    assert e.value.status == P.ERR_SCRATCH_LIMIT


def test_noalloc_under_graph_capture():
    """The callers this entry point serves capture it: after a first call has
    set the array up, forwards captured in a HIP graph and replayed (with eager
    calls between the replays) give the eager output bitwise."""
    L = Layer(4096, 14336, 0.02, "bf16", seed=5)
    x = to_dev(synth.make_x(1, 4096, "bf16", seed=6))
    p = L.proxy("int8_row")
    ref = torch.empty_like(x)
    P.ffn_forward_noalloc(x, L.w, p, 0.5, 0.7, ref)
    torch.cuda.synchronize()
    out = torch.empty_like(x)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(3):
                P.ffn_forward_noalloc(x, L.w, p, 0.5, 0.7, out)
    torch.cuda.synchronize()
    eager = torch.empty_like(x)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        P.ffn_forward_noalloc(x, L.w, p, 0.5, 0.7, eager)  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), ref.view(torch.int16))
