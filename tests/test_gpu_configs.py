"""GPU parity at the full sizes of the five evaluated workloads, in the
launch configuration the benchmark times: the 512x1376 fp32 toy layer, the
7B-like 4096x11008 layer (0/50/70/90% sparsity), the 8B-like 4096x14336
layer (B = 1, 4, 16), the 70B-like 8192x28672 layer (int4-g128 and int8
proxies, 50/70/90%).  The oracle computes every output element at these
sizes.  The 32-layer stack of 8B-like layers is in test_gpu_chain.py."""
import numpy as np
import pytest
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, TOL, from_dev, log, out_error, run_and_check, to_dev

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
_cache = {}


def layer(name, layer_idx=0):
    key = (name, layer_idx)
    if key not in _cache:
        w = W[name]
        log("building layer", key)
        _cache.clear() if name == "llama70b" else None
        _cache[key] = Layer(w.d, w.F, w.std, w.dtype, seed=0, layer=layer_idx)
    return _cache[key]


def test_toy_fp32():
    w = W["toy_fp32"]
    r = run_and_check(layer("toy_fp32"), synth.make_x(1, w.d, w.dtype, seed=0), w.mode, w.input_keep,
                      w.sparsities[0], label="toy_fp32")
    assert r["err"] <= 1e-5


@pytest.mark.parametrize("sp", W["llama7b"].sparsities)
def test_llama7b(sp):
    w = W["llama7b"]
    run_and_check(layer("llama7b"), synth.make_x(1, w.d, w.dtype, seed=0), w.mode, w.input_keep, sp,
                  label="llama7b sp=%g" % sp)


@pytest.mark.parametrize("B", W["llama8b"].batches)
def test_llama8b(B):
    w = W["llama8b"]
    run_and_check(layer("llama8b"), synth.make_x(B, w.d, w.dtype, seed=0), w.mode, w.input_keep,
                  w.sparsities[0], label="llama8b B=%d" % B)


@pytest.mark.parametrize("mode", ["int4_g128", "int8_row"])
@pytest.mark.parametrize("sp", W["llama70b"].sparsities)
def test_llama70b(mode, sp):
    w = W["llama70b"]
    run_and_check(layer("llama70b"), synth.make_x(1, w.d, w.dtype, seed=0), mode, w.input_keep, sp,
                  label="llama70b %s sp=%g" % (mode, sp))
