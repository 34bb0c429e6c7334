"""GPU parity of Stage 2 for batches (2..16 tokens, bf16 activations), which
runs on the matrix cores: gate/up tiles of 16 channels x 16 token slots with
the input dimension split over workgroups, and the down projection over rank
splits with s carried as three exact bf16 pieces.

Each case compares with the oracle's masked SwiGLU (binary64) on the same
mask, at shapes that leave ragged tiles everywhere: k not a multiple of 16
or 32 (the last gate/up tile, the zero-filled ranks up to 32), d not a
multiple of 1024 or 128 (the last input chunk and column tile), B below 16
(empty token slots), and one input chunk or several.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, TOL, from_dev, log, out_error, to_dev
from tests.test_gpu_fp8 import Fp8Layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    P.load_library()
    torch.cuda.init()


def _check(L, B, ks, seed, act="silu"):
    x = synth.make_x(B, L.d, "bf16", seed=seed)
    rng = np.random.default_rng(seed)
    for k in ks:
        sel = np.sort(rng.choice(L.F, size=k, replace=False)).astype(np.int32)
        log("batch stage2 d=%d F=%d B=%d k=%d act=%s" % (L.d, L.F, B, k, act))
        y = from_dev(P.stage2_exact(to_dev(x), L.w, torch.from_numpy(sel).cuda(), activation=act))
        torch.cuda.synchronize()
        if hasattr(L, "fp8"):
            y_ref, _ = oracle.ffn_masked_fp8(x, L.fp8, sel.astype(np.int64), act=act)
        else:
            y_ref, _ = oracle.ffn_masked(x, L.wg, L.wu, L.wd, sel.astype(np.int64), act=act)
        err = out_error(y, y_ref)
        assert err <= TOL["bf16"], (k, err)


@pytest.mark.parametrize("d,F,B", [(1000, 2048, 2), (1024, 1040, 16), (2048, 5632, 8), (8192, 1024, 3),
                                   (1536, 3008, 5)])
def test_batch_stage2_given_mask(d, F, B):
    L = Layer(d, F, 0.02, "bf16", seed=61)
    _check(L, B, (1, 15, 17, 33, F // 3 + 1, F), seed=61)


@pytest.mark.parametrize("d,F,B", [(1000, 4160, 3), (1536, 4112, 16)])
def test_batch_stage2_whole_and_chunked_tiles(d, F, B):
    # k = F gives 260 and 257 gate/up tiles: 256 run whole, the rest in
    # 512-input chunks (1000 = 512 + 488 inputs, 1536 = 3 x 512) whose sums
    # meet through a ticket; F // 3 + 1 stays below 256 tiles (chunks of 1024)
    L = Layer(d, F, 0.02, "bf16", seed=67)
    _check(L, B, (F, F - 5, F // 3 + 1), seed=67)


@pytest.mark.parametrize("B", [4, 16])
def test_batch_stage2_8b_shape(B):
    # the 4096 x 14336 layer at sparsity 0.7 (k = 4301) and every channel
    L = Layer(4096, 14336, 0.02, "bf16", seed=62)
    _check(L, B, (4301, 14336), seed=62)


def test_batch_stage2_geglu():
    L = Layer(1024, 2048, 0.02, "bf16", seed=63)
    _check(L, 4, (37, 700), seed=63, act="gelu_tanh")


@pytest.mark.parametrize("d,F,B", [(1024, 2048, 2), (832, 1200, 16), (4096, 14336, 16)])
def test_batch_stage2_fp8(d, F, B):
    L = Fp8Layer(d, F, 0.02, "bf16", seed=64)
    _check(L, B, (17, F // 3 + 1), seed=64)


def test_batch_deterministic():
    L = Layer(4096, 14336, 0.02, "bf16", seed=65)
    x = to_dev(synth.make_x(16, 4096, "bf16", seed=65))
    sel = torch.from_numpy(np.sort(np.random.default_rng(65).choice(14336, 4301, replace=False))
                           .astype(np.int32)).cuda()
    outs = [P.stage2_exact(x, L.w, sel).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


def test_batch_forward_every_channel_writes_iota():
    # sparsity 0: Stage 1 is skipped, the mask written is 0 .. F-1
    L = Layer(1024, 1040, 0.02, "bf16", seed=66)
    x = synth.make_x(3, 1024, "bf16", seed=66)
    sel = torch.full((1040,), -1, dtype=torch.int32, device="cuda")
    y = from_dev(P.ffn_forward(to_dev(x), L.w, L.proxy("int8_row"), 0.5, 0.0, sel_out=sel))
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), np.arange(1040))
    y_ref, _ = oracle.ffn_dense(x, L.wg, L.wu, L.wd)
    assert out_error(y, y_ref) <= TOL["bf16"]
