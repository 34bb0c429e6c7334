"""GPU parity: the HIP library against the CPU oracle, element by element.

Kernel-level: weight packing and proxy quantization bit-exact; the top-k
mask kernel bit-exact on identical score vectors (tie-heavy included);
Stage-1 scores within fp32 rounding and the mask within the near-tie
window; Stage 2 on a given mask within the output tolerance.  Whole
forward: small shapes spanning several tiles with ragged tails, edge cases
(k = 0, k = F, keep = 1, odd batches), determinism, residual add.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import Layer, TOL, from_dev, log, out_error, run_and_check, to_dev, unpack_proxy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    P.load_library()
    torch.cuda.init()


# ------------------------------------------------------------- offline

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_layout(dtype):
    d, F = 320, 208
    L = Layer(d, F, 0.02, dtype, seed=3)
    gu = from_dev(L.w.w_gu)
    dt = from_dev(L.w.w_down_t)
    f = oracle.as_f64
    np.testing.assert_array_equal(gu[:, 0, :], f(L.wg))
    np.testing.assert_array_equal(gu[:, 1, :], f(L.wu))
    np.testing.assert_array_equal(dt, f(L.wd).T)


@pytest.mark.parametrize("d,F,dtype,mode", [
    (256, 96, "f32", "int8_row"), (512, 1376, "bf16", "int8_row"), (384, 272, "bf16", "int4_g128"),
    (1024, 1040, "f32", "int4_g128"), (4096, 14336, "bf16", "int8_row"),
])
def test_quantize_bit_exact(d, F, dtype, mode):
    L = Layer(d, F, 0.02, dtype, seed=5)
    val = (lambda v: np.float32(v)) if dtype == "f32" else (lambda v: synth.f32_to_bf16_bits(np.float32([v]))[0])
    # planted: an all-zero row, a row whose absmax makes the scale exactly 1
    # with round-half-even ties, and (int4) an all-zero group
    L.wg[3, :] = val(0.0)
    L.wg[7, :] = val(0.0)
    L.wg[7, 10], L.wg[7, 11], L.wg[7, 12], L.wg[7, 13] = val(127.0), val(2.5), val(-3.5), val(126.5)
    if mode == "int4_g128":
        L.wu[2, 128:256] = val(0.0)
        L.wu[9, :128] = val(0.0)
        L.wu[9, 0], L.wu[9, 1], L.wu[9, 2] = val(7.0), val(2.5), val(-0.5)
    L.w = P.pack_weights(to_dev(L.wg), to_dev(L.wu), to_dev(L.wd))
    qg, scg, qu, scu = unpack_proxy(L.proxy(mode))
    oqg, oscg, oqu, oscu = L.oracle_proxy(mode)
    np.testing.assert_array_equal(scg, oscg)
    np.testing.assert_array_equal(scu, oscu)
    np.testing.assert_array_equal(qg, oqg)
    np.testing.assert_array_equal(qu, oqu)


# --------------------------------------------------------------- top-k

def _score_vectors():
    rng = np.random.default_rng(17)
    out = []
    for n in (16, 100, 1376, 4000, 14336, 28672, 65535):
        out.append(("normal", n, np.abs(rng.standard_normal(n)).astype(np.float32)))
    out.append(("ties", 14336, rng.integers(0, 7, 14336).astype(np.float32)))
    out.append(("all_equal", 5000, np.full(5000, 0.25, np.float32)))
    out.append(("zeros_and_ones", 3000, (rng.random(3000) < 0.3).astype(np.float32)))
    v = np.abs(rng.standard_normal(11008)).astype(np.float32)
    v[::7] = v[3]  # a heavy tie at an arbitrary level
    out.append(("planted_tie", 11008, v))
    out.append(("signed", 2048, rng.standard_normal(2048).astype(np.float32)))
    out.append(("wide_range", 8192, (np.exp(rng.uniform(-80, 80, 8192))).astype(np.float32)))
    out.append(("n1", 1, np.array([3.0], np.float32)))
    return out


@pytest.mark.parametrize("name,n,v", _score_vectors(), ids=[t[0] + str(t[1]) for t in _score_vectors()])
def test_topk_bit_exact(name, n, v):
    for frac in (0.0, 1.0 / n, 0.1, 0.3, 0.5, 0.7, 1.0):
        k = min(n, int(round(frac * n)))
        got = P.topk(to_dev(v), k).cpu().numpy().astype(np.int64)
        want, _ = oracle.topk_ascending(v.astype(np.float64), k)
        assert np.array_equal(got, want), (name, n, k)


# -------------------------------------------------------------- stages

def _tied_x(B, d, dtype, seed):
    """Inputs whose magnitudes take three values: input selection decides among ties."""
    rng = np.random.default_rng(seed)
    x = (rng.choice([0.5, 1.0, 2.0], size=(B, d)) * rng.choice([-1.0, 1.0], size=(B, d))).astype(np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("d,F,dtype,B,mode,pattern", [
    (512, 1376, "f32", 1, "int8_row", None), (1024, 2064, "bf16", 1, "int8_row", None),
    (768, 1040, "bf16", 3, "int8_row", None), (1024, 1536, "bf16", 1, "int4_g128", None),
    (640, 2000, "bf16", 4, "int4_g128", None), (512, 784, "bf16", 16, "int8_row", None),
    # exact ties among the scores (duplicated channels) and at zero (zeroed gate rows),
    # on the single-token kernel and on the batched path
    (1024, 2064, "bf16", 1, "int8_row", "dup"), (1024, 1536, "bf16", 1, "int4_g128", "dup"),
    (1024, 2064, "bf16", 1, "int8_row", "zeros"), (768, 1040, "bf16", 3, "int8_row", "zeros"),
    # tied input magnitudes
    (1024, 2064, "bf16", 1, "int8_row", "xties"), (2048, 4096, "f32", 1, "int8_row", "xties"),
    (768, 1040, "bf16", 2, "int8_row", "xties"),
    # the matrix-core proxy (bf16, more than 4 tokens): ties, and input splits
    # of a length that is not a multiple of 1024 (d = 2504: three splits of 864)
    (1024, 2064, "bf16", 6, "int8_row", "dup"), (768, 1040, "bf16", 8, "int8_row", "zeros"),
    (2504, 1040, "bf16", 8, "int8_row", None), (768, 1040, "bf16", 5, "int8_row", "xties"),
    # int4 beyond 16384 channels: the fused kernel scores, then the top-k launch
    # that starts from the channel blocks' score counts (random, duplicated and
    # mostly-zero scores: ties across blocks and a threshold at zero)
    (1024, 16416, "bf16", 1, "int4_g128", None), (1024, 16416, "bf16", 1, "int4_g128", "dup"),
    (1024, 16416, "bf16", 1, "int4_g128", "zeros"),
])
def test_stage1_scores_and_mask(d, F, dtype, B, mode, pattern):
    L = Layer(d, F, 0.02, dtype, seed=11, pattern=pattern if pattern != "xties" else None)
    xh = _tied_x(B, d, dtype, 11) if pattern == "xties" else synth.make_x(B, d, dtype, seed=11)
    sel, sc = P.stage1_select(to_dev(xh), L.w, L.proxy(mode), 0.5, 0.7, with_scores=True)
    torch.cuda.synchronize()
    ref = oracle.prox_forward(xh, L.wg, L.wu, L.wd, L.oracle_proxy(mode), 0.5, 0.7, mode)
    s = sc.cpu().numpy().astype(np.float64)
    scale = ref["score"].max()
    err = np.abs(s - ref["score"]).max() / scale
    log("stage1 %s score max err / max score = %.3g" % ((d, F, dtype, B, mode), err))
    assert err < 2e-5
    ok, msg = oracle.mask_admissible(sel.cpu().numpy(), ref["sel"], ref["score"], ref["T"], ref["k"])
    assert ok, msg
    # the GPU mask is the exact top-k of the GPU's own scores
    want, _ = oracle.topk_ascending(s, ref["k"])
    assert np.array_equal(sel.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("d,F,dtype,B", [(512, 1376, "f32", 1), (1000, 2048, "bf16", 1), (832, 1200, "bf16", 5),
                                         (4096, 14336, "bf16", 1)])
def test_stage2_on_given_mask(d, F, dtype, B):
    L = Layer(d, F, 0.02, dtype, seed=13)
    x = synth.make_x(B, d, dtype, seed=13)
    rng = np.random.default_rng(13)
    for k in (0, 1, 37, F // 3, F):
        sel = np.sort(rng.choice(F, size=k, replace=False)).astype(np.int32)
        out = P.stage2_exact(to_dev(x), L.w, torch.from_numpy(sel).to("cuda"))
        torch.cuda.synchronize()
        y = from_dev(out)
        y_ref, _ = oracle.ffn_masked(x, L.wg, L.wu, L.wd, sel.astype(np.int64))
        err = out_error(y, y_ref) if k else np.abs(y).max()
        assert err <= TOL[dtype], (k, err)


# ------------------------------------------------------- whole forward

SMALL = [
    # d, F, dtype, B, mode, keep, sparsity
    (512, 1376, "f32", 1, "int8_row", 0.5, 0.5),     # toy fp32 layer
    (256, 96, "f32", 2, "int8_row", 0.5, 0.5),
    (8, 16, "f32", 1, "int8_row", 0.5, 0.5),          # smallest supported shape
    (1000, 1040, "bf16", 1, "int8_row", 0.5, 0.7),    # ragged d and F tails
    (2048, 5504, "bf16", 1, "int8_row", 0.3, 0.9),
    (1536, 3008, "bf16", 3, "int8_row", 0.5, 0.7),
    (1024, 2048, "bf16", 5, "int8_row", 0.5, 0.6),
    (1024, 2048, "bf16", 16, "int8_row", 0.5, 0.7),
    (1024, 4096, "bf16", 1, "int4_g128", 0.4, 0.7),
    (1152, 1040, "bf16", 2, "int4_g128", 0.4, 0.5),
    (640, 1376, "f32", 1, "int4_g128", 0.4, 0.9),
    (1024, 2048, "bf16", 1, "int8_row", 1.0, 0.7),    # keep every input
    (1024, 2048, "bf16", 1, "int8_row", 0.5, 0.0),    # k = F: Stage 1 skipped
    (1024, 2048, "bf16", 2, "int8_row", 0.5, 1.0),    # k = 0: zeros
    (1024, 2048, "bf16", 1, "int8_row", 0.5, 0.9995),  # k = 1
]


@pytest.mark.parametrize("d,F,dtype,B,mode,keep,sp", SMALL)
def test_forward_small(d, F, dtype, B, mode, keep, sp):
    L = Layer(d, F, 0.02, dtype, seed=21)
    x = synth.make_x(B, d, dtype, seed=21)
    run_and_check(L, x, mode, keep, sp, label=str((d, F, dtype, B, mode, keep, sp)))


def test_forward_deterministic():
    L = Layer(2048, 5632, 0.02, "bf16", seed=23)
    x = to_dev(synth.make_x(4, 2048, "bf16", seed=23))
    p = L.proxy("int8_row")
    outs, sels = [], []
    for _ in range(3):
        sel = torch.empty(P.counts(2048, 5632, 0.5, 0.7)[1], dtype=torch.int32, device="cuda")
        outs.append(P.ffn_forward(x, L.w, p, 0.5, 0.7, sel_out=sel).clone())
        sels.append(sel)
    torch.cuda.synchronize()
    for o, s in zip(outs[1:], sels[1:]):
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
        assert torch.equal(s, sels[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_residual(dtype):
    d, F, B = 1024, 2816, 2
    L = Layer(d, F, 0.02, dtype, seed=29)
    x = synth.make_x(B, d, dtype, seed=29)
    r = synth.make_x(B, d, dtype, seed=30)
    run_and_check(L, x, "int8_row", 0.5, 0.7, residual=r, label="residual " + dtype)
    # in place: out aliases the residual
    rt = to_dev(r)
    out = P.ffn_forward(to_dev(x), L.w, L.proxy("int8_row"), 0.5, 0.7, residual=rt, out=rt)
    ref = P.ffn_forward(to_dev(x), L.w, L.proxy("int8_row"), 0.5, 0.7, residual=to_dev(r))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if dtype == "bf16" else out, ref.view(torch.int16) if dtype == "bf16" else ref)


@pytest.mark.parametrize("B,d,dtype", [(3, 4096, "bf16"), (2, 1000, "bf16"), (1, 16384, "bf16"),
                                       (2, 520, "f32"), (1, 16384, "f32")])
def test_rmsnorm(B, d, dtype):
    # every 16-byte vector of a row loaded at once: rows that end mid-way
    # through a thread's vectors (d = 1000, 520) and the largest d, where
    # every thread holds its full share
    h = synth.make_x(B, d, dtype, seed=31)
    out = P.rmsnorm(to_dev(h), 1e-5)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(h, 1e-5)
    got = from_dev(out)
    tol = 4e-3 if dtype == "bf16" else 1e-5  # bf16: output rounding; f32: the fp32 bar
    assert np.abs(got - ref).max() / np.abs(ref).max() < tol


def test_workspace_reuse_across_shapes():
    # one workspace serves calls of different sparsity and batch back to back
    L = Layer(1024, 2048, 0.02, "bf16", seed=37)
    ws = P.alloc_workspace(1024, 2048, 4)
    for B, sp in ((4, 0.7), (1, 0.5), (3, 0.0), (2, 0.9), (4, 0.7)):
        x = synth.make_x(B, 1024, "bf16", seed=B)
        xt = to_dev(x)
        out = P.ffn_forward(xt, L.w, L.proxy("int8_row"), 0.5, sp, workspace=ws)
        fresh = P.ffn_forward(xt, L.w, L.proxy("int8_row"), 0.5, sp)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), fresh.view(torch.int16)), (B, sp)


COUNTER_BYTES = 278528  # the workspace's leading counter block (include/prox.h)


def test_counters_left_zero():
    # every call hands the workspace back with its counters at zero: the
    # single-token kernels' tickets, per-split readiness lines and timeout flag
    L = Layer(1024, 4096, 0.02, "bf16", seed=41)
    n1, n3 = P.workspace_size(1024, 4096, 1), P.workspace_size(1024, 4096, 3)
    ws = P.alloc_workspace(1024, 4096, 3, extra=max(0, n1 - n3))  # serves B = 1 and B = 3

    def nonzero():
        torch.cuda.synchronize()
        return int(torch.count_nonzero(ws[:COUNTER_BYTES]).item())

    assert nonzero() == 0
    for B, sp in ((1, 0.7), (1, 0.33), (1, 0.93), (3, 0.7), (1, 0.0), (1, 0.7)):
        x = to_dev(synth.make_x(B, 1024, "bf16", seed=50 + B))
        P.ffn_forward(x, L.w, L.proxy("int8_row"), 0.5, sp, workspace=ws)
        assert nonzero() == 0, (B, sp)
    x = to_dev(synth.make_x(1, 1024, "bf16", seed=60))
    sel = torch.arange(0, 4096, 3, dtype=torch.int32, device="cuda")  # k = 1366: a ragged last split
    P.stage2_exact(x, L.w, sel, workspace=ws)
    assert nonzero() == 0
