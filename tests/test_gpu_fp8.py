"""GPU parity of the FP8 (OCP E4M3) exact-weight path against the CPU oracle.

Packing (codes and per-row scales) and the proxy built from FP8 weights are
bit-exact; Stage 2 on a given mask and the whole forward meet the output
tolerance against the oracle's Stage 2 on the dequantized weights (binary64),
and the mask lies within the near-tie window of the oracle's own.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import free_sparse_swiglu_stage1_amd as P
from tests.gpu_util import TOL, from_dev, log, out_error, to_dev, unpack_proxy

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    P.load_library()
    torch.cuda.init()


class Fp8Layer:
    """Seeded weights packed to FP8 on the device, and the oracle's FP8 copy."""

    def __init__(self, d, F, std, dtype, seed=0, crafted=False):
        self.d, self.F, self.dtype = d, F, dtype
        wg, wu, wd = synth.make_weights(d, F, std, dtype, seed=seed)
        if crafted:
            # a zero gate row; an up row and a down row whose scale is 2^-8
            # and whose entries sit exactly on E4M3 midpoints (ties)
            table = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
            mids = ((table[1:] + table[:-1]) / 2)[::3][: d - 1]
            row = np.resize(np.concatenate([[448.0], mids]), d) * 2.0 ** -8
            wd_row = np.resize(np.concatenate([[-448.0], -mids]) * 2.0 ** -8, F)
            if dtype == "bf16":
                enc = lambda a: (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
                keep = lambda a: oracle.as_f32(enc(a)).astype(np.float64) == np.asarray(a, dtype=np.float32)
                row = np.where(keep(row), row, 0.0)
                wd_row = np.where(keep(wd_row), wd_row, 0.0)
                wg[3] = 0
                wu[5] = enc(row)
                wd[7] = enc(wd_row)
            else:
                wg[3] = 0
                wu[5] = row.astype(np.float32)
                wd[7] = wd_row.astype(np.float32)
        self.wg, self.wu, self.wd = wg, wu, wd
        self.w = P.pack_weights_fp8(to_dev(wg), to_dev(wu), to_dev(wd))
        qg, sg = oracle.quantize_fp8(wg)
        qu, su = oracle.quantize_fp8(wu)
        qd, sd = oracle.quantize_fp8(wd)
        self.fp8 = (qg, sg, qu, su, qd, sd)
        self._proxy = {}

    def proxy(self, mode):
        if mode not in self._proxy:
            self._proxy[mode] = P.quantize_proxy(self.w, mode)
        return self._proxy[mode]

    def oracle_proxy(self, mode):
        qg, sg, qu, su, _, _ = self.fp8
        return oracle.quantize(oracle.dequant_fp8_f32(qg, sg), mode) + \
            oracle.quantize(oracle.dequant_fp8_f32(qu, su), mode)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_fp8_bit_exact(dtype):
    L = Fp8Layer(320, 208, 0.02, dtype, seed=21, crafted=True)
    qg, sg, qu, su, qd, sd = L.fp8
    gu = L.w.w_gu.cpu().numpy()
    gsc = L.w.gu_scales.cpu().numpy()
    np.testing.assert_array_equal(gu[:, 0, :], qg)
    np.testing.assert_array_equal(gu[:, 1, :], qu)
    np.testing.assert_array_equal(gsc[:, 0], sg)
    np.testing.assert_array_equal(gsc[:, 1], su)
    np.testing.assert_array_equal(L.w.w_down_t.cpu().numpy().T, qd)
    np.testing.assert_array_equal(L.w.down_scales.cpu().numpy(), sd)
    assert sg[3] == 0 and not qg[3].any()


@pytest.mark.parametrize("mode", ["int8_row", "int4_g128"])
def test_proxy_from_fp8_bit_exact(mode):
    L = Fp8Layer(256, 160, 0.02, "bf16", seed=22)
    qg, scg, qu, scu = unpack_proxy(L.proxy(mode))
    rg, rsg, ru, rsu = L.oracle_proxy(mode)
    np.testing.assert_array_equal(qg, rg)
    np.testing.assert_array_equal(qu, ru)
    np.testing.assert_array_equal(scg, rsg)
    np.testing.assert_array_equal(scu, rsu)


@pytest.mark.parametrize("d,F,dtype,B", [(512, 1376, "f32", 1), (1024, 2048, "bf16", 1), (832, 1200, "bf16", 5),
                                         (4096, 14336, "bf16", 1)])
def test_fp8_stage2_on_given_mask(d, F, dtype, B):
    L = Fp8Layer(d, F, 0.02, dtype, seed=23)
    rng = np.random.default_rng(23)
    x = synth.make_x(B, d, dtype, seed=23)
    for k in (1, 63, 65, (3 * F) // 10 + 1):
        sel = np.sort(rng.choice(F, size=k, replace=False)).astype(np.int32)
        log("fp8 stage2 d=%d F=%d %s B=%d k=%d" % (d, F, dtype, B, k))
        out = P.stage2_exact(to_dev(x), L.w, torch.from_numpy(sel).cuda())
        torch.cuda.synchronize()
        y_ref, _ = oracle.ffn_masked_fp8(x, L.fp8, sel.astype(np.int64))
        err = out_error(from_dev(out), y_ref)
        assert err <= TOL[dtype], (k, err)


def _forward_check(L, x, mode, keep, sp, residual=None, label=""):
    B = x.shape[0]
    k_in, k = P.counts(L.d, L.F, keep, sp)
    sel_t = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    res_t = to_dev(residual) if residual is not None else None
    out = P.ffn_forward(to_dev(x), L.w, L.proxy(mode), keep, sp, sel_out=sel_t, residual=res_t)
    torch.cuda.synchronize()
    y_gpu = from_dev(out)
    sel_gpu = sel_t[:k].cpu().numpy().astype(np.int64)
    ref = oracle.prox_forward(x, None, None, None, L.oracle_proxy(mode), keep, sp, mode, fp8=L.fp8)
    assert ref["k"] == k and ref["k_in"] == k_in
    ok, msg = oracle.mask_admissible(sel_gpu, ref["sel"], ref["score"], ref["T"], k)
    assert ok, "%s mask: %s" % (label, msg)
    y_ref, _ = oracle.ffn_masked_fp8(x, L.fp8, sel_gpu)
    if residual is not None:
        y_ref = y_ref + oracle.as_f64(residual)
    err = out_error(y_gpu, y_ref) if k > 0 or residual is not None else float(np.abs(y_gpu).max())
    log("%s k_in=%d k=%d mask %s err=%.3g" % (label, k_in, k, msg, err))
    assert err <= TOL[L.dtype], "%s output error %.3g" % (label, err)


@pytest.mark.parametrize("d,F,dtype,B,sp", [(1024, 2048, "bf16", 1, 0.7), (1024, 2048, "bf16", 3, 0.5),
                                            (512, 1376, "f32", 1, 0.5), (2048, 5632, "bf16", 4, 0.9),
                                            (1024, 2048, "bf16", 1, 0.0), (1024, 2048, "bf16", 2, 0.0),
                                            (8192, 1024, "bf16", 1, 0.7), (8192, 1024, "bf16", 2, 0.7)])
def test_fp8_forward(d, F, dtype, B, sp):
    L = Fp8Layer(d, F, 0.02, dtype, seed=24)
    x = synth.make_x(B, d, dtype, seed=24 + B)
    _forward_check(L, x, "int8_row", 0.5, sp, label="fp8 %dx%d %s B=%d sp=%g" % (d, F, dtype, B, sp))


def test_fp8_forward_residual_and_int4_proxy():
    L = Fp8Layer(1024, 2048, 0.02, "bf16", seed=25)
    x = synth.make_x(1, 1024, "bf16", seed=25)
    r = synth.make_x(1, 1024, "bf16", seed=26)
    _forward_check(L, x, "int8_row", 0.5, 0.7, residual=r, label="fp8 residual")
    _forward_check(L, x, "int4_g128", 0.5, 0.7, label="fp8 int4 proxy")


def test_fp8_forward_8b_shape():
    # the benchmark layer, 4096 x 14336 bf16, one token, sparsity 0.7
    L = Fp8Layer(4096, 14336, 0.02, "bf16", seed=0)
    x = synth.make_x(1, 4096, "bf16", seed=0)
    _forward_check(L, x, "int8_row", 0.5, 0.7, label="fp8 8B shape")
