"""Pins for the CPU oracle: checks against what the Prox pages and plain
mathematics fix, never against the oracle's own formulas retyped.

Each test names the mistake it is there to catch.  The pages print no
worked numerical example, so the pins are closed forms, brute force on
tiny inputs, library special cases (NumPy / SciPy routines), and the
method's invariants (one mask shared by all three projections; Stage 2
exact on the selected channels; 0% sparsity is the dense FFN).
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import expit

import synth


# ------------------------------------------------------------------ silu

def test_silu_closed_forms(oracle):
    # silu(z) = z * sigmoid(z): sigmoid(0) = 1/2, sigmoid(1) = e / (1 + e).
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(math.e / (1.0 + math.e), rel=1e-15)
    # odd part: silu(z) - silu(-z) = z  (catches exp(+z) for exp(-z), or a dropped z)
    for z in (0.25, 1.0, 3.5, -2.0, 17.0):
        assert oracle.silu(z) - oracle.silu(-z) == pytest.approx(z, rel=1e-14, abs=1e-14)
    # asymptotes: silu(z) -> z for z -> +inf, -> 0 for z -> -inf
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15
    # library special case: z * expit(z)
    for z in np.linspace(-12, 12, 97):
        assert oracle.silu(z) == pytest.approx(z * expit(z), rel=1e-14, abs=1e-300)


# ---------------------------------------------------------------- counts

@pytest.mark.parametrize("keep,n,expect", [
    (0.5, 512, 256), (0.5, 4096, 2048), (0.4, 8192, 3277), (1.0, 4096, 4096),
    (0.0, 4096, 1), (1e-9, 64, 1),
])
def test_input_count(oracle, keep, n, expect):
    # k_in = round-half-up(keep * d) on the binary32 keep value, clamped to [1, d]
    assert oracle.input_count(keep, n) == expect


@pytest.mark.parametrize("sp,F,expect", [
    (0.5, 1376, 688), (0.0, 11008, 11008), (0.5, 11008, 5504), (0.7, 11008, 3302),
    (0.9, 11008, 1101), (0.7, 14336, 4301), (0.5, 28672, 14336), (0.7, 28672, 8602),
    (0.9, 28672, 2867), (1.0, 14336, 0),
])
def test_channel_count(oracle, sp, F, expect):
    # (1 - 0.7f) * 14336 = 4300.8002 -> 4301 ; (1 - 0.9f) * 11008 = 1100.8003 -> 1101
    assert oracle.channel_count(sp, F) == expect


# ------------------------------------------------------------- quantizer

def test_quantize_int8_round_half_even(oracle):
    # absmax 127 -> scale exactly 1, so the codes are the rounded values:
    # ties go to even (2.5 -> 2, -3.5 -> -4, 0.5 -> 0, 126.5 -> 126).
    # Catches truncation, round-half-away and a scale of absmax/128 or /255.
    w = np.array([[127.0, 2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -127.0]], dtype=np.float32)
    q, sc = oracle.quantize(w, "int8_row")
    assert sc.tolist() == [1.0]
    assert q.tolist() == [[127, 2, -4, 0, 0, 2, 126, -127]]


def test_quantize_int8_integer_grid_roundtrip(oracle):
    # rows n * 2^-7 with integer n, max |n| = 127: scale 2^-7 and codes n, exactly
    rng = np.random.default_rng(3)
    n = rng.integers(-127, 128, size=(6, 40))
    n[:, 7] = 127 * np.array([1, -1, 1, -1, 1, -1])
    for r in range(6):  # force row-wise distinct magnitudes (catches per-column scales)
        n[r] = np.clip(n[r], -127, 127)
    scale = np.float32(2.0 ** -7) * (2.0 ** np.arange(6)).astype(np.float32)
    w = (n.astype(np.float32) * scale[:, None]).astype(np.float32)
    q, sc = oracle.quantize(w, "int8_row")
    np.testing.assert_array_equal(sc, scale)
    np.testing.assert_array_equal(q, n)


def test_quantize_int8_error_bound_and_extremes(oracle):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((33, 300)) * 0.02).astype(np.float32)
    q, sc = oracle.quantize(w, "int8_row")
    w64 = w.astype(np.float64)
    absmax = np.abs(w64).max(axis=1)
    np.testing.assert_allclose(sc, (absmax / 127).astype(np.float32), rtol=2 ** -23)
    err = np.abs(w64 - sc[:, None].astype(np.float64) * q)
    assert np.all(err <= sc[:, None] * (0.5 + 1e-5))
    # the absmax element maps to +-127
    am = np.abs(w64).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(33), am]) == 127)
    assert np.abs(q).max() == 127


def test_quantize_zero_rows(oracle):
    w = np.zeros((2, 256), dtype=np.float32)
    w[1, 5] = 1.0
    q, sc = oracle.quantize(w, "int8_row")
    assert sc[0] == 0.0 and not q[0].any()
    q4, sc4 = oracle.quantize(w, "int4_g128")
    assert sc4[0].tolist() == [0.0, 0.0] and not q4[0].any()
    assert sc4[1, 1] == 0.0 and sc4[1, 0] == np.float32(1.0 / 7)


def test_quantize_int4_groups(oracle):
    # Two groups of 128 with different magnitudes: each gets its own scale
    # (catches a per-row int4 scale and an i % 128 group index).
    n = np.tile(np.arange(-7, 8), 18)[:256].astype(np.float32)
    w = np.empty((3, 256), dtype=np.float32)
    w[0] = n * np.float32(2.0 ** -5)
    w[1, :128] = n[:128] * np.float32(2.0 ** -3)
    w[1, 128:] = n[128:] * np.float32(2.0 ** -9)
    w[2] = n * np.float32(2.0 ** -5)
    w[2, 200] = np.float32(3.5 * 2.0 ** -5)  # a tie inside group 1 (3.5 -> 4)
    q, sc = oracle.quantize(w, "int4_g128")
    np.testing.assert_array_equal(sc[0], [2.0 ** -5, 2.0 ** -5])
    np.testing.assert_array_equal(sc[1], [2.0 ** -3, 2.0 ** -9])
    np.testing.assert_array_equal(q[0], n)
    np.testing.assert_array_equal(q[1], n)
    assert q[2, 200] == 4
    assert q.min() >= -7 and q.max() <= 7


def test_quantize_int4_error_bound(oracle):
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((17, 512)) * 0.015).astype(np.float32)
    q, sc = oracle.quantize(w, "int4_g128")
    assert sc.shape == (17, 4)
    deq = np.repeat(sc.astype(np.float64), 128, axis=1) * q
    bound = np.repeat(sc.astype(np.float64), 128, axis=1) * (0.5 + 1e-5)
    assert np.all(np.abs(w - deq) <= bound)
    g = np.abs(w.reshape(17, 4, 128)).argmax(axis=2)
    qq = q.reshape(17, 4, 128)
    assert np.all(np.abs(np.take_along_axis(qq, g[:, :, None], axis=2)) == 7)


# ------------------------------------------------------------ top-k rank

def _brute_force_topk(v, k):
    """The unique k-subset S such that every member of S precedes every
    non-member under (|v| desc, index asc) -- found by enumerating subsets."""
    n = len(v)
    mags = [abs(float(t)) for t in v]

    def before(a, b):
        return mags[a] > mags[b] or (mags[a] == mags[b] and a < b)

    found = []
    for S in itertools.combinations(range(n), k):
        rest = [b for b in range(n) if b not in S]
        if all(before(a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1
    return list(found[0])


def test_topk_brute_force_ties(oracle):
    # values from a tiny alphabet force ties, +0/-0, and negative entries
    rng = np.random.default_rng(11)
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, 0.5])
    for trial in range(300):
        n = int(rng.integers(1, 9))
        v = rng.choice(alphabet, size=n)
        for k in range(0, n + 1):
            got, kth = oracle.topk_ascending(v, k)
            want = _brute_force_topk(v, k)
            assert got.tolist() == want, (v, k)
            if k:
                assert kth == min(abs(v[j]) for j in want)


def test_topk_invariants_large(oracle):
    rng = np.random.default_rng(12)
    v = np.round(rng.standard_normal(5000), 2)  # many exact ties
    k = 1234
    sel, T = oracle.topk_ascending(v, k)
    assert sel.size == k and np.all(np.diff(sel) > 0)
    m = np.abs(v)
    mask = np.zeros(v.size, bool)
    mask[sel] = True
    assert m[mask].min() >= m[~mask].max()
    # at the threshold, the lower indices were taken
    tied = np.nonzero(m == T)[0]
    taken = tied[mask[tied]]
    assert np.array_equal(taken, tied[:taken.size])


def test_input_select_brute_force(oracle):
    rng = np.random.default_rng(13)
    alphabet = np.array([0.0, 1.0, -1.0, 2.5, -2.5, 4.0], dtype=np.float32)
    for trial in range(100):
        B = int(rng.integers(1, 4))
        d = int(rng.integers(1, 9))
        x = rng.choice(alphabet, size=(B, d)).astype(np.float32)
        k_in = int(rng.integers(1, d + 1))
        xh = oracle.input_select(x, k_in)
        for b in range(B):
            keep = _brute_force_topk(x[b], k_in)
            want = np.zeros(d)
            want[keep] = x[b, keep]
            np.testing.assert_array_equal(xh[b], want)


# ----------------------------------------------------------------- proxy

def _numpy_proxy(xhat, qg, scg, qu, scu, mode):
    d = qg.shape[1]
    if mode == "int8_row":
        Wg = scg.astype(np.float64)[:, None] * qg
        Wu = scu.astype(np.float64)[:, None] * qu
    else:
        Wg = np.repeat(scg.astype(np.float64), 128, axis=1) * qg
        Wu = np.repeat(scu.astype(np.float64), 128, axis=1) * qu
    g = xhat @ Wg.T
    u = xhat @ Wu.T
    return g, u, np.abs(g * expit(g) * u).sum(axis=0)


@pytest.mark.parametrize("mode,B", [("int8_row", 1), ("int8_row", 3), ("int4_g128", 1), ("int4_g128", 2)])
def test_proxy_matches_numpy(oracle, mode, B):
    # NumPy matmul on the dequantized proxy; non-square shapes catch a
    # transposed operand, a wrong group index or a swapped gate/up.
    d, F = 256, 72
    wg, wu, _ = synth.make_weights(d, F, 0.02, "f32", seed=1)
    x = synth.make_x(B, d, "f32", seed=1)
    qg, scg = oracle.quantize(wg, mode)
    qu, scu = oracle.quantize(wu, mode)
    xh = oracle.input_select(x, 100)
    g, u, sc = oracle.proxy(xh, qg, scg, qu, scu, mode)
    g2, u2, sc2 = _numpy_proxy(xh, qg, scg, qu, scu, mode)
    np.testing.assert_allclose(g, g2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(u, u2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sc, sc2, rtol=1e-12, atol=1e-300)


def test_proxy_lossless_full_keep_equals_exact_salience(oracle):
    # With every input kept and weights on the quantizer's integer grid, the
    # proxy IS the exact intermediate state, so the proxy mask equals the
    # mask of the exact |s| ranking (the method's ideal signal).
    rng = np.random.default_rng(21)
    d, F, B = 64, 96, 2
    wg = (rng.integers(-127, 128, size=(F, d)) * 2.0 ** -9).astype(np.float32)
    wu = (rng.integers(-127, 128, size=(F, d)) * 2.0 ** -9).astype(np.float32)
    wg[:, 0] = 127 * 2.0 ** -9
    wu[:, 0] = -127 * 2.0 ** -9
    wd = (rng.standard_normal((d, F)) * 0.02).astype(np.float32)
    x = rng.standard_normal((B, d)).astype(np.float32)
    qg, scg = oracle.quantize(wg, "int8_row")
    qu, scu = oracle.quantize(wu, "int8_row")
    res = oracle.prox_forward(x, wg, wu, wd, (qg, scg, qu, scu), 1.0, 0.75, "int8_row")
    _, s_exact = oracle.ffn_dense(x, wg, wu, wd)
    exact_score = np.abs(s_exact).sum(axis=0)
    np.testing.assert_allclose(res["score"], exact_score, rtol=1e-13)
    want, _ = oracle.topk_ascending(exact_score, res["k"])
    assert res["sel"].tolist() == want.tolist()


def test_batch_identical_tokens_and_permutation(oracle):
    d, F = 128, 200
    wg, wu, wd = synth.make_weights(d, F, 0.02, "f32", seed=4)
    qg, scg = oracle.quantize(wg, "int8_row")
    qu, scu = oracle.quantize(wu, "int8_row")
    P = (qg, scg, qu, scu)
    x1 = synth.make_x(1, d, "f32", seed=4)
    r1 = oracle.prox_forward(x1, wg, wu, wd, P, 0.5, 0.6, "int8_row")
    r3 = oracle.prox_forward(np.repeat(x1, 3, axis=0), wg, wu, wd, P, 0.5, 0.6, "int8_row")
    assert r1["sel"].tolist() == r3["sel"].tolist()
    np.testing.assert_allclose(r3["score"], 3 * r1["score"], rtol=1e-14)
    x4 = synth.make_x(4, d, "f32", seed=5)
    ra = oracle.prox_forward(x4, wg, wu, wd, P, 0.5, 0.6, "int8_row")
    rb = oracle.prox_forward(x4[[2, 0, 3, 1]], wg, wu, wd, P, 0.5, 0.6, "int8_row")
    assert ra["sel"].tolist() == rb["sel"].tolist()
    np.testing.assert_array_equal(ra["y"][[2, 0, 3, 1]], rb["y"])


# ---------------------------------------------------------------- Stage 2

def _numpy_dense(x, wg, wu, wd):
    g = x @ wg.T.astype(np.float64)
    u = x @ wu.T.astype(np.float64)
    s = g * expit(g) * u
    return s @ wd.T.astype(np.float64), s


def test_tiny_swiglu_by_hand(oracle):
    # x = (1, 2); gate rows pick g = (1, 2); up rows give u = (3, -2);
    # s = (3 sigmoid(1), -4 sigmoid(2)); W_down = [[1, 1], [2, -1]].
    x = np.array([[1.0, 2.0]], dtype=np.float32)
    wg = np.array([[1, 0], [0, 1]], dtype=np.float32)
    wu = np.array([[3, 0], [0, -1]], dtype=np.float32)
    wd = np.array([[1, 1], [2, -1]], dtype=np.float32)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    s1, s2 = 3 * sig(1.0), -4 * sig(2.0)
    y, s = oracle.ffn_dense(x, wg, wu, wd)
    np.testing.assert_allclose(s[0], [s1, s2], rtol=1e-15)
    np.testing.assert_allclose(y[0], [s1 + s2, 2 * s1 - s2], rtol=1e-15)
    # mask {1} only: y = W_down[:, 1] * s2
    y1, _ = oracle.ffn_masked(x, wg, wu, wd, np.array([1]))
    np.testing.assert_allclose(y1[0], [s2, -s2], rtol=1e-15)


@pytest.mark.parametrize("B", [1, 3])
def test_dense_matches_numpy(oracle, B):
    d, F = 192, 160
    wg, wu, wd = synth.make_weights(d, F, 0.02, "bf16", seed=7)
    x = synth.make_x(B, d, "bf16", seed=7)
    y, s = oracle.ffn_dense(x, wg, wu, wd)
    f = oracle.as_f64
    y2, s2 = _numpy_dense(f(x), f(wg), f(wu), f(wd))
    np.testing.assert_allclose(s, s2, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(y, y2, rtol=1e-11, atol=1e-14)


def test_masked_is_dense_with_dropped_channels_zeroed(oracle):
    d, F = 160, 224
    wg, wu, wd = synth.make_weights(d, F, 0.02, "f32", seed=8)
    x = synth.make_x(2, d, "f32", seed=8)
    rng = np.random.default_rng(8)
    sel = np.sort(rng.choice(F, size=67, replace=False))
    y, s = oracle.ffn_masked(x, wg, wu, wd, sel)
    _, s_all = _numpy_dense(x.astype(np.float64), wg, wu, wd)
    s_z = np.zeros_like(s_all)
    s_z[:, sel] = s_all[:, sel]
    np.testing.assert_allclose(s, s_all[:, sel], rtol=1e-12)
    np.testing.assert_allclose(y, s_z @ wd.T.astype(np.float64), rtol=1e-11, atol=1e-15)
    # complement additivity: y(S) + y(S^c) = y(all)
    comp = np.setdiff1d(np.arange(F), sel)
    yc, _ = oracle.ffn_masked(x, wg, wu, wd, comp)
    ya, _ = oracle.ffn_dense(x, wg, wu, wd)
    np.testing.assert_allclose(y + yc, ya, rtol=1e-12, atol=1e-15)


def test_zero_sparsity_is_dense_and_stage2_uses_dense_x(oracle):
    d, F = 128, 176
    wg, wu, wd = synth.make_weights(d, F, 0.02, "bf16", seed=2)
    x = synth.make_x(1, d, "bf16", seed=2)
    qg, scg = oracle.quantize(oracle.as_f32(wg), "int8_row")
    qu, scu = oracle.quantize(oracle.as_f32(wu), "int8_row")
    P = (qg, scg, qu, scu)
    r0 = oracle.prox_forward(x, wg, wu, wd, P, 0.5, 0.0, "int8_row")
    yd, _ = oracle.ffn_dense(x, wg, wu, wd)
    assert r0["k"] == F
    np.testing.assert_array_equal(r0["y"], yd)
    # at 70%: the output is the numpy SwiGLU on the DENSE x restricted to the
    # mask (catches Stage 2 reusing the sparsified x or a different mask)
    r = oracle.prox_forward(x, wg, wu, wd, P, 0.5, 0.7, "int8_row")
    f = oracle.as_f64
    _, s_all = _numpy_dense(f(x), f(wg), f(wu), f(wd))
    s_z = np.zeros_like(s_all)
    s_z[:, r["sel"]] = s_all[:, r["sel"]]
    np.testing.assert_allclose(r["y"], s_z @ f(wd).T, rtol=1e-11, atol=1e-15)
    # full sparsity: nothing selected, output zero
    r1 = oracle.prox_forward(x, wg, wu, wd, P, 0.5, 1.0, "int8_row")
    assert r1["k"] == 0 and not r1["y"].any()


# ------------------------------------------------- activation and signals

def _torch_gelu_tanh(z):
    import torch
    return torch.nn.functional.gelu(torch.as_tensor(np.asarray(z, dtype=np.float64)), approximate="tanh").numpy()


def test_gelu_tanh_closed_forms_and_library(oracle):
    # catches a wrong constant or a dropped cubic term
    assert oracle.gelu_tanh(0.0) == 0.0
    for z in (0.3, 1.0, 2.5, 7.0):
        assert abs(oracle.gelu_tanh(z) - oracle.gelu_tanh(-z) - z) < 1e-15 * max(1.0, z)
    assert oracle.gelu_tanh(40.0) == 40.0 and oracle.gelu_tanh(-40.0) == 0.0
    zs = np.linspace(-8, 8, 161)
    np.testing.assert_allclose([oracle.gelu_tanh(z) for z in zs], _torch_gelu_tanh(zs), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_signals_match_numpy(oracle, act):
    # the three proxy signals from the same g~, u~: |h~ u~|, |h~|, |u~|,
    # h~ = act(g~), summed over the batch (catches a branch swapped or unsummed)
    d, F, B = 128, 96, 2
    wg, wu, _ = synth.make_weights(d, F, 0.05, "f32", seed=17)
    x = synth.make_x(B, d, "f32", seed=17)
    xh = oracle.input_select(x, 64)
    qg, scg = oracle.quantize(wg, "int8_row")
    qu, scu = oracle.quantize(wu, "int8_row")
    g, u, _ = oracle.proxy(xh, qg, scg, qu, scu, "int8_row")
    h = g * expit(g) if act == "silu" else _torch_gelu_tanh(g)
    for sig, want in (("s", np.abs(h * u).sum(0)), ("h", np.abs(h).sum(0)), ("u", np.abs(u).sum(0))):
        _, _, sc = oracle.proxy(xh, qg, scg, qu, scu, "int8_row", act, sig)
        np.testing.assert_allclose(sc, want, rtol=1e-12, atol=1e-18)


def test_exact_signal_is_the_exact_state(oracle):
    # exact_s scores are |s| of the dense FFN; with keep 1 and weights on a
    # lossless int8 grid the Prox proxy mask equals the exact-state mask
    d, F = 64, 80
    rng = np.random.default_rng(18)
    wg = (rng.integers(-127, 128, (F, d)) * 2.0 ** -9).astype(np.float32)
    wu = (rng.integers(-127, 128, (F, d)) * 2.0 ** -9).astype(np.float32)
    wg[:, 0], wu[:, 0] = 127 * 2.0 ** -9, -127 * 2.0 ** -9
    wd = synth.make_weights(d, F, 0.02, "f32", seed=18)[2]
    x = synth.make_x(2, d, "f32", seed=18)
    for act in ("silu", "gelu_tanh"):
        sc = oracle.exact_scores(x, wg, wu, wd, act)
        g, u = x.astype(np.float64) @ wg.T.astype(np.float64), x.astype(np.float64) @ wu.T.astype(np.float64)
        h = g * expit(g) if act == "silu" else _torch_gelu_tanh(g)
        np.testing.assert_allclose(sc, np.abs(h * u).sum(0), rtol=1e-12)
        P = oracle.quantize(wg, "int8_row") + oracle.quantize(wu, "int8_row")
        r_proxy = oracle.prox_forward(x, wg, wu, wd, P, 1.0, 0.6, "int8_row", act=act, signal="s")
        r_exact = oracle.prox_forward(x, wg, wu, wd, P, 1.0, 0.6, "int8_row", act=act, signal="exact_s")
        np.testing.assert_array_equal(r_proxy["sel"], r_exact["sel"])
        np.testing.assert_allclose(r_proxy["score"], r_exact["score"], rtol=1e-12)


def test_geglu_dense_matches_numpy(oracle):
    d, F = 160, 128
    wg, wu, wd = synth.make_weights(d, F, 0.05, "f32", seed=19)
    x = synth.make_x(2, d, "f32", seed=19)
    y, s = oracle.ffn_dense(x, wg, wu, wd, "gelu_tanh")
    f = oracle.as_f64
    g, u = f(x) @ f(wg).T, f(x) @ f(wu).T
    s2 = _torch_gelu_tanh(g) * u
    np.testing.assert_allclose(s, s2, rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(y, s2 @ f(wd).T, rtol=1e-11, atol=1e-15)


# ------------------------------------------------------------- FP8 E4M3
# Facts of the OCP E4M3 format (not of the pages, which name FP8 only):
# bias 7, subnormals down to 2^-9, largest finite 448, S.1111.111 = NaN.

def _e4m3_values(oracle):
    return np.array([oracle.e4m3_decode(c) for c in range(256)])


def test_e4m3_decode_spec_values(oracle):
    # catches a wrong exponent bias, subnormal scale or NaN encoding
    spec = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3F: 1.875,
            0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in spec.items():
        assert oracle.e4m3_decode(c) == v, hex(c)
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))
    assert math.copysign(1.0, oracle.e4m3_decode(0x80)) == -1.0 and oracle.e4m3_decode(0x80) == 0.0


def test_e4m3_decode_structure(oracle):
    # magnitudes rise with the code; the sign bit negates; each binade holds
    # 8 evenly spaced values; the subnormals continue the first binade's step
    v = _e4m3_values(oracle)
    mag = v[:0x7F]
    assert np.all(np.diff(mag) > 0)
    np.testing.assert_array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    for e in range(1, 16):
        row = v[8 * e:8 * e + 8] if e < 15 else v[8 * e:8 * e + 7]
        steps = np.diff(np.concatenate([row, [2.0 ** (e - 6)]])) if e < 15 else np.diff(row)
        assert np.all(steps == steps[0]) and steps[0] == 2.0 ** (e - 10), e
    assert np.all(np.diff(v[0:9]) == 2.0 ** -9)
    assert np.isfinite(v).sum() == 254


def _nearest_code_brute(v, table):
    # the definition of the conversion by exhaustive search: nearest finite
    # value, ties to the code with an even mantissa, saturation at 448
    a = abs(float(v))
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    if a >= 448.0:
        return sign | 0x7E
    dist = np.abs(table[:0x7F] - a)
    best = np.flatnonzero(dist == dist.min())
    if len(best) > 1:
        best = [c for c in best if c % 2 == 0]
    return sign | int(best[0])


def test_e4m3_encode_nearest_ties_even(oracle):
    # catches ties away from zero, truncation, missing saturation
    table = _e4m3_values(oracle)
    rng = np.random.default_rng(11)
    vals = list(np.float32(rng.uniform(-1, 1, 400) * 2.0 ** rng.uniform(-12, 9.5, 400)))
    mags = table[:0x7F]
    vals += list(np.float32((mags[1:] + mags[:-1]) / 2))          # every midpoint (a tie)
    vals += list(np.float32(-(mags[1:] + mags[:-1]) / 2))
    vals += list(np.float32(mags)) + [np.float32(449.0), np.float32(464.0), np.float32(1e30), np.float32(-600.0)]
    for v in vals:
        assert oracle.e4m3_encode(v) == _nearest_code_brute(v, table), float(v)
    assert oracle.e4m3_encode(np.float32(-0.0)) == 0x80 and oracle.e4m3_encode(np.float32(0.0)) == 0x00
    for c in range(256):
        if c not in (0x7F, 0xFF):
            assert oracle.e4m3_encode(np.float32(table[c])) == c, hex(c)


def test_quantize_fp8_rows(oracle):
    # the absmax element reaches +-448; every code is finite; error at most
    # half a step of E4M3 at the scaled magnitude; an all-zero row stays zero
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((6, 300)) * np.array([[1e-3], [0.02], [1.0], [50.0], [0.0], [3e-6]])).astype(np.float32)
    w[5, 17] = -0.25
    q, sc = oracle.quantize_fp8(w)
    table = _e4m3_values(oracle)
    assert sc[4] == 0.0 and not q[4].any()
    for r in range(6):
        if r == 4:
            continue
        a = np.abs(w[r]).max()
        i = int(np.abs(w[r]).argmax())
        assert q[r, i] & 0x7F == 0x7E and (q[r, i] >> 7) == (w[r, i] < 0)
        assert np.float32(a / 448.0) == sc[r] or abs(float(sc[r]) * 448.0 / float(a) - 1.0) < 2 ** -23
        assert np.all((q[r] & 0x7F) != 0x7F)
        t = np.abs(w[r].astype(np.float64) / float(sc[r]))
        err = np.abs(table[q[r]] * float(sc[r]) - w[r].astype(np.float64)) / float(sc[r])
        step = np.where(t >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3), 2.0 ** -9)
        assert np.all(err <= step / 2 * (1 + 1e-6) + 1e-30)


def test_ffn_masked_fp8_equals_masked_on_exact_weights(oracle):
    # rows whose absmax is 1.75 * 2^e get the scale 2^(e-8) exactly, so
    # scale * decode is exact in binary32: the FP8 Stage 2 must then equal the
    # pinned masked FFN on those dequantized weights, bit for bit.  The
    # scales differ from row to row, so a scale taken from the wrong row or
    # projection shows.
    d, F = 96, 80
    rng = np.random.default_rng(13)

    def rows(n, m):
        e = rng.integers(-1, 3, n)
        w = (rng.uniform(-1.7, 1.7, (n, m)) * 2.0 ** e[:, None]).astype(np.float32)
        w[np.arange(n), rng.integers(0, m, n)] = (1.75 * 2.0 ** e * np.where(rng.random(n) < 0.5, -1, 1)).astype(np.float32)
        return w, (2.0 ** (e - 8)).astype(np.float32)

    (wg, eg), (wu, eu), (wd, ed) = rows(F, d), rows(F, d), rows(d, F)
    qg, sg = oracle.quantize_fp8(wg)
    qu, su = oracle.quantize_fp8(wu)
    qd, sd = oracle.quantize_fp8(wd)
    np.testing.assert_array_equal(sg, eg)
    np.testing.assert_array_equal(su, eu)
    np.testing.assert_array_equal(sd, ed)
    dq = lambda q, s: oracle.dequant_fp8_f32(q, s)
    x = synth.make_x(2, d, "f32", seed=13)
    sel = np.sort(rng.choice(F, size=29, replace=False))
    y8, s8 = oracle.ffn_masked_fp8(x, (qg, sg, qu, su, qd, sd), sel)
    y, s = oracle.ffn_masked(x, dq(qg, sg), dq(qu, su), dq(qd, sd), sel)
    np.testing.assert_array_equal(s8, s)
    np.testing.assert_array_equal(y8, y)
    # and the dequantized weights are the table values times the row's power of two
    np.testing.assert_array_equal(dq(qg, sg), (_e4m3_values(oracle)[qg] * eg[:, None].astype(np.float64)).astype(np.float32))


# --------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms(oracle):
    c = 3.0
    r = oracle.rmsnorm(np.full((1, 64), c, dtype=np.float32), 1e-5)
    np.testing.assert_allclose(r, c / math.sqrt(c * c + 1e-5), rtol=1e-15)
    r = oracle.rmsnorm(np.array([[3.0, 4.0]], dtype=np.float32), 1e-5)
    np.testing.assert_allclose(r[0], np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-5), rtol=1e-15)


def test_rmsnorm_batch_rows_independent(oracle):
    """Every token is normalized by its own mean square: rows of different
    closed forms in one batch (a constant row c -> c / sqrt(c^2 + eps), the
    [3, 4] row -> [3, 4] / sqrt(12.5 + eps), a zero row -> 0, a row whose
    entries cancel in a plain sum), each as it is on its own."""
    eps = 1e-5
    h = np.array([[7.0, 7.0], [3.0, 4.0], [0.0, 0.0], [-6.0, 6.0], [0.5, -0.25]], dtype=np.float32)
    r = oracle.rmsnorm(h, eps)
    np.testing.assert_allclose(r[0], 7.0 / math.sqrt(49.0 + eps), rtol=1e-15)
    np.testing.assert_allclose(r[1], np.array([3.0, 4.0]) / math.sqrt(12.5 + eps), rtol=1e-15)
    assert np.all(r[2] == 0.0)
    np.testing.assert_allclose(r[3], np.array([-6.0, 6.0]) / math.sqrt(36.0 + eps), rtol=1e-15)
    np.testing.assert_allclose(r[4], np.array([0.5, -0.25]) / math.sqrt(0.15625 + eps), rtol=1e-15)
    # and each row equals the row normalized alone, whatever its neighbours
    for b in range(h.shape[0]):
        np.testing.assert_array_equal(oracle.rmsnorm(h[b:b + 1], eps)[0], r[b])
        np.testing.assert_array_equal(oracle.rmsnorm(h[::-1], eps)[h.shape[0] - 1 - b], r[b])


# ------------------------------------------------------- acceptance rule

def test_mask_admissible_rule(oracle):
    score = np.array([5.0, 4.0, 3.00001, 3.0, 2.0, 1.0])
    ref, T = oracle.topk_ascending(score, 3)  # {0, 1, 2}, T = 3.00001
    assert oracle.mask_admissible(ref, ref, score, T, 3)[0]
    # 3 and 2 lie within 1e-4 of T: swapping them is admissible
    assert oracle.mask_admissible(np.array([0, 1, 3]), ref, score, T, 3)[0]
    # dropping a clear member is not
    assert not oracle.mask_admissible(np.array([0, 2, 3]), ref, score, T, 3)[0]
    assert not oracle.mask_admissible(np.array([0, 1, 4]), ref, score, T, 3)[0]
    assert not oracle.mask_admissible(np.array([0, 1]), ref, score, T, 3)[0]
    assert not oracle.mask_admissible(np.array([0, 1, 1]), ref, score, T, 3)[0]
