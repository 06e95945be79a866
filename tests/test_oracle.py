"""Pins for the fp64 CPU oracle (no GPU).

Each check ties the oracle to something other than itself: an independent
NumPy/SciPy brute force, a textbook routine, a closed form, an invariant, or
the worked magnitude example printed on the GEMM-logsumexp page. The set is
chosen so that a plausible slip in the oracle (a flipped kernel, a swapped
kh/kw, a dropped bias, a wrong sign or constant in an activation, a missing
max shift, a wrong pool divisor) fails at least one of them;
``test_oracle_mutants.py`` plants such slips in a copy of the oracle and
checks that these pins catch every one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.optimize
import scipy.signal
import scipy.special

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ independent helpers
def np_gelu(v):
    return v * scipy.special.ndtr(v)


def np_gelu_tanh(v):
    # 0.5 (1 + tanh(u)) = sigmoid(2u): the page's tanh form evaluated through the logistic function
    return v * scipy.special.expit(2.0 * math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3))


def np_mish(v):
    return v * np.tanh(np.logaddexp(0.0, v))


def np_act(v, act):
    if act == oracle.ACT_GELU:
        return np_gelu(v)
    if act == oracle.ACT_MISH2:
        return np_mish(np_mish(v))
    if act == oracle.ACT_GELU_TANH:
        return np_gelu_tanh(v)
    return v


def np_conv_valid(x, w, b):
    """Sliding-window cross-correlation in float64 (independent of the oracle's loops)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    win = np.lib.stride_tricks.sliding_window_view(x, (3, 3), axis=(2, 3))  # N,Cin,OH,OW,3,3
    return np.einsum("ncyxij,ocij->noyx", win, w) + np.asarray(b, np.float64)[None, :, None, None]


def rng_case(seed, N, Cin, H, W, Cout, wscale=0.3):
    r = np.random.default_rng(seed)
    x = r.uniform(-1, 1, (N, Cin, H, W)).astype(np.float32)
    w = r.uniform(-wscale, wscale, (Cout, Cin, 3, 3)).astype(np.float32)
    b = r.uniform(-0.5, 0.5, Cout).astype(np.float32)
    return x, w, b


# ------------------------------------------------------------------ activations
@pytest.mark.parametrize("v,expect", [(0.0, 0.0), (1.0, 0.8413447460685429),
                                      (-1.0, -0.15865525393145707), (2.0, 1.9544997361036416)])
def test_gelu_closed_form_values(v, expect):
    # GELU(v) = v * Phi(v); Phi(1) = 0.8413447460685429 (standard normal table)
    assert oracle.gelu(v) == pytest.approx(expect, abs=1e-15)
    assert oracle.act(v, oracle.ACT_GELU) == pytest.approx(expect, abs=1e-15)


def test_gelu_matches_normal_cdf_and_reflection():
    vs = np.linspace(-8, 8, 161)
    for v in vs:
        g = oracle.gelu(v)
        assert g == pytest.approx(np_gelu(v), rel=1e-13, abs=1e-15)
        # Phi(-v) = 1 - Phi(v)  =>  GELU(-v) = GELU(v) - v
        assert oracle.gelu(-v) == pytest.approx(g - v, abs=1e-13)


def test_gelu_tanh_logistic_form_and_reflection():
    for v in np.linspace(-10, 10, 201):
        g = oracle.gelu_tanh(v)
        assert oracle.act(v, oracle.ACT_GELU_TANH) == g
        assert g == pytest.approx(np_gelu_tanh(v), rel=1e-13, abs=1e-15)
        # tanh is odd  =>  GELU_tanh(v) - GELU_tanh(-v) = v
        assert g - oracle.gelu_tanh(-v) == pytest.approx(v, abs=1e-13)
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh(30.0) == 30.0
    assert abs(oracle.gelu_tanh(-30.0)) < 1e-300


def test_gelu_tanh_is_the_close_approximation_of_exact_gelu():
    # The tanh form approximates v * Phi(v) to within 4.8e-4 everywhere (the cubic
    # coefficient is fitted for that); its largest gap, 4.73e-4, sits near |v| = 2.70.
    # A dropped cubic term or a wrong constant moves the gap to 1e-3 .. 3e-2.
    vs = np.linspace(-12, 12, 24001)
    d = np.array([oracle.gelu_tanh(v) for v in vs]) - np_gelu(vs)
    assert np.max(np.abs(d)) < 4.8e-4
    assert np.max(np.abs(d)) > 4.6e-4
    assert abs(abs(vs[np.argmax(np.abs(d))]) - 2.70) < 0.05  # the gap is even in v


def test_softplus_matches_logaddexp():
    for v in np.concatenate([np.linspace(-50, 50, 201), [-700.0, 700.0]]):
        assert oracle.softplus(v) == pytest.approx(np.logaddexp(0.0, v), rel=1e-14, abs=1e-300)


@pytest.mark.parametrize("v,expect", [(0.0, 0.0), (1.0, 0.8650983882673103), (-1.0, -0.30340146137410895)])
def test_mish_values(v, expect):
    assert oracle.mish(v) == pytest.approx(expect, abs=1e-15)


def test_mish_algebraic_identity_and_limits():
    # mish(v) = v * tanh(log(1+e^v)) = v * (e^2v + 2e^v) / (e^2v + 2e^v + 2)
    for v in np.linspace(-20, 20, 401):
        e = math.exp(v)
        n = e * e + 2 * e
        assert oracle.mish(v) == pytest.approx(v * n / (n + 2), rel=1e-12, abs=1e-300)
    assert oracle.mish(60.0) == pytest.approx(60.0, rel=1e-15)
    assert abs(oracle.mish(-60.0)) < 1e-20


def test_mish_minimum():
    res = scipy.optimize.minimize_scalar(oracle.mish, bounds=(-3, 0), method="bounded",
                                         options={"xatol": 1e-10})
    assert res.x == pytest.approx(-1.19243, abs=1e-4)
    assert res.fun == pytest.approx(-0.308843, abs=1e-6)


def test_mish2_is_composition():
    assert oracle.act(1.0, oracle.ACT_MISH2) == pytest.approx(0.725479054960684, abs=1e-15)
    for v in np.linspace(-6, 6, 49):
        assert oracle.act(v, oracle.ACT_MISH2) == pytest.approx(np_mish(np_mish(v)), rel=1e-12, abs=1e-15)
    assert oracle.act(0.37, oracle.ACT_NONE) == 0.37


# ------------------------------------------------------------------ convolution
@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_GELU, oracle.ACT_MISH2, oracle.ACT_GELU_TANH])
@pytest.mark.parametrize("shape", [(2, 3, 16, 16, 8), (3, 5, 9, 11, 7), (1, 1, 3, 3, 1), (2, 4, 3, 7, 3)])
def test_conv_matches_bruteforce(act, shape):
    N, Cin, H, W, Cout = shape
    x, w, b = rng_case(sum(shape) + act, N, Cin, H, W, Cout)
    ref = np_act(np_conv_valid(x, w, b), act)
    full = oracle.conv_act_pool(x, w, b, act, 0)
    np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-13)
    pooled = oracle.conv_act_pool(x, w, b, act, 1)
    np.testing.assert_allclose(pooled, ref.mean(axis=(2, 3)), rtol=1e-12, atol=1e-13)


def test_conv_tiny_workload_bruteforce():
    spec = synth.CONV_WORKLOADS["conv_tiny"]
    x, w, b = synth.conv_inputs(spec)
    out = oracle.conv_act_pool(x, w, b, spec["act"], spec["pool"])
    assert out.shape == (2, 8)
    ref = np_gelu(np_conv_valid(x, w, b)).mean(axis=(2, 3))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_conv_single_channel_is_textbook_correlation():
    r = np.random.default_rng(7)
    x = r.normal(size=(1, 1, 13, 10)).astype(np.float32)
    w = r.normal(size=(1, 1, 3, 3)).astype(np.float32)
    b = np.array([0.25], np.float32)
    ref = scipy.signal.correlate2d(x[0, 0].astype(np.float64), w[0, 0].astype(np.float64), mode="valid") + 0.25
    out = oracle.conv_act_pool(x, w, b, oracle.ACT_NONE, 0)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-13, atol=1e-13)
    # and it is not the flipped-kernel convolution
    conv = scipy.signal.convolve2d(x[0, 0].astype(np.float64), w[0, 0].astype(np.float64), mode="valid") + 0.25
    assert np.abs(out[0, 0] - conv).max() > 1e-2


@pytest.mark.parametrize("kh,kw", [(a, c) for a in range(3) for c in range(3)])
def test_conv_shifted_delta_reproduces_input(kh, kw):
    N, C, H, W = 2, 3, 8, 9
    r = np.random.default_rng(11)
    x = r.normal(size=(N, C, H, W)).astype(np.float32)
    w = np.zeros((C, C, 3, 3), np.float32)
    for c in range(C):
        w[c, c, kh, kw] = 1.0
    b = np.zeros(C, np.float32)
    out = oracle.conv_act_pool(x, w, b, oracle.ACT_NONE, 0)
    np.testing.assert_array_equal(out, x[:, :, kh:kh + H - 2, kw:kw + W - 2].astype(np.float64))


def test_conv_zero_weights_give_act_of_bias():
    N, Cin, H, W, Cout = 2, 3, 6, 7, 4
    x = np.random.default_rng(3).normal(size=(N, Cin, H, W)).astype(np.float32)
    w = np.zeros((Cout, Cin, 3, 3), np.float32)
    b = np.array([-1.5, 0.0, 0.3, 2.0], np.float32)
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        full = oracle.conv_act_pool(x, w, b, act, 0)
        expect = np.array([oracle.act(float(v), act) for v in b])
        np.testing.assert_allclose(full, np.broadcast_to(expect[None, :, None, None], full.shape), rtol=0, atol=0)
        pooled = oracle.conv_act_pool(x, w, b, act, 1)
        np.testing.assert_allclose(pooled, np.broadcast_to(expect, pooled.shape), rtol=1e-15, atol=1e-16)


def test_conv_constant_map_pool_equals_activation():
    N, Cin, H, W, Cout = 2, 4, 10, 12, 3
    c = 0.75
    x = np.full((N, Cin, H, W), c, np.float32)
    r = np.random.default_rng(5)
    w = r.uniform(-0.4, 0.4, (Cout, Cin, 3, 3)).astype(np.float32)
    b = r.uniform(-0.2, 0.2, Cout).astype(np.float32)
    pre = b.astype(np.float64) + c * w.astype(np.float64).sum(axis=(1, 2, 3))
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        pooled = oracle.conv_act_pool(x, w, b, act, 1)
        np.testing.assert_allclose(pooled, np.broadcast_to(np_act(pre, act), pooled.shape), rtol=1e-13)


def test_conv_pool_divisor_is_valid_area():
    # x = 0, w = 0: every output equals act(b); with a non-constant act(b) the mean must
    # still be act(b), which only holds if the divisor counts exactly the valid OHxOW map.
    N, Cin, H, W, Cout = 1, 1, 5, 8, 1
    x = np.zeros((N, Cin, H, W), np.float32)
    w = np.zeros((Cout, Cin, 3, 3), np.float32)
    w[0, 0, 0, 0] = 1.0
    x[0, 0, 0, 0] = 6.0  # exactly one valid output differs
    b = np.zeros(1, np.float32)
    pooled = oracle.conv_act_pool(x, w, b, oracle.ACT_NONE, 1)
    assert pooled[0, 0] == pytest.approx(6.0 / ((H - 2) * (W - 2)), rel=1e-15)


def test_conv_linearity():
    N, Cin, H, W, Cout = 2, 3, 7, 6, 5
    x1, w, b = rng_case(21, N, Cin, H, W, Cout)
    x2, _, _ = rng_case(22, N, Cin, H, W, Cout)
    x1 = (np.round(x1 * 256) / 256).astype(np.float32)  # multiples of 2^-8: the
    x2 = (np.round(x2 * 256) / 256).astype(np.float32)  # combination below is exact in fp32
    x3 = (np.float32(0.5) * x1 - np.float32(2.0) * x2).astype(np.float32)
    y1 = oracle.conv_act_pool(x1, w, b, 0, 0) - b[None, :, None, None]
    y2 = oracle.conv_act_pool(x2, w, b, 0, 0) - b[None, :, None, None]
    y3 = oracle.conv_act_pool(x3, w, b, 0, 0) - b[None, :, None, None]
    np.testing.assert_allclose(y3, 0.5 * y1 - 2.0 * y2, rtol=1e-12, atol=1e-13)


def test_conv_samples_agree_with_full():
    N, Cin, H, W, Cout = 3, 4, 11, 9, 6
    x, w, b = rng_case(31, N, Cin, H, W, Cout)
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        full = oracle.conv_act_pool(x, w, b, act, 0)
        pooled = oracle.conv_act_pool(x, w, b, act, 1)
        r = np.random.default_rng(1)
        n, oc = r.integers(0, N, 20), r.integers(0, Cout, 20)
        oh, ow = r.integers(0, H - 2, 20), r.integers(0, W - 2, 20)
        pts = oracle.conv_point_sample(x, w, b, act, n, oc, oh, ow)
        np.testing.assert_array_equal(pts, full[n, oc, oh, ow])
        ps = oracle.conv_pool_sample(x, w, b, act, n, oc)
        np.testing.assert_array_equal(ps, pooled[n, oc])


def test_conv_bf16_widening_is_exact():
    N, Cin, H, W, Cout = 2, 3, 6, 6, 2
    x, w, b = rng_case(41, N, Cin, H, W, Cout)
    xb, wb = synth.to_bf16_bits(x).reshape(x.shape), synth.to_bf16_bits(w).reshape(w.shape)
    xf, wf = synth.bf16_bits_to_f32(xb), synth.bf16_bits_to_f32(wb)
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        np.testing.assert_array_equal(oracle.conv_act_pool(xb, wb, b, act, 0),
                                      oracle.conv_act_pool(xf, wf, b, act, 0))
    np.testing.assert_allclose(oracle.conv_act_pool(xb, wb, b, 0, 0), np_conv_valid(xf, wf, b), rtol=1e-12)


def test_conv_rejects_bad_shapes():
    x = np.zeros((1, 2, 2, 5), np.float32)
    w = np.zeros((1, 2, 3, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.conv_act_pool(x, w, np.zeros(1, np.float32), 1, 1)


# ------------------------------------------------------------------ GEMM + logsumexp
def np_gemm_lse_mish(X, W, b, scale, cmin, cmax):
    y = scale * (X.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64))
    c = np.clip(y, cmin, cmax)
    z = scipy.special.logsumexp(c, axis=1)
    return z * np_mish(z), z


@pytest.mark.parametrize("M,K,N", [(5, 7, 9), (16, 64, 48), (3, 1, 1), (37, 19, 53)])
def test_gemm_lse_matches_blas_and_logsumexp(M, K, N):
    r = np.random.default_rng(M * 1000 + K * 10 + N)
    X = r.normal(size=(M, K)).astype(np.float32)
    W = r.uniform(-0.5, 0.5, (N, K)).astype(np.float32)
    b = r.uniform(-0.5, 0.5, N).astype(np.float32)
    for scale, cmin, cmax in [(4.0, -10.0, 10.0), (4.0, -0.5, 0.7), (1.0, -1e30, 1e30)]:
        out, z = oracle.gemm_lse_mish(X, W, b, scale, cmin, cmax)
        ro, rz = np_gemm_lse_mish(X, W, b, scale, cmin, cmax)
        np.testing.assert_allclose(z, rz, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,K,N", [(5, 8, 9), (7, 37, 40)])
def test_gemm_lse_bf16_inputs_match_blas_on_widened_values(M, K, N):
    # bfloat16 is the top half of a float32: widening appends 16 zero bits
    r = np.random.default_rng(M + K + N)
    Xb = r.integers(0, 1 << 16, (M, K), dtype=np.uint16)
    Wb = r.integers(0, 1 << 16, (N, K), dtype=np.uint16)
    # keep finite, moderate values: exponent field 0x7A..0x82 (about 2^-5 .. 2^3), random signs
    Xb = (Xb & 0x807F) | (((Xb >> 8) % 9 + 0x7A) << 7).astype(np.uint16)
    Wb = (Wb & 0x807F) | (((Wb >> 8) % 9 + 0x7A) << 7).astype(np.uint16)
    b = r.uniform(-0.5, 0.5, N).astype(np.float32)
    Xf = (Xb.astype(np.uint32) << 16).view(np.float32)
    Wf = (Wb.astype(np.uint32) << 16).view(np.float32)
    for scale, cmin, cmax in [(4.0, -10.0, 10.0), (0.01, -1.0, 2.0)]:
        out, z = oracle.gemm_lse_mish(Xb, Wb, b, scale, cmin, cmax)
        ro, rz = np_gemm_lse_mish(Xf, Wf, b, scale, cmin, cmax)
        np.testing.assert_allclose(z, rz, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-12)
    with pytest.raises(TypeError):
        oracle.gemm_lse_mish(Xb, Wf, b, 4.0, -10.0, 10.0)


def test_lse_constant_row():
    M, K, N = 3, 4, 6144
    X = np.ones((M, K), np.float32)
    W = np.zeros((N, K), np.float32)
    for beta in (-0.3, 0.0, 0.01, 1.5, 9.0):
        b = np.full(N, beta, np.float32)
        out, z = oracle.gemm_lse_mish(X, W, b, 4.0, -10.0, 10.0)
        c = min(max(4.0 * float(np.float32(beta)), -10.0), 10.0)
        np.testing.assert_allclose(z, c + math.log(N), rtol=1e-14)
        zz = c + math.log(N)
        np.testing.assert_allclose(out, zz * zz * math.tanh(math.log1p(math.exp(zz))), rtol=1e-13)


def test_lse_clamp_bounds_and_max_bounds():
    M, K, N = 6, 32, 500
    r = np.random.default_rng(9)
    X = r.normal(scale=3.0, size=(M, K)).astype(np.float32)
    W = r.normal(size=(N, K)).astype(np.float32)
    b = r.normal(size=N).astype(np.float32)
    cmin, cmax = -10.0, 10.0
    _, z = oracle.gemm_lse_mish(X, W, b, 4.0, cmin, cmax)
    assert np.all(z >= cmin + math.log(N) - 1e-12) and np.all(z <= cmax + math.log(N) + 1e-12)
    y = np.clip(4.0 * (X.astype(np.float64) @ W.T.astype(np.float64) + b), cmin, cmax)
    assert np.all(z >= y.max(axis=1) - 1e-12) and np.all(z <= y.max(axis=1) + math.log(N) + 1e-12)


def test_lse_shift_equivariance_and_column_permutation():
    r = np.random.default_rng(12)
    c = r.uniform(-5, 5, (4, 257))
    _, z = oracle.lse_mish_rows(c)
    _, z2 = oracle.lse_mish_rows(c + 3.25)
    np.testing.assert_allclose(z2, z + 3.25, rtol=1e-14)
    _, z3 = oracle.lse_mish_rows(c[:, r.permutation(257)])
    np.testing.assert_allclose(z3, z, rtol=1e-14)
    # no overflow without the shift being applied: huge values must still work
    _, z4 = oracle.lse_mish_rows(c + 800.0)
    np.testing.assert_allclose(z4, z + 800.0, rtol=1e-14)


def _mish_rational(v):
    """mish(v) = v (e^2v + 2e^v) / (e^2v + 2e^v + 2): tanh(log(1 + t)) = ((1+t)^2 - 1) / ((1+t)^2 + 1),
    t = e^v -- an algebraic form with no tanh or softplus in it."""
    t = np.exp(v)
    q = t * t + 2.0 * t
    return v * q / (q + 2.0)


def test_lse_mish_rows_matches_scipy_and_closed_forms():
    # random rows: z against SciPy's logsumexp, out against z * mish(z) in the rational form
    r = np.random.default_rng(31)
    c = r.uniform(-10.0, 10.0, (5, 613))
    out, z = oracle.lse_mish_rows(c)
    rz = scipy.special.logsumexp(c, axis=1)
    np.testing.assert_allclose(z, rz, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out, rz * _mish_rational(rz), rtol=1e-13)
    # a constant row c gives z = c + ln N exactly (every shifted term is e^0 = 1)
    for cval, N in ((-10.0, 6144), (0.0, 1), (2.5, 7), (10.0, 8192)):
        out, z = oracle.lse_mish_rows(np.full((2, N), cval))
        zz = cval + math.log(N)
        np.testing.assert_allclose(z, zz, rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(out, zz * _mish_rational(zz), rtol=1e-13, atol=1e-15)
    # the l2_p22 page's worked example: every value clamped at 10 over 8192 columns
    g = json.load(open(os.path.join(GOLDEN, "lse_all_clamped.json")))
    out, z = oracle.lse_mish_rows(np.full((1, g["N"]), g["clamp_value"]))
    assert abs(z[0] - g["lse_approx"]) < g["lse_approx_tol"]
    assert abs(out[0] - g["out_approx"]) < g["out_approx_tol"]
    # one dominant entry: z lies in [max, max + ln N] and tends to the max
    row = np.full((1, 100), -50.0)
    row[0, 37] = 3.0
    _, z = oracle.lse_mish_rows(row)
    assert 3.0 <= z[0] <= 3.0 + 99 * math.exp(-53.0) + 1e-15


def test_lse_pages_worked_magnitude_example():
    g = json.load(open(os.path.join(GOLDEN, "lse_all_clamped.json")))
    N, v = g["N"], g["clamp_value"]
    M, K = 2, 8
    X = np.ones((M, K), np.float32)
    W = np.full((N, K), 1.0, np.float32)  # every y = 4*(8+0) = 32 -> clamped to 10
    b = np.zeros(N, np.float32)
    out, z = oracle.gemm_lse_mish(X, W, b, 4.0, -10.0, v)
    assert np.all(np.abs(z - g["lse_approx"]) < g["lse_approx_tol"])
    assert np.all(np.abs(out - g["out_approx"]) < g["out_approx_tol"])
    np.testing.assert_allclose(z, v + math.log(N), rtol=1e-15)


def test_gemm_row_selection_matches_all_rows():
    spec = dict(M=9, K=33, N=70, w_bound=0.2, b_bound=0.2)
    X, W, b = synth.gemm_inputs(spec, seed_cfg=77)
    out, z = oracle.gemm_lse_mish(X, W, b, 4.0, -10.0, 10.0)
    rows = np.array([8, 0, 3, 3])
    o2, z2 = oracle.gemm_lse_mish(X, W, b, 4.0, -10.0, 10.0, rows=rows)
    np.testing.assert_array_equal(o2, out[rows])
    np.testing.assert_array_equal(z2, z[rows])


def test_gemm_bias_is_added_before_scale():
    X = np.zeros((1, 2), np.float32)
    W = np.zeros((3, 2), np.float32)
    b = np.array([0.5, 0.5, 0.5], np.float32)
    _, z = oracle.gemm_lse_mish(X, W, b, 4.0, -10.0, 10.0)
    assert z[0] == pytest.approx(2.0 + math.log(3), rel=1e-15)


# ------------------------------------------------------------------ general geometry (K x K, stride, padding)
def np_conv2d(x, w, b, stride, pad):
    """Zero-pad, then take strided K x K windows (independent of the oracle's loops)."""
    x = np.pad(np.asarray(x, np.float64), ((0, 0), (0, 0), (pad, pad), (pad, pad)))
    K = w.shape[-1]
    win = np.lib.stride_tricks.sliding_window_view(x, (K, K), axis=(2, 3))[:, :, ::stride, ::stride]
    return np.einsum("ncyxij,ocij->noyx", win, np.asarray(w, np.float64)) + np.asarray(b, np.float64)[None, :, None, None]


GEOMS = [(1, 1, 0), (1, 2, 0), (3, 1, 1), (3, 2, 1), (3, 2, 0), (5, 1, 2), (5, 2, 2), (5, 1, 0), (3, 1, 2)]


@pytest.mark.parametrize("K,S,P", GEOMS)
@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_GELU, oracle.ACT_MISH2, oracle.ACT_GELU_TANH])
def test_conv2d_matches_torch_and_bruteforce(K, S, P, act):
    import torch
    r = np.random.default_rng(K * 100 + S * 10 + P + act)
    x = r.uniform(-1, 1, (2, 3, 11, 9)).astype(np.float32)
    w = r.uniform(-0.3, 0.3, (4, 3, K, K)).astype(np.float32)
    b = r.uniform(-0.5, 0.5, 4).astype(np.float32)
    pre = torch.nn.functional.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                                     torch.from_numpy(b).double(), stride=S, padding=P).numpy()
    np.testing.assert_allclose(np_conv2d(x, w, b, S, P), pre, rtol=1e-12, atol=1e-13)
    ref = np_act(pre, act)
    full = oracle.conv2d_act_pool(x, w, b, S, P, act, 0)
    assert full.shape == ref.shape == (2, 4) + oracle.conv2d_out_size(11, 9, K, S, P)
    np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.conv2d_act_pool(x, w, b, S, P, act, 1), ref.mean(axis=(2, 3)),
                               rtol=1e-12, atol=1e-13)


def test_conv2d_reduces_to_the_3x3_valid_oracle():
    x, w, b = rng_case(77, 2, 5, 10, 12, 6)
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        for pool in (0, 1):
            np.testing.assert_array_equal(oracle.conv2d_act_pool(x, w, b, 1, 0, act, pool),
                                          oracle.conv_act_pool(x, w, b, act, pool))


def test_conv2d_1x1_is_a_channel_matmul():
    r = np.random.default_rng(3)
    x = r.normal(size=(2, 6, 5, 7)).astype(np.float32)
    w = r.normal(size=(3, 6, 1, 1)).astype(np.float32)
    b = r.normal(size=3).astype(np.float32)
    expect = np.einsum("nchw,oc->nohw", x.astype(np.float64), w[:, :, 0, 0].astype(np.float64)) + b[None, :, None, None]
    np.testing.assert_allclose(oracle.conv2d_act_pool(x, w, b, 1, 0, oracle.ACT_NONE, 0), expect, rtol=1e-13)
    # stride 2 keeps every other row and column
    np.testing.assert_allclose(oracle.conv2d_act_pool(x, w, b, 2, 0, oracle.ACT_NONE, 0), expect[:, :, ::2, ::2],
                               rtol=1e-13)


def test_conv2d_zero_padding_counts_taps_at_the_border():
    # x = 1 everywhere, w = 1 everywhere, b = 0, 3x3 with padding 1: an output sums the
    # in-range taps times Cin -- 4 at a corner, 6 on an edge, 9 inside
    Cin = 2
    x = np.ones((1, Cin, 5, 6), np.float32)
    w = np.ones((1, Cin, 3, 3), np.float32)
    out = oracle.conv2d_act_pool(x, w, np.zeros(1, np.float32), 1, 1, oracle.ACT_NONE, 0)[0, 0]
    assert out.shape == (5, 6)
    assert out[0, 0] == out[0, -1] == out[-1, 0] == out[-1, -1] == 4 * Cin
    assert out[0, 2] == out[2, 0] == out[-1, 3] == out[3, -1] == 6 * Cin
    assert np.all(out[1:-1, 1:-1] == 9 * Cin)
    # zero weights: act(b) everywhere, padded border included; the mean divides by OH * OW
    b = np.array([0.7], np.float32)
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        full = oracle.conv2d_act_pool(x, 0 * w, b, 2, 2, act, 0)
        assert full.shape == (1, 1, 4, 4)
        np.testing.assert_allclose(full, oracle.act(float(b[0]), act), rtol=1e-15)
        assert oracle.conv2d_act_pool(x, 0 * w, b, 2, 2, act, 1)[0, 0] == pytest.approx(oracle.act(float(b[0]), act),
                                                                                       rel=1e-15)


def test_conv2d_samples_match_full():
    x, w, b = rng_case(5, 3, 4, 13, 12, 5)
    w5 = np.random.default_rng(1).uniform(-0.2, 0.2, (5, 4, 5, 5)).astype(np.float32)
    full = oracle.conv2d_act_pool(x, w5, b, 2, 2, oracle.ACT_GELU, 0)
    pooled = oracle.conv2d_act_pool(x, w5, b, 2, 2, oracle.ACT_GELU, 1)
    n, oc = np.array([0, 2, 1]), np.array([4, 0, 2])
    np.testing.assert_array_equal(oracle.conv2d_pool_sample(x, w5, b, 2, 2, oracle.ACT_GELU, n, oc), pooled[n, oc])
    oh, ow = np.array([0, 6, 3]), np.array([5, 0, 2])
    np.testing.assert_array_equal(oracle.conv2d_point_sample(x, w5, b, 2, 2, oracle.ACT_GELU, n, oc, oh, ow),
                                  full[n, oc, oh, ow])
    with pytest.raises(ValueError):
        oracle.conv2d_point_sample(x, w5, b, 2, 2, oracle.ACT_GELU, [0], [0], [7], [0])  # OH = 7


# ------------------------------------------------------------------ epilogue-only operations
@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_GELU, oracle.ACT_MISH2, oracle.ACT_GELU_TANH])
def test_act_pool_map_matches_numpy(act):
    r = np.random.default_rng(100 + act)
    x = r.normal(scale=2.0, size=(3, 5, 7, 9)).astype(np.float32)
    got = oracle.act_pool_map(x, act)
    ref = np_act(x.astype(np.float64), act).mean(axis=(2, 3))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_act_pool_map_constant_map_and_divisor():
    x = np.full((2, 3, 4, 6), -0.75, np.float32)
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        np.testing.assert_allclose(oracle.act_pool_map(x, act), np.full((2, 3), oracle.act(-0.75, act)), rtol=1e-15)
    x = np.zeros((1, 1, 5, 8), np.float32)
    x[0, 0, 4, 7] = 40.0  # act none: a single non-zero element divided by the whole map
    assert oracle.act_pool_map(x, oracle.ACT_NONE)[0, 0] == pytest.approx(1.0, rel=1e-15)


def test_act_pool_map_equals_conv_oracle_on_its_output():
    N, Cin, H, W, Cout = 2, 3, 9, 8, 4
    x, w, b = rng_case(123, N, Cin, H, W, Cout)
    pre = oracle.conv_act_pool(x, w, b, oracle.ACT_NONE, 0)
    for act in (oracle.ACT_GELU, oracle.ACT_MISH2):
        fused = oracle.conv_act_pool(x, w, b, act, 1)
        np.testing.assert_allclose(oracle.act_pool_map(pre.astype(np.float32), act), fused, rtol=0, atol=1e-6)


@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_GELU, oracle.ACT_MISH2, oracle.ACT_GELU_TANH])
def test_act_elementwise_matches_numpy(act):
    x = np.linspace(-30, 30, 1001).astype(np.float32)
    # atol: for v << 0 the exact-form GELU's 1 + erf(v/sqrt2) cancels in fp64 (|error| < 1e-15)
    np.testing.assert_allclose(oracle.act_elementwise(x, act), np_act(x.astype(np.float64), act), rtol=1e-13,
                               atol=1e-15)


def test_scale_clamp_lse_mish_matches_scipy_and_gemm_oracle():
    r = np.random.default_rng(5)
    y = r.normal(scale=3.0, size=(6, 333)).astype(np.float32)
    for scale, cmin, cmax in [(4.0, -10.0, 10.0), (-1.5, -2.0, 0.5)]:
        out, z = oracle.scale_clamp_lse_mish(y, scale, cmin, cmax)
        c = np.clip(scale * y.astype(np.float64), cmin, cmax)
        rz = scipy.special.logsumexp(c, axis=1)
        np.testing.assert_allclose(z, rz, rtol=1e-13)
        np.testing.assert_allclose(out, rz * np_mish(rz), rtol=1e-13)
    # the GEMM path is this function applied to the Linear output (up to fp32 rounding of y)
    X = r.normal(size=(4, 16)).astype(np.float32)
    W = r.uniform(-0.3, 0.3, (50, 16)).astype(np.float32)
    b = r.uniform(-0.3, 0.3, 50).astype(np.float32)
    y32 = (X.astype(np.float64) @ W.T.astype(np.float64) + b).astype(np.float32)
    o1, _ = oracle.gemm_lse_mish(X, W, b, 4.0, -10.0, 10.0)
    o2, _ = oracle.scale_clamp_lse_mish(y32, 4.0, -10.0, 10.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-6)


def test_scale_clamp_lse_constant_rows_and_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "lse_all_clamped.json")))
    y = np.full((2, g["N"]), 7.0, np.float32)  # 4 * 7 = 28 -> clamped to 10 everywhere
    out, z = oracle.scale_clamp_lse_mish(y, 4.0, -10.0, g["clamp_value"])
    assert np.all(np.abs(z - g["lse_approx"]) < g["lse_approx_tol"])
    assert np.all(np.abs(out - g["out_approx"]) < g["out_approx_tol"])
    np.testing.assert_allclose(z, 10.0 + math.log(g["N"]), rtol=1e-15)
