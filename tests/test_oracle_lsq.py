"""Pins for the oracle's LSQ int8 QAT linear layer: weight step, quantiser,
int8 GEMM, dequantisation, straight-through backward and SwiGLU.

Method: onedev.kr summary of Open-1B, section "Use" (LSQ int8 QAT on every
attention/FFN linear, weight step 2*mean(|w|)/sqrt(q_max) recomputed every
step, SwiGLU gate and up computed by one GEMM) and section "How" (unfused
multiply then add, fixed reduction order, FTZ).  Readings for what the pages
leave open: RNE, clamp [-127,127], select +0 outside the STE range, s_x a
caller constant.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ---- weight step -------------------------------------------------------------
def test_sqrt127_bits():
    assert _bits(oracle.sqrt(np.float32(127))) == 0x41344F93


@pytest.mark.parametrize("shape", [(512, 512), (96, 64), (7, 33)])
def test_weight_scale_closed_form(shape):
    """W = +-c with c = 2^-6: every partial sum is exact, mean = c, so
    s_w = fl(2c / fl(sqrt 127)) computed by hand in host binary32."""
    g = np.random.default_rng(1)
    c = np.float32(2.0 ** -6)
    W = np.where(g.random(shape) < 0.5, -c, c).astype(np.float32)
    r = np.float32(np.sqrt(np.float64(127)))
    want = np.float32(np.float32(2 * c) / r)
    assert _bits(oracle.weight_scale(W)) == _bits(want)


def test_weight_scale_error_bound():
    """Random W: s_w is within the CanonSum error bound (Higham, Accuracy and
    Stability of Numerical Algorithms, ch. 4: |S - S_exact| <= gamma_h sum|w|
    with h = 31 + ceil(log2 J)) plus three roundings of 2*mean/sqrt(127)."""
    g = np.random.default_rng(2)
    W = (g.standard_normal((300, 700)) * 0.02).astype(np.float32)
    n = W.size
    J = (n + 31) // 32
    h = 31 + int(np.ceil(np.log2(J)))
    u = 2.0 ** -24
    gamma = h * u / (1 - h * u)
    exact = 2 * float(np.abs(W.astype(np.float64)).sum()) / n / np.sqrt(127.0)
    got = float(oracle.weight_scale(W))
    assert abs(got - exact) <= (gamma + 4 * u) * exact


def test_weight_scale_zero():
    assert oracle.weight_scale(np.zeros((4, 8), np.float32)) == 0.0


# ---- quantiser ------------------------------------------------------------------
def test_quantize_table():
    case = json.load(open(os.path.join(GOLDEN, "quantize_cases.json")))
    for c in case["cases"]:
        v = np.float32(c["v"])
        q, inr = oracle.quantize(np.array([v]), np.float32(c["s"]))
        assert int(q[0]) == c["q"] and bool(inr[0]) == c["in"], c


def test_quantize_halves_round_to_even():
    """t = k/2 exactly (v = t * 0.5, s = 0.5); clamp to [-127, 127]; in-range
    inclusive.  Expected values from Python's round-half-even."""
    for k in range(-300, 301):
        t = k / 2
        for tt in (np.float32(t), np.nextafter(np.float32(t), np.float32(1e9)),
                   np.nextafter(np.float32(t), np.float32(-1e9))):
            tt = np.float32(tt)
            v = np.float32(tt * np.float32(0.5))   # exact: power-of-two scaling
            q, inr = oracle.quantize(np.array([v]), np.float32(0.5))
            want_q = max(-127, min(127, round(float(tt))))
            assert int(q[0]) == want_q, (tt, q)
            assert bool(inr[0]) == (-127 <= float(tt) <= 127), tt


def test_quantize_zero_step():
    q, inr = oracle.quantize(np.array([0.0, -0.0, 1e-3], np.float32), 0.0)
    assert (q == 0).all() and inr.all()


# ---- int8 GEMM -----------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (17, 64, 9), (64, 300, 33)])
def test_gemm_i8_brute_force(M, K, N):
    g = np.random.default_rng(M * 1000 + K)
    qx = g.integers(-127, 128, (M, K)).astype(np.int8)
    qw = g.integers(-127, 128, (N, K)).astype(np.int8)
    acc, amax = oracle.gemm_i8(qx, qw)
    want = qx.astype(np.int64) @ qw.astype(np.int64).T
    assert (acc == want).all() and amax == np.abs(want).max()


def test_gemm_i8_extreme_fits_int32():
    K = 5632
    qx = np.full((2, K), 127, np.int8)
    qw = np.full((2, K), -127, np.int8)
    acc, amax = oracle.gemm_i8(qx, qw)
    assert amax == 127 * 127 * K and amax < 2**31


# ---- forward ------------------------------------------------------------------
def _small_inputs(M=37, K=70, N=45, seed=5):
    g = np.random.default_rng(seed)
    X = g.standard_normal((M, K)).astype(np.float32) * np.float32(3)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    return X, W


def test_fwd_is_dequantised_integer_product():
    """Y = fl(acc) * (s_x * s_w), recomputed here from the quantised operands
    with numpy int64 products and host binary32 multiplies."""
    X, W = _small_inputs()
    s_x = np.float32(0.05)
    Y = oracle.linear_fwd(X, W, s_x)
    s_w = oracle.weight_scale(W)
    qx, _ = oracle.quantize(X, s_x)
    qw, _ = oracle.quantize(W, s_w)
    acc = qx.astype(np.int64) @ qw.astype(np.int64).T
    want = acc.astype(np.float32) * np.float32(s_x * s_w)
    assert (_bits(Y) == _bits(want)).all()


def test_fwd_addend_is_unfused():
    X, W = _small_inputs()
    g = np.random.default_rng(9)
    Cadd = g.standard_normal((X.shape[0], W.shape[0])).astype(np.float32)
    s_x = np.float32(0.05)
    Y0 = oracle.linear_fwd(X, W, s_x)
    Y1 = oracle.linear_fwd(X, W, s_x, addend=Cadd)
    assert (_bits(Y1) == _bits(Y0 + Cadd)).all()
    # a fused version (exact product + addend, one rounding) differs somewhere
    s_w = oracle.weight_scale(W)
    qx, _ = oracle.quantize(X, s_x)
    qw, _ = oracle.quantize(W, s_w)
    acc = qx.astype(np.int64) @ qw.astype(np.int64).T
    s_y = float(np.float32(s_x * s_w))
    fused = (acc.astype(np.float64) * s_y + Cadd.astype(np.float64)).astype(np.float32)
    assert (_bits(fused) != _bits(Y1)).any()


# ---- backward ------------------------------------------------------------------
def test_ste_dyadic_exact():
    """With s_x and s_w powers of two and dyadic dY, every product and every
    partial sum is exact, so dX and dW equal the exact masked products in
    any order (float64 reference)."""
    g = np.random.default_rng(11)
    M, K, N = 70, 40, 90
    s_x = np.float32(2.0 ** -4)
    s_w = np.float32(2.0 ** -6)
    X = (g.integers(-140, 141, (M, K)) * 2.0 ** -4).astype(np.float32)       # some out of range
    W = (g.integers(-130, 131, (N, K)) * 2.0 ** -6).astype(np.float32)
    dY = (g.integers(-8, 9, (M, N)) * 2.0 ** -10).astype(np.float32)
    dX = oracle.dx_rows(dY, X, W, s_x, np.arange(M), s_w=s_w)
    dW = oracle.dw_rows(np.ascontiguousarray(dY.T), X, W, s_x, np.arange(N), s_w=s_w)
    qx = np.clip(np.round(X / s_x), -127, 127)
    qw = np.clip(np.round(W / s_w), -127, 127)
    inx = np.abs(X / s_x) <= 127
    inw = np.abs(W / s_w) <= 127
    wantX = np.where(inx, dY.astype(np.float64) @ (qw * s_w), 0.0)
    wantW = np.where(inw, dY.astype(np.float64).T @ (qx * s_x), 0.0)
    assert (dX == wantX).all() and (dW == wantW).all()
    assert (_bits(dX[~inx]) == 0).all() and (_bits(dW[~inw]) == 0).all()   # +0, not -0
    assert (~inx).any() and (~inw).any()


def test_ste_mask_is_the_surrogate_derivative():
    """Inside the range the straight-through gradient is the derivative of
    the surrogate f(v) = clamp(v/s, -127, 127) * s, i.e. 1; outside it is 0.
    Central finite differences in float64 at points away from the edges."""
    s = 0.05
    pts = np.array([-7.0, -6.36, -6.2, -1.0, 0.0, 0.3, 6.2, 6.34, 6.4, 9.0], np.float32)
    h = 1e-4
    f = lambda v: np.clip(v / s, -127, 127) * s
    slope = (f(pts.astype(np.float64) + h) - f(pts.astype(np.float64) - h)) / (2 * h)
    _, inr = oracle.quantize(pts, np.float32(s))
    assert ((slope > 0.5) == inr).all()


def test_bwd_error_bound_vs_float64():
    """dX and dW are within the CanonSum error bound of the exact sums of the
    same rounded products (plus one rounding per product)."""
    g = np.random.default_rng(13)
    M, K, N = 96, 40, 200
    X = g.standard_normal((M, K)).astype(np.float32)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    dY = (g.standard_normal((M, N)) * 1e-3).astype(np.float32)
    s_x = np.float32(0.05)
    dX, dW = oracle.linear_bwd(dY, X, W, s_x)
    s_w = oracle.weight_scale(W)
    qx, inx = oracle.quantize(X, s_x)
    qw, inw = oracle.quantize(W, s_w)
    What = (qw.astype(np.float32) * s_w).astype(np.float64)
    Xhat = (qx.astype(np.float32) * s_x).astype(np.float64)
    u = 2.0 ** -24
    for got, A, B, mask, n in ((dX, dY.astype(np.float64), What, inx, N),
                               (dW, dY.astype(np.float64).T, Xhat, inw, M)):
        exact = A @ B
        absum = np.abs(A) @ np.abs(B)
        h = 31 + int(np.ceil(np.log2(max(2, (n + 31) // 32)))) + 1
        bound = h * u / (1 - h * u) * absum
        assert (np.abs(np.where(mask, exact, 0) - got) <= bound + 1e-45).all()


def test_daz_invariance_on_subnormal_dy():
    """Subnormal dY entries act as zeros of the same sign."""
    case = synth.small_case("t", 42, 48, 64, 40, subnormal_frac=0.05)
    inp = synth.linear_inputs(case)
    dY = inp.dY
    sub = (np.abs(dY) < np.finfo(np.float32).tiny) & (dY != 0)
    assert sub.any()
    dY0 = np.where(sub, np.copysign(np.float32(0), dY), dY).astype(np.float32)
    a = oracle.linear_bwd(dY, inp.X, inp.W, np.float32(0.05))
    b = oracle.linear_bwd(dY0, inp.X, inp.W, np.float32(0.05))
    assert all((_bits(x) == _bits(y)).all() for x, y in zip(a, b))


def test_microbatch_running_sum():
    """dW over 3 microbatches = ((dW_0 + dW_1) + dW_2) in binary32."""
    g = np.random.default_rng(17)
    M, K, N = 96, 24, 20
    X = g.standard_normal((M, K)).astype(np.float32)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    dY = (g.standard_normal((M, N)) * 1e-3).astype(np.float32)
    s_x = np.float32(0.05)
    s_w = oracle.weight_scale(W)
    full = oracle.dw_rows(np.ascontiguousarray(dY.T), X, W, s_x, np.arange(N), mb=32, s_w=s_w)
    parts = [oracle.dw_rows(np.ascontiguousarray(dY[32 * b:32 * b + 32].T), X[32 * b:32 * b + 32],
                            W, s_x, np.arange(N), s_w=s_w) for b in range(3)]
    want = (parts[0] + parts[1]) + parts[2]
    assert (_bits(full) == _bits(want)).all()


def test_thread_count_invariance():
    X, W = _small_inputs(64, 50, 40)
    dY = np.random.default_rng(3).standard_normal((64, 40)).astype(np.float32)
    n0 = oracle.num_threads()
    try:
        oracle.set_threads(1)
        a = oracle.linear_bwd(dY, X, W, np.float32(0.05))
        oracle.set_threads(max(2, n0))
        b = oracle.linear_bwd(dY, X, W, np.float32(0.05))
    finally:
        oracle.set_threads(n0)
    assert all((_bits(x) == _bits(y)).all() for x, y in zip(a, b))


# ---- SwiGLU and the own exp -----------------------------------------------
def _ulp_err(got, want64):
    got64 = got.astype(np.float64)
    ulp = np.spacing(np.abs(want64).astype(np.float32)).astype(np.float64)
    return np.abs(got64 - want64) / ulp


def test_exp_constants():
    c = oracle.exp_constants()
    l2e, hi, lo = (float(x) for x in c[:3])
    assert abs(hi + lo - np.log(2.0)) < 1e-13
    assert Fraction(hi).denominator <= 2 ** 16            # 16 significant bits
    assert l2e == float(np.float32(1 / np.log(2.0)))
    fact = 1
    for i in range(8):
        fact = fact * max(i, 1)
        assert c[3 + i] == np.float32(1.0 / fact)


def test_exp_accuracy():
    xs = np.concatenate([np.linspace(-87.0, 88.0, 20001, dtype=np.float32),
                         np.linspace(-3, 3, 4001, dtype=np.float32)])
    got = np.array([oracle.exp(x) for x in xs], np.float32)
    err = _ulp_err(got, np.exp(xs.astype(np.float64)))
    assert err.max() <= 2.0, err.max()
    assert oracle.exp(np.float32(0)) == 1.0
    assert oracle.exp(np.float32(100)) == np.inf and oracle.exp(np.float32(-120)) == 0.0
    assert oracle.exp(np.float32(-88.5)) == 0.0                       # below 2^-126: flushed


def test_swiglu_forward_accuracy():
    g = np.random.default_rng(4)
    ypre = (g.standard_normal((8, 64)) * 2).astype(np.float32)
    a = oracle.swiglu_fwd(ypre)
    gate, up = ypre[:, :32].astype(np.float64), ypre[:, 32:].astype(np.float64)
    want = gate / (1 + np.exp(-gate)) * up
    assert np.allclose(a, want, rtol=1e-6, atol=1e-30)


def test_swiglu_backward_matches_derivative():
    """dg, du agree with float64 central differences of (g*sigma(g))*u."""
    g = np.random.default_rng(6)
    ypre = (g.standard_normal((4, 40)) * 2).astype(np.float32)
    dA = g.standard_normal((4, 20)).astype(np.float32)
    d = oracle.swiglu_bwd(ypre, dA).astype(np.float64)
    gate, up = ypre[:, :20].astype(np.float64), ypre[:, 20:].astype(np.float64)
    f = lambda x, y: x / (1 + np.exp(-x)) * y
    h = 1e-6
    dg = (f(gate + h, up) - f(gate - h, up)) / (2 * h) * dA
    du = (f(gate, up + h) - f(gate, up - h)) / (2 * h) * dA
    assert np.allclose(d[:, :20], dg, rtol=1e-4, atol=1e-6)
    assert np.allclose(d[:, 20:], du, rtol=1e-4, atol=1e-6)


def test_fwd_swiglu_epilogue():
    X, W = _small_inputs(20, 64, 48)
    s_x = np.float32(0.05)
    Y, ypre = oracle.linear_fwd(X, W, s_x, epilogue=1)
    assert (_bits(ypre) == _bits(oracle.linear_fwd(X, W, s_x))).all()
    assert (_bits(Y) == _bits(oracle.swiglu_fwd(ypre))).all()


def test_fwd_columns_match_rows():
    """Column sampling of Y is the same definition as row sampling."""
    X, W = _small_inputs(50, 40, 30)
    Y = oracle.linear_fwd(X, W, np.float32(0.05))
    cols = [0, 7, 29]
    assert (_bits(oracle.fwd_cols(X, W, np.float32(0.05), cols)) == _bits(Y[:, cols].T)).all()
