"""Pins of the AdamW oracle (oracle.c or_adamw, oracle.lr_at / adamw_scalars),
CPU only: the schedule's closed forms, the scalars' definitions, agreement of
the binary32 update with a binary64 evaluation of the same formula within its
rounding-error bound (a dropped term or swapped beta fails it by orders of
magnitude), flushed subnormal gradients, and the decay switch."""
import math

import numpy as np
import pytest

import oracle

C = oracle.ADAMW


def test_schedule_closed_forms():
    W, T, pk, mn = C["warmup_tokens"], C["total_tokens"], C["peak_lr"], C["min_lr"]
    assert oracle.lr_at(0.0) == 0.0
    assert math.isclose(oracle.lr_at(W / 2), pk / 2, rel_tol=1e-15)
    assert math.isclose(oracle.lr_at(W), pk, rel_tol=1e-15)
    assert math.isclose(oracle.lr_at((W + T) / 2), (pk + mn) / 2, rel_tol=1e-12)
    assert math.isclose(oracle.lr_at(T), mn, rel_tol=1e-15)
    assert oracle.lr_at(10 * T) == oracle.lr_at(T)
    xs = np.linspace(W, T, 1000)
    lrs = [oracle.lr_at(x) for x in xs]
    assert all(a >= b for a, b in zip(lrs, lrs[1:]))


def test_scalars():
    s = oracle.adamw_scalars(1, 1e9)
    assert s["c1"] == float(np.float32(0.1)) and s["bc1"] == s["c1"]
    assert s["c2"] == float(np.float32(0.05)) and s["bc2"] == s["c2"]
    s = oracle.adamw_scalars(100000, 1e11)
    assert s["bc1"] == 1.0 and s["bc2"] == 1.0
    assert s["d"] == float(np.float32(s["lr"] * 0.1)) or abs(s["d"] - s["lr"] * 0.1) < 1e-12


def _ref64(p, g, m, v, sc, decay):
    p, g, m, v = (x.astype(np.float64) for x in (p, g, m, v))
    m = sc["beta1"] * m + sc["c1"] * g
    v = sc["beta2"] * v + sc["c2"] * g * g
    u = (m / sc["bc1"]) / (np.sqrt(v / sc["bc2"]) + sc["eps"])
    if decay:
        p = p - sc["d"] * p
    return p - sc["lr"] * u, m, v


@pytest.mark.parametrize("step,tokens,decay", [(1, 1e8, True), (7, 3e9, False), (5000, 2e11, True)])
def test_update_matches_binary64_within_rounding(step, tokens, decay):
    g_ = np.random.default_rng(step)
    n = 20000
    p = g_.standard_normal(n).astype(np.float32)
    g = (g_.standard_normal(n) * 1e-2).astype(np.float32)
    m = (g_.standard_normal(n) * 1e-3).astype(np.float32)
    v = (np.abs(g_.standard_normal(n)) * 1e-5).astype(np.float32)
    sc = oracle.adamw_scalars(step, tokens)
    wp, wm, wv = _ref64(p, g, m, v, sc, decay)
    P, M, V = p.copy(), m.copy(), v.copy()
    oracle.adamw(P, g, M, V, sc, decay)
    eps32 = 2.0 ** -24
    assert np.all(np.abs(M - wm) <= 4 * eps32 * (np.abs(sc["beta1"] * m) + np.abs(sc["c1"] * g)) + 1e-45)
    assert np.all(np.abs(V - wv) <= 6 * eps32 * (np.abs(sc["beta2"] * v) + np.abs(sc["c2"] * g * g)) + 1e-45)
    # the step lr*u with |u| <~ sqrt(1/((1-b2)...)): bound the p error by ulps of p and of the step
    step_mag = np.abs(sc["lr"] * (wm / sc["bc1"]) / (np.sqrt(wv / sc["bc2"]) + sc["eps"]))
    assert np.all(np.abs(P - wp) <= 4 * eps32 * np.abs(wp) + 12 * eps32 * step_mag + 1e-45)
    # and the update really moved p by about the Adam step (a dropped term fails this)
    assert np.median(np.abs(P - p)) > 0.1 * sc["lr"]


def test_subnormal_gradients_read_as_zero():
    n = 64
    p = np.linspace(-1, 1, n).astype(np.float32)
    m = np.full(n, 1e-3, np.float32)
    v = np.full(n, 1e-6, np.float32)
    sc = oracle.adamw_scalars(3, 1e9)
    g_sub = np.full(n, 1e-40, np.float32)
    g_sub[::2] *= -1
    outs = []
    for g in (g_sub, np.zeros(n, np.float32)):
        P, M, V = p.copy(), m.copy(), v.copy()
        oracle.adamw(P, g, M, V, sc, True)
        outs.append((P, M, V))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_no_decay_and_zero_moments_leave_p():
    n = 100
    p = np.random.default_rng(4).standard_normal(n).astype(np.float32)
    p[0] = -0.0
    z = np.zeros(n, np.float32)
    sc = oracle.adamw_scalars(2, 1e9)
    P = p.copy()
    oracle.adamw(P, z, z.copy(), z.copy(), sc, False)
    assert np.array_equal(P.view(np.uint32), p.view(np.uint32))
    P = p.copy()
    oracle.adamw(P, z, z.copy(), z.copy(), sc, True)      # pure decay: p - d*p
    assert np.all(np.abs(P - p * (1 - sc["d"])) <= 2 * 2.0 ** -24 * np.abs(p))
