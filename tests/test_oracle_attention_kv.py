"""Pins of the oracle's key and value gradients of the int8 P.V attention
(onedev.kr summary, "Use", attention paragraph; the pages give the 64-bit
fixed-point accumulation for the query gradient only, and the same format is
this library's reading for dK and dV).  Each test fixes or_attn_bwd_dkdv_rows
against something other than itself: the float64 gradient of the textbook
attention (checked by central differences), a closed form where the softmax
is exact, the grouped-query structure, the LSQ range mask of V, and the
identity that ties dK to the separately pinned dQ."""
import numpy as np
import pytest

import oracle

D = 128
C = 1.0 / np.sqrt(D)


def _inputs(B, S, Hq, Hkv, seed, q_scale=0.5):
    g = np.random.default_rng(seed)
    Q = (g.standard_normal((B, S, Hq, D)) * q_scale).astype(np.float32)
    K = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    V = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    dO = (g.standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    return Q, K, V, dO


def _lo(i, window):
    return max(0, i - window + 1) if window > 0 else 0


def _quantize_v(V, s_v):
    """LSQ quantiser written independently: IEEE binary32 quotient (numpy),
    round half to even, clamp to [-127, 127]; with the range mask."""
    t = (V / np.float32(s_v)).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int64), np.abs(t) <= 127


def _f64_grads(Q, K, Vh, dO, window):
    """Output, and the gradients with respect to K and Vh, of
    f = sum(dO * softmax(Q K^T / sqrt(D)) Vh) in float64, with the
    magnitudes that bound binary32 rounding of each gradient entry."""
    B, S, Hq, _ = Q.shape
    Hkv = K.shape[2]
    O = np.zeros(Q.shape)
    dK, dV = np.zeros(K.shape), np.zeros(K.shape)
    mK, mV = np.zeros(K.shape), np.zeros(K.shape)
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(S):
                lo = _lo(i, window)
                k = K[b, lo:i + 1, hk].astype(np.float64)
                q = Q[b, i, h].astype(np.float64)
                go = dO[b, i, h].astype(np.float64)
                s = k @ q * C
                P = np.exp(s - s.max())
                P /= P.sum()
                v = Vh[b, lo:i + 1, hk]
                O[b, i, h] = P @ v
                dp = v @ go
                delta = P @ dp
                dK[b, lo:i + 1, hk] += C * np.outer(P * (dp - delta), q)
                dV[b, lo:i + 1, hk] += np.outer(P, go)
                mag = np.abs(v) @ np.abs(go) + np.abs(O[b, i, h]) @ np.abs(go)
                mK[b, lo:i + 1, hk] += C * np.outer(P * mag, np.abs(q))
                mV[b, lo:i + 1, hk] += np.outer(P, np.abs(go))
    return O, dK, dV, mK, mV


def _f64_loss(Q, K, Vh, dO, window):
    B, S, Hq, _ = Q.shape
    Hkv = K.shape[2]
    tot = 0.0
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(S):
                lo = _lo(i, window)
                s = K[b, lo:i + 1, hk].astype(np.float64) @ Q[b, i, h].astype(np.float64) * C
                P = np.exp(s - s.max())
                tot += (P / P.sum()) @ Vh[b, lo:i + 1, hk] @ dO[b, i, h].astype(np.float64)
    return tot


def test_zero_output_gradient_gives_zero():
    Q, K, V, dO = _inputs(1, 70, 2, 1, seed=41)
    O = oracle.attn_fwd(Q, K, V, 0, 0.05)
    dk, dv = oracle.attn_bwd_dkdv(Q, K, V, O, np.zeros_like(dO), 0, 0.05)
    assert np.all(dk.view(np.uint32) == 0) and np.all(dv.view(np.uint32) == 0)


@pytest.mark.parametrize("window", [0, 20])
def test_match_the_float64_gradient(window):
    """With O given as the float64 attention output rounded to binary32 (so
    that Delta = dO . O is the textbook one), dK and dV agree with the float64
    gradient to binary32 rounding (1e-6 of the entry's magnitude) plus the
    2^-40 grid of every tile sum.  Two query tiles, a ragged tail and two query
    heads per KV head.  Planted mistakes in the float64 reference (no 1/sqrt(D),
    no Delta, the wrong head of the group) leave the bound."""
    B, S, Hq, Hkv, s_v = 1, 70, 4, 2, 0.05
    Q, K, V, dO = _inputs(B, S, Hq, Hkv, seed=43 + window)
    qv, inr = _quantize_v(V, s_v)
    Vh = (qv.astype(np.float32) * np.float32(s_v)).astype(np.float64)
    O64, rk, rv, mk, mv = _f64_grads(Q, K, Vh, dO, window)
    # the float64 gradients against central differences of the float64 loss
    for (j, hk, d) in [(0, 0, 0), (33, 1, 7), (69, 0, 127)]:
        e = 1e-3
        Kp, Km = K.astype(np.float64).copy(), K.astype(np.float64).copy()
        Kp[0, j, hk, d] += e
        Km[0, j, hk, d] -= e
        fd = (_f64_loss(Q, Kp, Vh, dO, window) - _f64_loss(Q, Km, Vh, dO, window)) / (2 * e)
        assert abs(fd - rk[0, j, hk, d]) <= 1e-6 * max(1.0, abs(fd)) + 1e-9
        Vp, Vm = Vh.copy(), Vh.copy()
        Vp[0, j, hk, d] += e
        Vm[0, j, hk, d] -= e
        fd = (_f64_loss(Q, K, Vp, dO, window) - _f64_loss(Q, K, Vm, dO, window)) / (2 * e)
        assert abs(fd - rv[0, j, hk, d]) <= 1e-6 * max(1.0, abs(fd)) + 1e-9
    dk, dv = oracle.attn_bwd_dkdv(Q, K, V, O64.astype(np.float32), dO, window, s_v)
    tiles = 2 * (Hq // Hkv) * 2.0 ** -40
    bk = 1e-6 * mk + tiles
    bv = 1e-6 * mv + tiles
    assert np.all(np.abs(dk - rk) <= bk)
    assert np.all(np.abs(dv - np.where(inr, rv, 0.0)) <= bv)
    # planted mistakes
    assert np.any(np.abs(dk - rk / C) > bk)
    rk_nodelta = np.zeros(K.shape)
    for h in range(Hq):
        hk = h // (Hq // Hkv)
        for i in range(S):
            lo = _lo(i, window)
            k = K[0, lo:i + 1, hk].astype(np.float64)
            s = k @ Q[0, i, h].astype(np.float64) * C
            P = np.exp(s - s.max())
            P /= P.sum()
            dp = Vh[0, lo:i + 1, hk] @ dO[0, i, h].astype(np.float64)
            rk_nodelta[0, lo:i + 1, hk] += C * np.outer(P * dp, Q[0, i, h])
    assert np.any(np.abs(dk - rk_nodelta) > bk)
    swapped = dO.copy()
    swapped[:, :, [0, 1]] = dO[:, :, [1, 0]]
    _, _, rv_swapped, _, _ = _f64_grads(Q, K, Vh, swapped, window)
    assert np.any(np.abs(dv - np.where(inr, rv_swapped, 0.0)) > bv)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2)])
def test_window_of_one_closed_form(Hq, Hkv):
    """Window 1: every row attends only itself, so P = E(0) / E(0) = 1 and dV_j
    is the sum of the group's dO rows at j, added exactly (dO on a 2^-20 grid)
    and rounded once.  With O = V^ given as the output, dP and Delta are the
    same canonical sum, dS = +0 and dK = 0 exactly."""
    B, S, s_v = 2, 70, 0.05
    Q, K, V, _ = _inputs(B, S, Hq, Hkv, seed=47)
    g = np.random.default_rng(48)
    dO = (g.integers(-2 ** 19, 2 ** 19, size=Q.shape) * 2.0 ** -20).astype(np.float32)
    qv, inr = _quantize_v(V, s_v)
    Vh = (qv.astype(np.float32) * np.float32(s_v)).astype(np.float32)
    O = np.repeat(Vh, Hq // Hkv, axis=2)
    dk, dv = oracle.attn_bwd_dkdv(Q, K, V, O, dO, 1, s_v)
    assert np.all(dk.view(np.uint32) == 0)
    want = dO.astype(np.float64).reshape(B, S, Hkv, Hq // Hkv, D).sum(axis=3).astype(np.float32)
    want = np.where(inr, want, np.float32(0.0))
    assert np.array_equal(dv.view(np.uint32), want.view(np.uint32))


def test_head_with_zero_gradient_adds_nothing():
    """Two query heads on one KV head, the second with dO = 0: dK and dV are
    bit-identical to the one-head problem."""
    B, S, s_v, window = 1, 90, 0.05, 30
    Q, K, V, dO = _inputs(B, S, 2, 1, seed=49)
    dO[:, :, 1] = 0.0
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    dk2, dv2 = oracle.attn_bwd_dkdv(Q, K, V, O, dO, window, s_v)
    dk1, dv1 = oracle.attn_bwd_dkdv(Q[:, :, :1], K, V, O[:, :, :1], dO[:, :, :1], window, s_v)
    assert np.array_equal(dk2.view(np.uint32), dk1.view(np.uint32))
    assert np.array_equal(dv2.view(np.uint32), dv1.view(np.uint32))
    assert np.any(dk1 != 0) and np.any(dv1 != 0)


def test_out_of_range_values_get_no_gradient():
    """The STE of V's LSQ quantiser: entries with |v / s_v| > 127 get +0 and
    the others are unchanged."""
    B, S, s_v, window = 1, 80, 0.05, 0
    Q, K, V, dO = _inputs(B, S, 2, 1, seed=51)
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    _, dv_ref = oracle.attn_bwd_dkdv(Q, K, V, O, dO, window, s_v)
    V2 = V.copy()
    V2[0, 5, 0, 3] = 10.0          # 200 steps: clamped
    V2[0, 64, 0, 100] = -6.4       # 128 steps: clamped
    V2[0, 7, 0, 9] = 6.35          # 127 steps exactly: in range
    _, dv = oracle.attn_bwd_dkdv(Q, K, V2, O, dO, window, s_v)
    assert dv[0, 5, 0, 3].view(np.uint32) == 0 and dv[0, 64, 0, 100].view(np.uint32) == 0
    assert dv[0, 7, 0, 9] != 0
    keep = np.ones(dv.shape, bool)
    keep[0, 5, 0, 3] = keep[0, 64, 0, 100] = False
    # dV does not depend on V's values (P comes from Q and K; O is given)
    assert np.array_equal(dv[keep].view(np.uint32), dv_ref[keep].view(np.uint32))


@pytest.mark.parametrize("window", [0, 25])
def test_dk_and_dq_share_the_logit_gradient(window):
    """sum_id dQ_id Q_id and sum_jd dK_jd K_jd both equal
    sum_ij dS_ij s_ij: the separately pinned dQ oracle and the dK oracle agree
    on it to rounding."""
    B, S, Hq, Hkv, s_v = 1, 100, 4, 1, 0.05
    Q, K, V, dO = _inputs(B, S, Hq, Hkv, seed=53 + window)
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    dq = oracle.attn_bwd_dq(Q, K, V, O, dO, window, s_v).astype(np.float64)
    dk, _ = oracle.attn_bwd_dkdv(Q, K, V, O, dO, window, s_v)
    a = np.sum(dq * Q)
    b = np.sum(dk.astype(np.float64) * K)
    scale = np.sum(np.abs(dq * Q)) + np.sum(np.abs(dk.astype(np.float64) * K))
    assert abs(a - b) <= 1e-5 * scale
    assert abs(a) > 1e-3 * scale     # the identity is not trivially 0 = 0


def test_sampled_rows_agree_with_the_full_call():
    B, S, Hq, Hkv, s_v, window = 2, 100, 4, 2, 0.05, 40
    Q, K, V, dO = _inputs(B, S, Hq, Hkv, seed=57)
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    dk, dv = oracle.attn_bwd_dkdv(Q, K, V, O, dO, window, s_v)
    rows = np.array([0, 63, 64, 199, 250, 399], np.int64)
    sk, sv = oracle.attn_bwd_dkdv(Q, K, V, O, dO, window, s_v, rows=rows)
    assert np.array_equal(sk, dk.reshape(-1, D)[rows])
    assert np.array_equal(sv, dv.reshape(-1, D)[rows])
