"""Pins of the attention oracle (int8 P.V with high-precision logits and
softmax; onedev.kr summary, "Use", attention paragraph).  Each test fixes the
oracle against something other than itself: closed forms on inputs where the
softmax is exact, a float64 textbook attention within the quantisation error
bound, and the causal / sliding-window / grouped-query structure."""
import numpy as np
import pytest

import oracle

D = 128


def _inputs(B, S, Hq, Hkv, seed, q_scale=1.0):
    g = np.random.default_rng(seed)
    Q = (g.standard_normal((B, S, Hq, D)) * q_scale).astype(np.float32)
    K = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    V = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    return Q, K, V


def _quantize_v(V, s_v):
    """LSQ quantiser written independently: IEEE binary32 quotient (numpy),
    round half to even, clamp to [-127, 127]."""
    t = (V / np.float32(s_v)).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int64)


def _lo(i, window):
    return max(0, i - window + 1) if window > 0 else 0


@pytest.mark.parametrize("window", [0, 1, 7, 33])
def test_equal_logits_give_the_window_mean(window):
    """Q = 0 makes every logit 0, so p = E(0) = 1 on the row's keys, l is the
    key count and q_p = 127: O is the mean of the dequantised V rows in the
    window, (127 * sum q_v * s_v) / (n * 127) with each step rounded."""
    B, S, Hq, Hkv, s_v = 2, 70, 4, 2, 0.05
    _, K, V = _inputs(B, S, Hq, Hkv, seed=window)
    Q = np.zeros((B, S, Hq, D), np.float32)
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    qv = _quantize_v(V, s_v)
    f = np.float32
    for b in range(B):
        for i in range(S):
            lo = _lo(i, window)
            n = i - lo + 1
            for h in range(Hq):
                acc = 127 * qv[b, lo:i + 1, h // (Hq // Hkv), :].sum(axis=0)
                want = (acc.astype(np.float32) * f(s_v)).astype(np.float32) / f(n * 127)
                assert np.array_equal(O[b, i, h].view(np.uint32), want.astype(np.float32).view(np.uint32)), (b, i, h)


def test_first_row_is_its_own_value():
    """Row 0 sees only key 0: p = 1, l = 1, O = (127 q_v s_v) / 127."""
    Q, K, V = _inputs(1, 9, 4, 1, seed=3)
    s_v = 0.0371
    O = oracle.attn_fwd(Q, K, V, 0, s_v)
    qv = _quantize_v(V, s_v)
    want = ((127 * qv[0, 0, 0]).astype(np.float32) * np.float32(s_v)).astype(np.float32) / np.float32(127)
    for h in range(4):
        assert np.array_equal(O[0, 0, h], want.astype(np.float32))


def _f64_attention(Q, K, V, window, scale):
    B, S, Hq, _ = Q.shape
    Hkv = K.shape[2]
    O = np.zeros(Q.shape, np.float64)
    bound_terms = np.zeros(Q.shape, np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(S):
                lo = _lo(i, window)
                s = K[b, lo:i + 1, hk].astype(np.float64) @ Q[b, i, h].astype(np.float64) * scale
                w = np.exp(s - s.max())
                O[b, i, h] = w @ V[b, lo:i + 1, hk].astype(np.float64) / w.sum()
                bound_terms[b, i, h] = np.abs(V[b, lo:i + 1, hk]).astype(np.float64).sum(axis=0) / w.sum()
    return O, bound_terms


@pytest.mark.parametrize("window", [0, 24])
def test_matches_float64_attention_within_the_quantisation_bound(window):
    """|O - softmax(QK^T/sqrt(D)) V| <= (1/2 + 2^-16 * 127) / 127 * sum|v| / l
    + s_v / 2 + 1e-5: quantising p * 127 moves each weight by at most half a
    step of 1/127 (relative to l >= 1) and quantising v by at most s_v / 2
    (no value here reaches the clamp).  The same data against a softmax
    without the 1/sqrt(D) scale leaves the bound, so the check is sharp
    enough to see a dropped scale."""
    B, S, Hq, Hkv, s_v = 1, 48, 4, 2, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=11, q_scale=0.7)
    assert np.abs(V).max() < 127 * s_v
    O = oracle.attn_fwd(Q, K, V, window, s_v).astype(np.float64)
    ref, terms = _f64_attention(Q, K, V, window, 1.0 / np.sqrt(D))
    bound = (0.5 / 127 + 2.0 ** -16) * terms + s_v / 2 + 1e-5
    assert np.all(np.abs(O - ref) <= bound)
    wrong, _ = _f64_attention(Q, K, V, window, 1.0)
    assert np.any(np.abs(O - wrong) > bound)


def test_causal_window_and_head_groups():
    """Changing key j0 of KV head 1 changes only rows i in [j0, j0 + window)
    of the query heads that read KV head 1 (heads 2, 3 with Hq = 4, Hkv = 2)."""
    B, S, Hq, Hkv, s_v, window = 1, 60, 4, 2, 0.05, 10
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=5)
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    j0 = 30
    K2, V2 = K.copy(), V.copy()
    K2[0, j0, 1] += 0.5
    V2[0, j0, 1] += 1.0
    O2 = oracle.attn_fwd(Q, K2, V2, window, s_v)
    diff = np.any(O2 != O, axis=3)[0]                      # [S, Hq]
    inside = np.zeros((S, Hq), bool)
    inside[j0:j0 + window, 2:4] = True
    assert not np.any(diff & ~inside)
    assert np.all(diff[j0:j0 + window, 2:4])


def test_row_sum_runs_over_the_whole_key_axis():
    """l is CanonSum over all S keys with +0 outside the window (block
    boundaries at absolute key positions), not over the window alone.  Rebuilt
    here from the oracle's binary32 primitives for a few rows, and shown to
    differ from the window-only sum on this data."""
    B, S, Hq, Hkv, s_v, window = 1, 200, 1, 1, 0.05, 77
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=8)
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    qv = _quantize_v(V, s_v)
    c = oracle.div(np.float32(1.0), oracle.sqrt(np.float32(D)))
    differs = 0
    for i in (76, 120, 150, 199):
        lo = _lo(i, window)
        s = np.array([oracle.mul(oracle.canon_sum(np.array([oracle.mul(Q[0, i, 0, d], K[0, j, 0, d]) for d in range(D)],
                                                          np.float32)), c) for j in range(lo, i + 1)], np.float32)
        m = s.max()
        p = np.zeros(S, np.float32)
        p[lo:i + 1] = [oracle.exp(oracle.sub(x, m)) for x in s]
        l_full = oracle.canon_sum(p)
        l_win = oracle.canon_sum(p[lo:i + 1].copy())
        differs += int(l_full != l_win)
        qp = np.array([min(127.0, oracle.rne(oracle.mul(x, np.float32(127.0)))) for x in p[lo:i + 1]]).astype(np.int64)
        acc = qp @ qv[0, lo:i + 1, 0]
        t = oracle.mul(l_full, np.float32(127.0))
        want = np.array([oracle.div(oracle.mul(oracle.i2f(int(a)), np.float32(s_v)), t) for a in acc], np.float32)
        assert np.array_equal(O[0, i, 0], want), i
    assert differs > 0


def test_exp_of_zero_is_one():
    assert oracle.exp(np.float32(0.0)) == np.float32(1.0)
    assert oracle.exp(np.float32(-0.0)) == np.float32(1.0)


def test_sampled_rows_agree_with_the_full_call():
    Q, K, V = _inputs(2, 90, 4, 2, seed=13)
    O = oracle.attn_fwd(Q, K, V, 20, 0.05)
    rows = np.array([0, 5, 77, 2 * 90 * 4 - 1, 90 * 4 + 17])
    got = oracle.attn_fwd_rows(Q, K, V, 20, 0.05, rows)
    assert np.array_equal(got, O.reshape(-1, D)[rows])


# ---- dQ with fixed-point accumulation ----------------------------------------------
def _dequant_v(V, s_v):
    return (_quantize_v(V, s_v).astype(np.float32) * np.float32(s_v)).astype(np.float64)


def _f64_dq(Q, K, Vh, dO, window):
    """Gradient of f(Q) = sum(dO * softmax(Q K^T / sqrt(D)) Vh) in float64,
    with the bound term |K| weighted by P for the error budget."""
    B, S, Hq, _ = Q.shape
    Hkv = K.shape[2]
    c = 1.0 / np.sqrt(D)
    dq = np.zeros(Q.shape)
    wk = np.zeros(Q.shape)
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(S):
                lo = _lo(i, window)
                k = K[b, lo:i + 1, hk].astype(np.float64)
                s = k @ Q[b, i, h].astype(np.float64) * c
                P = np.exp(s - s.max())
                P /= P.sum()
                dp = Vh[b, lo:i + 1, hk] @ dO[b, i, h].astype(np.float64)
                dq[b, i, h] = c * ((P * (dp - P @ dp)) @ k)
                wk[b, i, h] = c * (P @ np.abs(k))
    return dq, wk


def _f64_loss(Q, K, Vh, dO, window):
    B, S, Hq, _ = Q.shape
    Hkv = K.shape[2]
    tot = 0.0
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(S):
                lo = _lo(i, window)
                s = K[b, lo:i + 1, hk].astype(np.float64) @ Q[b, i, h].astype(np.float64) / np.sqrt(D)
                P = np.exp(s - s.max())
                tot += (P / P.sum()) @ Vh[b, lo:i + 1, hk] @ dO[b, i, h].astype(np.float64)
    return tot


def test_dq_zero_output_gradient_gives_zero():
    Q, K, V = _inputs(1, 40, 2, 1, seed=21)
    O = oracle.attn_fwd(Q, K, V, 0, 0.05)
    dq = oracle.attn_bwd_dq(Q, K, V, O, np.zeros_like(O), 0, 0.05)
    assert np.all(dq.view(np.uint32) == 0)


@pytest.mark.parametrize("window", [0, 20])
def test_dq_matches_the_float64_gradient_within_the_quantisation_bound(window):
    """The float64 gradient of sum(dO * softmax(QK^T/sqrt(D)) V^) (itself
    checked by central differences) bounds the oracle's dQ: the only
    departures are the forward's quantised P inside Delta = dO . O (at most
    (1/2 + 2^-16 * 127)/127 of sum|v^|/l per unit of |dO|, times the
    P-weighted |K| c), binary32 rounding (1e-5 relative) and the 2^-40
    fixed-point grid.  The same data with Delta left out leaves the bound."""
    B, S, Hq, Hkv, s_v = 1, 50, 2, 1, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=31, q_scale=0.5)
    g = np.random.default_rng(32)
    dO = (g.standard_normal(Q.shape) * 1e-2).astype(np.float32)
    O = oracle.attn_fwd(Q, K, V, window, s_v)
    dq = oracle.attn_bwd_dq(Q, K, V, O, dO, window, s_v).astype(np.float64)
    Vh = _dequant_v(V, s_v)
    ref, wk = _f64_dq(Q, K, Vh, dO, window)
    # the float64 gradient against central differences of the float64 loss
    for (i, h, d) in [(0, 0, 0), (17, 1, 5), (49, 0, 127)]:
        e = 1e-3
        Qp, Qm = Q.astype(np.float64).copy(), Q.astype(np.float64).copy()
        Qp[0, i, h, d] += e
        Qm[0, i, h, d] -= e
        fd = (_f64_loss(Qp, K, Vh, dO, window) - _f64_loss(Qm, K, Vh, dO, window)) / (2 * e)
        assert abs(fd - ref[0, i, h, d]) <= 1e-6 * max(1.0, abs(fd)) + 1e-9
    _, terms = _f64_attention(Q, K, Vh.astype(np.float32), window, 1.0 / np.sqrt(D))
    delta_err = np.abs(dO).astype(np.float64).sum(axis=3, keepdims=True) * (0.5 / 127 + 2.0 ** -16) \
        * terms.max(axis=3, keepdims=True)
    bound = wk * delta_err + 1e-5 * np.abs(ref) + 1e-7 + S * 2.0 ** -40
    assert np.all(np.abs(dq - ref) <= bound)
    no_delta, _ = _f64_dq(Q, K, Vh, dO, window)
    # planted mistake: without the Delta term the gradient is far off
    planted = np.zeros_like(no_delta)
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                lo = _lo(i, window)
                k = K[b, lo:i + 1, 0].astype(np.float64)
                s = k @ Q[b, i, h].astype(np.float64) / np.sqrt(D)
                P = np.exp(s - s.max())
                P /= P.sum()
                planted[b, i, h] = (P * (Vh[b, lo:i + 1, 0] @ dO[b, i, h].astype(np.float64))) @ k / np.sqrt(D)
    assert np.any(np.abs(dq - planted) > bound)
