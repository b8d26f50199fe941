"""Skipping keys when a row's exact maximum is formed from approximate
logits: a record of why such a rule must bound from both sides.

The attention forward (attn_fwd; onedev.kr summary of Open-1B, "Use",
attention paragraph: logits and softmax in high precision) needs the exact
maximum m_i of the canonical binary32 logits of each row.  It now computes
every logit exactly once and keeps them in its workspace, so it skips no
key.  An earlier version first formed approximate logits a_ij from bf16
operands on the matrix cores, each within E_ij = c * 0.0158 * |q_i| |k_j| +
2^-80 of the exact logit s_ij, and computed exact logits only for keys that
could still hold the maximum.

This file emulates that approximation on the host (bf16 round-to-nearest-
even of the operands, fp32 sums in several orders, the bound) and checks
the sound rule (keep key j unless a_ij + E_ij < L_i, with L_i the largest
a_il - E_il over the row's keys).  It also shows that the first rule, which
dropped j when a_ij < A_i - 2 E_ij with A_i the largest approximate logit,
loses the true maximum on a constructed row whose keys differ in norm.  The
GPU tests run the same witness through the kernels.
"""
import numpy as np

f32 = np.float32
D = 128
C = f32(f32(1.0) / np.sqrt(f32(D)))
EBOUND = float(C) * 0.0158


def bf16(x):
    """Round binary32 values to bfloat16 (nearest, ties to even), as binary32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def exact_logit(q, k):
    """s = CanonSum_d(q_d * k_d) * c in binary32: four 32-term blocks left to
    right, then (b0 + b1) + (b2 + b3)."""
    prod = (q.astype(np.float32) * k.astype(np.float32)).astype(np.float32)
    b = []
    for blk in range(4):
        s = prod[32 * blk]
        for x in prod[32 * blk + 1: 32 * blk + 32]:
            s = f32(s + x)
        b.append(s)
    return f32(f32(f32(b[0] + b[1]) + f32(b[2] + b[3])) * C)


def approx_logits(q, k):
    """a = fl32(sum of bf16 products) * c, with the fp32 sum taken in three
    different orders (the matrix cores' order is not specified)."""
    p = (bf16(q).astype(np.float64) * bf16(k).astype(np.float64)).astype(np.float32)
    out = []
    for order in (np.arange(D), np.arange(D)[::-1], np.argsort(np.abs(p))):
        s = f32(0.0)
        for i in order:
            s = f32(s + p[i])
        out.append(f32(s * C))
    out.append(f32(f32(p.astype(np.float64).sum()) * C))
    return out


def bound(q, k):
    nq = np.sqrt((q.astype(np.float64) ** 2).sum()) * (1 + 2 ** -30)
    nk = np.sqrt((k.astype(np.float64) ** 2).sum()) * (1 + 2 ** -30)
    return EBOUND * nq * nk + 2.0 ** -80


def kept_sound(a, e):
    L = max(float(ai) - ei for ai, ei in zip(a, e))
    return [not (float(ai) + ei < L) for ai, ei in zip(a, e)]


def kept_earlier_rule(a, e):
    A = max(float(ai) for ai in a)
    return [float(ai) >= A - 2 * ei for ai, ei in zip(a, e)]


def witness():
    """q all ones; key l alternates +64(1+2^-8+2^-16) and -64(1+2^-8-2^-16):
    its bf16 operands are 64(1+2^-7) and -64, so a_l = 32 c = 2.83 while the
    exact logit is 64 * 2^-9 * c = 0.011, and E_l = 11.4.  Key j is 0.125
    everywhere: a_j = s_j = 16 c = 1.414 (the true row maximum), E_j =
    0.022."""
    q = np.ones(D, np.float32)
    hi = f32(64.0 * (1 + 2.0 ** -8 + 2.0 ** -16))
    lo = f32(-64.0 * (1 + 2.0 ** -8 - 2.0 ** -16))
    kl = np.where(np.arange(D) % 2 == 0, hi, lo).astype(np.float32)
    kj = np.full(D, 0.125, np.float32)
    return q, [kl, kj]


def test_bounds_hold_on_the_witness():
    q, keys = witness()
    for k in keys:
        s = exact_logit(q, k)
        for a in approx_logits(q, k):
            assert abs(float(a) - float(s)) <= bound(q, k)
    s = [exact_logit(q, k) for k in keys]
    assert s[1] > s[0] and abs(float(s[1]) - 1.4142135) < 1e-6 and abs(float(s[0]) - 0.011048543) < 1e-7


def test_earlier_rule_drops_the_maximum_and_the_sound_rule_keeps_it():
    q, keys = witness()
    a = [approx_logits(q, k)[0] for k in keys]
    e = [bound(q, k) for k in keys]
    assert abs(float(a[0]) - 2.8284271) < 1e-6 and abs(e[0] - 11.44) < 0.05
    # the earlier rule: 1.414 < 2.83 - 2 * 0.022, so key j (the maximum) is dropped
    assert kept_earlier_rule(a, e) == [True, False]
    # the rule the kernel uses keeps both: L = 1.414 - 0.022, and 1.414 + 0.022 >= L
    assert kept_sound(a, e) == [True, True]


def test_sound_rule_keeps_the_maximum_for_spread_key_norms():
    """Random rows of 64 keys whose norms spread over 1e-2 .. 1e2 within the
    row, queries of several scales: the exact maximum is always kept, for
    every order of the approximate sums."""
    g = np.random.default_rng(7)
    for trial in range(60):
        q = (g.standard_normal(D) * 10.0 ** g.uniform(-1, 1)).astype(np.float32)
        K = g.standard_normal((64, D)) * (10.0 ** g.uniform(-2, 2, 64))[:, None]
        if trial % 3 == 0:            # near-ties of the exact logits
            K[5] = K[9] * (1 + 1e-7)
        K = K.astype(np.float32)
        s = np.array([exact_logit(q, k) for k in K], np.float32)
        jmax = int(np.argmax(s))
        e = [bound(q, k) for k in K]
        for v in range(4):
            a = [approx_logits(q, k)[v] for k in K]
            keep = kept_sound(a, e)
            assert keep[jmax], (trial, v)
            # every key whose exact logit equals the maximum is kept
            for j in np.nonzero(s == s[jmax])[0]:
                assert keep[j], (trial, v, j)
