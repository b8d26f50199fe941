"""The kernels' fast form of the LSQ quantiser, emulated on the host.

The quantiser's code is q = clamp(rne(T), -127, 127) and its straight-
through mask in = (-127 <= T <= 127), with T = fl32(v / s) the correctly
rounded binary32 quotient (onedev.kr summary of Open-1B, "Use": 8-bit
weights and activations; the quotient reading is the library's).  The
kernels first form t = fl32(v * fl32(1 / s)) and trust rne(t) unless t lies
within 2^-15 of a rounding midpoint k + 1/2 (for the mask: of +-127); the
unsure values are redone exactly.  This file checks that rule in host
binary32 arithmetic against the exact quotient, on steps of several sizes
and on values placed at and next to every midpoint and the range ends, so
the rule's error bound is tested on the inputs where it matters.
"""
from fractions import Fraction

import numpy as np

f32 = np.float32


def exact_T(v, s):
    return f32(float(Fraction(float(v)) / Fraction(float(s))))   # binary64 of the exact quotient, then binary32


def code(t):
    r = np.rint(np.float32(t))
    return int(min(127.0, max(-127.0, r)))


def fast(v, s):
    t = f32(f32(v) * f32(f32(1.0) / f32(s)))
    r = np.rint(t)
    unsure_q = abs(float(t) - float(r)) > 0.5 - 2.0 ** -15
    unsure_m = abs(abs(float(t)) - 127.0) < 2.0 ** -15
    return t, unsure_q, unsure_m


def boundary_values(s, g, n_random=4000):
    """Values whose quotients lie at and a few ulp around every midpoint
    k + 1/2 and around +-127 and +-127.5, plus random ones."""
    vals = []
    targets = [k + 0.5 for k in range(-128, 128)] + [-127.0, 127.0, -127.5, 127.5]
    for q in targets:
        v0 = f32(q * float(s))
        for k in range(-6, 7):
            vk = v0
            for _ in range(abs(k)):
                vk = np.nextafter(vk, f32(np.inf) if k > 0 else f32(-np.inf), dtype=np.float32)
            vals.append(vk)
    vals += list((g.standard_normal(n_random) * 60 * float(s)).astype(np.float32))
    vals += list((g.standard_normal(200) * 400 * float(s)).astype(np.float32))
    return np.array(vals, np.float32)


def test_fast_path_agrees_with_the_exact_quotient_whenever_it_is_sure():
    g = np.random.default_rng(1)
    steps = [f32(0.05), f32(0.0371), f32(1.0 / 3.0), f32(2.5e-3), f32(2.0 ** -6), f32(0.0158447),
             f32(7.3e-4), f32(12.5)]
    unsure_seen = sure_seen = 0
    for s in steps:
        for v in boundary_values(s, g):
            T = exact_T(v, s)
            t, uq, um = fast(v, s)
            if not uq:
                assert code(t) == code(T), (float(v), float(s), float(t), float(T))
                sure_seen += 1
            else:
                unsure_seen += 1
            if not um:
                assert (abs(float(t)) <= 127.0) == (abs(float(T)) <= 127.0), (float(v), float(s))
    # the set reaches both outcomes of the rule
    assert unsure_seen > 1000 and sure_seen > 10000, (unsure_seen, sure_seen)


def test_rule_is_needed():
    """Without the fallback the fast quotient would give other codes on this
    set: the exact path is not dead code."""
    g = np.random.default_rng(2)
    s = f32(0.05)
    diff = sum(code(fast(v, s)[0]) != code(exact_T(v, s)) for v in boundary_values(s, g, 0))
    assert diff > 0
