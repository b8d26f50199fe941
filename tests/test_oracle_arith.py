"""Pins for the oracle's binary32 primitives, rounding and flush rules.

The numerics rules come from the onedev.kr summary, section "How" (fixed
order, multiply and add never fused, subnormals flushed on every backend).
The primitives are pinned against the host's own IEEE binary32 arithmetic
(numpy float32 on SSE, which rounds correctly and keeps subnormals), with
the flush rule applied on top, and against hand-derived directed cases.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

TINY = np.float32(np.finfo(np.float32).tiny)   # 2^-126


def _flush(x):
    x = np.asarray(x, np.float32)
    return np.where(np.abs(x) < TINY, np.copysign(np.float32(0), x), x).astype(np.float32)


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _rand_pairs(n, seed):
    g = np.random.default_rng(seed)
    a = (g.standard_normal(n) * np.exp(g.uniform(-40, 40, n))).astype(np.float32)
    b = (g.standard_normal(n) * np.exp(g.uniform(-40, 40, n))).astype(np.float32)
    return a, b


@pytest.mark.parametrize("op,npop", [("add", np.add), ("sub", np.subtract),
                                     ("mul", np.multiply), ("div", np.divide)])
def test_primitives_match_ieee_binary32_with_flush(op, npop):
    a, b = _rand_pairs(4000, 7)
    # add subnormal operands to exercise DAZ
    a[:50] = (np.arange(1, 51, dtype=np.uint32) * 99991).view(np.float32)
    b[50:100] = -(np.arange(1, 51, dtype=np.uint32) * 7919).view(np.float32)
    with np.errstate(all="ignore"):
        want = _flush(npop(_flush(a), _flush(b)))
    # host binary32 rounds tiny results at subnormal precision; the two rules
    # can only differ for results within half a 24-bit ulp below 2^-126, which
    # these random operands never produce (checked here)
    with np.errstate(all="ignore"):
        exact = npop(_flush(a).astype(np.float64), _flush(b).astype(np.float64))
    near = (np.abs(exact) < float(TINY)) & (np.abs(exact) > float(TINY) * (1 - 2.0 ** -24))
    assert not near.any()
    fn = getattr(oracle, op)
    got = np.array([fn(x, y) for x, y in zip(a, b)], np.float32)
    same = (_bits(got) == _bits(want)) | (np.isnan(got) & np.isnan(want))
    assert same.all(), f"{op}: first mismatch at {np.argmin(same)}"


def test_sqrt_matches_ieee():
    g = np.random.default_rng(3)
    a = np.abs(g.standard_normal(3000) * np.exp(g.uniform(-80, 80, 3000))).astype(np.float32)
    want = _flush(np.sqrt(_flush(a)))
    got = np.array([oracle.sqrt(x) for x in a], np.float32)
    assert (_bits(got) == _bits(want)).all()


def test_flush_keeps_sign_and_daz():
    sub = np.float32(1e-40)
    assert _bits(oracle.mul(np.float32(1e-20), np.float32(-1e-20))) == _bits(np.float32(-0.0))
    assert _bits(oracle.mul(np.float32(1e-20), np.float32(1e-20))) == 0
    # exact subnormal difference of two normals is flushed
    r = oracle.sub(np.float32(1.5) * TINY, TINY)
    assert _bits(r) == 0
    r = oracle.sub(TINY, np.float32(1.5) * TINY)
    assert _bits(r) == _bits(np.float32(-0.0))
    # denormal operands read as zero of the same sign
    assert _bits(oracle.add(-sub, np.float32(-0.0))) == _bits(np.float32(-0.0))
    assert _bits(oracle.add(sub, np.float32(-0.0))) == 0
    assert oracle.mul(sub, np.float32(3e38)) == 0
    assert oracle.add(sub, np.float32(1.0)) == 1.0


def test_ftz_tininess_after_rounding():
    """Flush is decided on the result rounded to 24 bits with an unbounded
    exponent (IEEE 754 tininess after rounding).  Hand-derived cases:
    (1 - 2^-24) * 2^-126 is exactly representable at 24 bits and below
    2^-126, so it is flushed; 31 * 1082401 = 2^25 - 1, so
    0.96875 * (1082401 * 2^-146) = 2^-126 (1 - 2^-25), which ties to the even
    24-bit value 2^-126 and is kept."""
    assert _bits(oracle.mul(np.float32(1.0 - 2.0 ** -24), TINY)) == 0
    b = np.float32(1082401 * 2.0 ** -146)
    assert oracle.mul(np.float32(0.96875), b) == TINY
    assert _bits(oracle.mul(np.float32(-0.96875), b)) == _bits(-TINY)
    # just above the tie: 2^-126 (1 - 2^-25) is the exact value, so a product
    # one step further below is flushed
    assert oracle.mul(np.float32(0.96875), np.float32(np.nextafter(b, np.float32(0)))) == 0.0


def test_no_fusion():
    """(1+2^-12)^2 - (1+2^-11): unfused gives 0, a fused multiply-add 2^-24."""
    x = np.float32(1 + 2.0 ** -12)
    assert oracle.sub(oracle.mul(x, x), np.float32(1 + 2.0 ** -11)) == 0.0
    exact = Fraction(float(x)) ** 2 - Fraction(1 + 2.0 ** -11)    # what one fused rounding keeps
    assert exact == Fraction(1, 2 ** 24)


def test_rne_table():
    """Integers round half to even, checked against Python's round() on all
    halves k/2 with |k| <= 260 and their float neighbours."""
    for k in range(-260, 261):
        t = np.float32(k / 2)
        for v in (t, np.nextafter(t, np.float32(-1e9)), np.nextafter(t, np.float32(1e9))):
            v = np.float32(v)
            want = float(round(float(v)))
            got = float(oracle.rne(v))
            assert got == want, (v, got, want)
    assert _bits(oracle.rne(np.float32(-0.3))) == _bits(np.float32(-0.0))
    assert oracle.rne(np.float32(2.5)) == 2.0 and oracle.rne(np.float32(3.5)) == 4.0
    assert oracle.rne(np.float32(-2.5)) == -2.0


def test_int_to_float_rne():
    vals = np.array([0, 1, -1, 2**24, 2**24 + 1, 2**24 + 3, -(2**24 + 1), 2**25 + 2,
                     2**31 - 1, -2**31, 90_832_000, 123_456_789], np.int64)
    for v in vals:
        assert oracle.i2f(int(v)) == np.float32(np.int32(v))  # numpy converts with RNE
    assert oracle.i2f(2**24 + 1) == 2.0 ** 24        # tie -> even
    assert oracle.i2f(2**24 + 3) == 2.0 ** 24 + 4
