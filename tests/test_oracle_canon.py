"""Pins for CanonSum: 32-wide sequential blocks, then a fixed pairwise tree.

The order is the one the method fixes for every reduction (onedev.kr summary,
"How": one reduction order on all hardware).  The block width (32) and the
"blocks first, then a pairwise tree" shape are this library's reading of
it.  Pins: exact-sum inputs, hand-derived order-revealing inputs
(tests/golden/canon_sum_cases.json), agreement with an independently written
description of the same tree (split at the largest power of two) evaluated in
host binary32, and sensitivity checks showing that other plausible orders
give other bits on the test data.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ---- independent descriptions of the tree (symbolic) -----------------------
def tree_level_by_level(J):
    nodes = list(range(J))
    while len(nodes) > 1:
        nxt = [(nodes[i], nodes[i + 1]) for i in range(0, len(nodes) - 1, 2)]
        if len(nodes) % 2:
            nxt.append(nodes[-1])
        nodes = nxt
    return nodes[0] if nodes else None


def tree_left_complete(lo, hi):
    """Split [lo, hi) at the largest power of two strictly below its size."""
    n = hi - lo
    if n == 1:
        return lo
    p = 1
    while p * 2 < n:
        p *= 2
    return (tree_left_complete(lo, lo + p), tree_left_complete(lo + p, hi))


def tree_chunked(J, c):
    """Aligned chunks of 2^c leaves reduced first, then the chunk roots."""
    size = 1 << c
    roots = []
    for lo in range(0, J, size):
        sub = tree_level_by_level(min(size, J - lo))
        roots.append(_shift(sub, lo))
    return _subst(tree_level_by_level(len(roots)), roots)


def _shift(t, d):
    return t + d if isinstance(t, int) else (_shift(t[0], d), _shift(t[1], d))


def _subst(t, leaves):
    return leaves[t] if isinstance(t, int) else (_subst(t[0], leaves), _subst(t[1], leaves))


def tree_midpoint(lo, hi):
    n = hi - lo
    if n == 1:
        return lo
    mid = lo + (n + 1) // 2
    return (tree_midpoint(lo, mid), tree_midpoint(mid, hi))


def eval_tree(t, b):
    if isinstance(t, int):
        return b[t]
    return np.float32(eval_tree(t[0], b) + eval_tree(t[1], b))


def test_tree_descriptions_agree():
    """Level-by-level with odd carry == left-complete split, for all J < 1200;
    and any aligned 2^c chunking gives the same tree (so a kernel may split
    the reduction at aligned power-of-two subtree boundaries)."""
    for J in range(1, 1200):
        t = tree_level_by_level(J)
        assert t == tree_left_complete(0, J), J
        for c in (1, 2, 3, 5):
            assert tree_chunked(J, c) == t, (J, c)


def test_block_sum_is_sequential_from_first_term():
    case = json.load(open(os.path.join(GOLDEN, "canon_sum_cases.json")))
    for c in case["cases"]:
        p = np.array([float.fromhex(v) if isinstance(v, str) else v for v in c["input"]], np.float32)
        want = np.float32(float.fromhex(c["expect"]) if isinstance(c["expect"], str) else c["expect"])
        got = oracle.canon_sum(p)
        assert _bits(got) == _bits(want), (c["name"], got, want)


def _block_sums(p, width=32):
    b = []
    for j in range(0, len(p), width):
        s = p[j]
        for x in p[j + 1: j + width]:
            s = np.float32(s + x)
        b.append(s)
    return b


def test_golden_alternatives_differ():
    """Cases that list the values of other orders must be separated by them:
    the midpoint split and the plain sequential sum are recomputed here in
    host binary32 and give the stated, different bits."""
    case = json.load(open(os.path.join(GOLDEN, "canon_sum_cases.json")))
    checked = 0
    for c in case["cases"]:
        alt = c.get("alternatives")
        if not alt:
            continue
        p = np.array(c["input"], np.float32)
        want = np.float32(c["expect"])
        b = _block_sums(p)
        got = {"midpoint": eval_tree(tree_midpoint(0, len(b)), b)}
        seq = p[0]
        for x in p[1:]:
            seq = np.float32(seq + x)
        got["sequential"] = seq
        for name, v in alt.items():
            assert _bits(got[name]) == _bits(np.float32(v)), (c["name"], name, got[name])
            assert _bits(got[name]) != _bits(want), (c["name"], name)
            checked += 1
    assert checked >= 1


def test_exact_sums():
    g = np.random.default_rng(0)
    for n in (1, 5, 31, 32, 33, 64, 95, 96, 97, 1000, 3000):
        p = g.integers(-1000, 1000, n).astype(np.float32) * np.float32(0.25)
        assert oracle.canon_sum(p) == np.float32(p.astype(np.float64).sum())
    assert _bits(oracle.canon_sum(np.zeros(0, np.float32))) == 0


def test_first_term_sign_of_zero():
    """Sums start from the first term, not from +0: all -0 terms give -0."""
    p = np.full(70, -0.0, np.float32)
    assert _bits(oracle.canon_sum(p)) == _bits(np.float32(-0.0))


@pytest.mark.parametrize("n", [33, 96, 97, 352 * 32, 1000, 3 * 2**10 * 32 + 7])
def test_matches_left_complete_description_in_host_binary32(n):
    g = np.random.default_rng(n)
    p = (g.standard_normal(n) * np.exp(g.uniform(-8, 8, n))).astype(np.float32)
    J = (n + 31) // 32
    b = []
    for j in range(J):
        blk = p[32 * j: 32 * j + 32]
        s = blk[0]
        for x in blk[1:]:
            s = np.float32(s + x)
        b.append(s)
    want = eval_tree(tree_left_complete(0, J), b) if J > 1 else b[0]
    assert _bits(oracle.canon_sum(p)) == _bits(want)


def test_order_sensitivity():
    """On Gaussian data with 96 blocks the canonical tree, a midpoint split
    and a plain sequential sum disagree in most trials, so the pins above
    would catch a wrong order."""
    diff_mid = diff_seq = 0
    trials = 40
    for seed in range(trials):
        g = np.random.default_rng(1000 + seed)
        p = g.standard_normal(96 * 32).astype(np.float32)
        b = []
        for j in range(96):
            s = p[32 * j]
            for x in p[32 * j + 1: 32 * j + 32]:
                s = np.float32(s + x)
            b.append(s)
        want = oracle.canon_sum(p)
        diff_mid += _bits(eval_tree(tree_midpoint(0, 96), b)) != _bits(want)
        seq = p[0]
        for x in p[1:]:
            seq = np.float32(seq + x)
        diff_seq += _bits(seq) != _bits(want)
    assert diff_mid > trials // 2 and diff_seq > trials // 2, (diff_mid, diff_seq)


def test_pair_tree_odd_carry():
    # J = 3: (b0 + b1) + b2 ;  with b = [2^24, 1, 1] -> 2^24 (ties to even twice)
    assert oracle.pair_tree([2.0**24, 1.0, 1.0]) == 2.0**24
    # J = 3 reversed association would give 2^24 + 2
    assert np.float32(np.float32(2.0**24) + np.float32(2.0)) == 2.0**24 + 2
    # J = 5: ((b0+b1)+(b2+b3)) + b4
    assert oracle.pair_tree([1.0, 2.0**24, -2.0**24, 1.0, 1.0]) == 2.0
