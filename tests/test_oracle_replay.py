"""Pins for the oracle's audit replay of the gradient reduction and the global
norm clip.

Method: onedev.kr summary of Open-1B, "Limits", audit paragraph (running-sum
reduce-scatter over virtual ranks in mesh order, replica-major and
shard-minor, one partial resident at a time; TreeFold in the pairing order of
the cluster's recursive-doubling all-reduce) and recipe paragraph (global L2
gradient-norm clipping at 1.0).  For six replicas the fold of ranks 4 and 5
into 0 and 1 before recursive doubling is the plain reading of recursive
doubling on a non-power-of-two group.
"""
import itertools

import numpy as np
import pytest

import oracle


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _vecs(R, L, seed):
    g = np.random.default_rng(seed)
    # mixed magnitudes so that different pairings round differently
    return [(g.standard_normal(L) * np.exp(g.uniform(-6, 6, L))).astype(np.float32) for _ in range(R)]


def _all_trees(leaves):
    """Every full binary tree (unordered children) over the given leaves."""
    leaves = tuple(leaves)
    if len(leaves) == 1:
        yield leaves[0]
        return
    first, rest = leaves[0], leaves[1:]
    # split into two non-empty groups; the group holding `first` is the left
    for r in range(0, len(rest)):
        for comb in itertools.combinations(rest, r):
            left = (first,) + comb
            right = tuple(x for x in rest if x not in comb)
            if not right:
                continue
            for lt in _all_trees(left):
                for rt in _all_trees(right):
                    yield (lt, rt)


def _eval(t, A):
    if isinstance(t, int):
        return A[t]
    return (_eval(t[0], A) + _eval(t[1], A)).astype(np.float32)


def _canon(t):
    if isinstance(t, int):
        return t
    a, b = _canon(t[0]), _canon(t[1])
    return tuple(sorted((a, b), key=repr))


def test_treefold_six_replicas_is_unique_pairing():
    """Of the 945 pairing trees over 6 replicas exactly one reproduces the
    oracle's TreeFold on the test data, and it is ((A0+A4)+(A1+A5))+(A2+A3)."""
    A = _vecs(6, 4096, 1)
    T = oracle.treefold(A)
    trees = list(_all_trees(range(6)))
    assert len(trees) == 945
    matches = [t for t in trees if (_bits(_eval(t, A)) == _bits(T)).all()]
    assert len(matches) == 1
    assert _canon(matches[0]) == _canon((((0, 4), (1, 5)), (2, 3)))


@pytest.mark.parametrize("R", list(range(1, 17)))
def test_treefold_fold_then_pairwise(R):
    """Recursive doubling with the extra ranks folded first equals: leaves
    L_i = A_i + A_{i+p} (i < R-p) or A_i, then the pairwise tree
    ((L0+L1)+(L2+L3))+... over the p leaves."""
    A = _vecs(R, 512, 100 + R)
    p = 1
    while p * 2 <= R:
        p *= 2
    Lv = [(A[i] + A[i + p]).astype(np.float32) if i + p < R else A[i] for i in range(p)]
    while len(Lv) > 1:
        Lv = [(Lv[2 * i] + Lv[2 * i + 1]).astype(np.float32) for i in range(len(Lv) // 2)]
    assert (_bits(oracle.treefold(A)) == _bits(Lv[0])).all()


def test_running_sum_in_mesh_order():
    """A_r = ((G_{rS} + G_{rS+1}) + ...) + G_{rS+S-1}; reversing the shard
    order changes bits on the test data."""
    R, S, L = 2, 8, 2048
    G = _vecs(R * S, L, 7)
    T, nu, A = oracle.replay(G, R, S, max_norm=1e30)
    for r in range(R):
        acc = G[r * S].copy()
        for s in range(1, S):
            acc = (acc + G[r * S + s]).astype(np.float32)
        assert (_bits(A[r]) == _bits(acc)).all()
        rev = G[r * S + S - 1].copy()
        for s in range(S - 2, -1, -1):
            rev = (rev + G[r * S + s]).astype(np.float32)
        assert (_bits(rev) != _bits(acc)).any()
    assert (_bits(T) == _bits((A[0] + A[1]).astype(np.float32))).all()


def test_norm_closed_form():
    """g_i = +-2^-k: squares and sums exact; n = 4096 gives nu = 64 * 2^-k."""
    g = np.random.default_rng(0)
    for k in (0, 3, 10, 20):
        T = np.where(g.random(4096) < 0.5, -1.0, 1.0).astype(np.float32) * np.float32(2.0 ** -k)
        assert oracle.l2norm(T) == np.float32(64 * 2.0 ** -k)
    assert oracle.l2norm(np.zeros(0, np.float32)) == 0.0


def test_norm_error_bound():
    g = np.random.default_rng(1)
    T = (g.standard_normal(100_003) * 1e-3).astype(np.float32)
    exact = np.sqrt(np.sum(T.astype(np.float64) ** 2))
    J = (T.size + 31) // 32
    h = 32 + int(np.ceil(np.log2(J)))
    u = 2.0 ** -24
    assert abs(float(oracle.l2norm(T)) - exact) <= (h * u + 2 * u) * exact


def test_clip():
    g = np.random.default_rng(2)
    T = g.standard_normal(1000).astype(np.float32)
    nu = oracle.l2norm(T)
    assert nu > 1.0
    T2 = T.copy()
    kappa = oracle.clip(T2, nu, 1.0, 0.0)
    assert kappa == np.float32(np.float32(1.0) / nu)
    assert (_bits(T2) == _bits(T * kappa)).all()
    # no clip when the norm is within the bound
    T3 = (T / np.float32(100)).astype(np.float32)
    T4 = T3.copy()
    assert oracle.clip(T4, oracle.l2norm(T3), 1.0, 0.0) == 1.0
    assert (_bits(T4) == _bits(T3)).all()
    # nu exactly at the bound: no clip
    T5 = np.zeros(16, np.float32)
    T5[0] = 1.0
    assert oracle.l2norm(T5) == 1.0 and oracle.clip(T5.copy(), 1.0, 1.0, 0.0) == 1.0


def test_replay_flushes_subnormal_sums():
    """A running sum whose exact value is subnormal is flushed, sign kept."""
    tiny = np.float32(np.finfo(np.float32).tiny)
    G = [np.array([1.5 * tiny, -tiny], np.float32), np.array([-tiny, 1.5 * tiny], np.float32)]
    T, nu, A = oracle.replay(G, 1, 2)
    assert _bits(A[0][0]) == 0 and _bits(A[0][1]) == 0
    G = [np.array([tiny], np.float32), np.array([-1.5 * tiny], np.float32)]
    _, _, A = oracle.replay(G, 1, 2)
    assert _bits(A[0][0]) == _bits(np.float32(-0.0))
