"""The audit property on the oracle (CPU): a replayed step -- the 6x8
ordered reduction, norm, clip, AdamW update -- reproduces its state hash bit
for bit, and each of the deviations the method rules out changes the hash:
a corrupted partial, a wrong mesh order, a wrong TreeFold pairing, a fused
multiply-add in the optimizer (onedev.kr summary, sections "How" and "Limits",
audit paragraph; the state hash is this library's reading, a tree of SHA-256 digests)."""
import numpy as np

import oracle
import synth
from oracle import state_hash as sh

R, S, L = 6, 8, 4099


def _partials():
    return [synth.replay_partial_host(11, v, L, std=1e-2) for v in range(R * S)]


def _step(parts, fold=None, norm=None, adam=None):
    A = [np.empty(L, np.float32) for _ in range(R)]
    for v in range(R * S):
        r, s = divmod(v, S)
        oracle.replay_accumulate(A[r], parts[v], first=(s == 0))
    T = oracle.treefold(A) if fold is None else fold(A)
    nu = oracle.l2norm(T) if norm is None else norm(T)
    oracle.clip(T, nu, 1.0, 0.0)
    # a later step (moments already set), so the update depends on the gradient's scale
    p = np.linspace(-1, 1, L).astype(np.float32)
    m = np.full(L, 1e-3, np.float32)
    v = np.full(L, 1e-5, np.float32)
    (oracle.adamw if adam is None else adam)(p, T, m, v, oracle.adamw_scalars(5, 2.4e7), True)
    return sh.state_hash([p, m, v])


def _add(a, b):
    return np.array([oracle.add(x, y) for x, y in zip(a, b)], np.float32)


def test_replay_reproduces_its_hash():
    parts = _partials()
    assert _step(parts) == _step([p.copy() for p in parts])


def test_corrupted_partial_changes_the_hash():
    parts = _partials()
    h = _step(parts)
    bad = [p.copy() for p in parts]
    bad[13][100] = np.float32(bad[13][100] * 2.0)
    assert _step(bad) != h


def test_wrong_mesh_order_changes_the_hash():
    parts = _partials()
    h = _step(parts)
    swapped = list(parts)
    swapped[2], swapped[3] = swapped[3], swapped[2]     # shards 2 and 3 of replica 0
    assert _step(swapped) != h


def test_wrong_fold_pairing_changes_the_hash():
    parts = _partials()
    h = _step(parts)

    def sequential_pairs(A):     # ((A0+A1)+(A2+A3))+(A4+A5): not recursive doubling
        return _add(_add(_add(A[0], A[1]), _add(A[2], A[3])), _add(A[4], A[5]))

    assert _step(parts, fold=sequential_pairs) != h


def test_fused_multiply_add_changes_the_hash():
    parts = _partials()
    h = _step(parts)

    def adamw_fused_first_moment(p, g, m, v, sc, decay):
        # the stored first moment beta1*m + fl(c1*g) with the product and the add
        # fused (one rounding; exact binary64 product, binary64 add, one narrowing)
        c1g = (np.float64(sc["c1"]) * g.astype(np.float64)).astype(np.float32)
        m_fused = (np.float64(sc["beta1"]) * m.astype(np.float64) + c1g.astype(np.float64)).astype(np.float32)
        oracle.adamw(p, g, m, v, sc, decay)
        assert not np.array_equal(m_fused.view(np.uint32), m.view(np.uint32))
        m[:] = m_fused

    assert _step(parts, adam=adamw_fused_first_moment) != h
