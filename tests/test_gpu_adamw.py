"""GPU parity of adamw_step against the oracle's or_adamw: p, m and v bit for
bit, with and without decay, at warm-up / cosine / end-of-budget scalars,
ragged sizes (the scalar tail), 4-byte-aligned arrays, and inputs with
zeros, signed zeros and subnormals."""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import oracle

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _inputs(n, seed):
    g_ = np.random.default_rng(seed)
    p = g_.standard_normal(n).astype(np.float32)
    g = (g_.standard_normal(n) * 1e-2).astype(np.float32)
    m = (g_.standard_normal(n) * 1e-3).astype(np.float32)
    v = (np.abs(g_.standard_normal(n)) * 1e-5).astype(np.float32)
    if n >= 16:
        g[:4] = [0.0, -0.0, 1e-40, -1e-40]
        m[4:8] = [0.0, -0.0, 1e-39, 0.0]
        v[8:12] = [0.0, 0.0, 1e-41, 3e-39]
        p[12:16] = [0.0, -0.0, 1e-40, 1e30]
    return p, g, m, v


@pytest.mark.parametrize("decay", [True, False])
@pytest.mark.parametrize("n,step,tokens", [(1, 1, 1e6), (3, 2, 1e9), (4099, 667, 2.1e9), (1 << 20, 5000, 1e11),
                                           ((1 << 20) + 3, 120000, 4.5e11), (0, 1, 0.0)])
def test_adamw_parity(n, step, tokens, decay):
    p, g, m, v = _inputs(n, n + step)
    sc = brl.adamw_scalars_for_step(step, tokens)
    P, G, M, V = (torch.from_numpy(x.copy()).cuda() for x in (p, g, m, v))
    brl.adamw_step(P, G, M, V, sc, decay=decay)
    torch.cuda.synchronize()
    wp, wm, wv = p.copy(), m.copy(), v.copy()
    oracle.adamw(wp, g, wm, wv, sc.as_dict(), decay)
    assert np.array_equal(_bits(P.cpu().numpy()), _bits(wp)), "p"
    assert np.array_equal(_bits(M.cpu().numpy()), _bits(wm)), "m"
    assert np.array_equal(_bits(V.cpu().numpy()), _bits(wv)), "v"


def test_adamw_four_byte_aligned_arrays():
    n = 10001
    p, g, m, v = _inputs(n, 5)
    sc = brl.adamw_scalars_for_step(9, 5e9)
    bufs = []
    for x in (p, g, m, v):
        t = torch.empty(n + 1, dtype=torch.float32, device="cuda")
        t[1:] = torch.from_numpy(x)
        bufs.append(t[1:])
    assert bufs[0].data_ptr() % 16 != 0
    brl.adamw_step(*bufs, sc)
    torch.cuda.synchronize()
    wp, wm, wv = p.copy(), m.copy(), v.copy()
    oracle.adamw(wp, g, wm, wv, sc.as_dict(), True)
    assert np.array_equal(_bits(bufs[0].cpu().numpy()), _bits(wp))
    assert np.array_equal(_bits(bufs[2].cpu().numpy()), _bits(wm))
    assert np.array_equal(_bits(bufs[3].cpu().numpy()), _bits(wv))


def test_adamw_steps_in_sequence():
    """Ten consecutive steps (moments carried on the device) stay bit-identical."""
    n = 50000
    p, g, m, v = _inputs(n, 77)
    P, M, V = (torch.from_numpy(x.copy()).cuda() for x in (p, m, v))
    rng = np.random.default_rng(78)
    for t in range(1, 11):
        gt = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        sc = brl.adamw_scalars_for_step(t, t * 4.7e6)
        brl.adamw_step(P, torch.from_numpy(gt).cuda(), M, V, sc)
        oracle.adamw(p, gt, m, v, sc.as_dict(), True)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(P.cpu().numpy()), _bits(p))
    assert np.array_equal(_bits(M.cpu().numpy()), _bits(m))
    assert np.array_equal(_bits(V.cpu().numpy()), _bits(v))
