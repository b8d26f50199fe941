"""A seeded sweep of the attention kernels over random shapes against the
oracle, every output bit for bit: batch 1-2, sequence 1-320, 1-4 KV heads
with 1-4 query heads per KV head, causal or a window of 1 to beyond the
sequence, the value step drawn from [0.01, 0.1], query scales from 0.05 to 3
(sharp and flat softmax rows); the forward (O and its statistics), dQ, and
dK/dV formed again or read from the forward's kept logits.  The draws are
fixed (seed 77): the same cases run every time."""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import oracle

pytestmark = pytest.mark.gpu

D = 128


def _cases(n=16, seed=77):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(g.integers(1, 321))
        hkv = int(g.integers(1, 5))
        window = 0 if i % 3 == 0 else int(g.integers(1, S + 80))
        out.append(dict(i=i, B=int(g.integers(1, 3)), S=S, Hkv=hkv, Hq=hkv * int(g.integers(1, 5)),
                        window=window, s_v=float(np.float32(g.uniform(0.01, 0.1))),
                        scale=float(np.exp(g.uniform(np.log(0.05), np.log(3.0)))), keep=i % 2 == 1))
    return out


def _bits(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def _same(got, want, what, c):
    g, w = _bits(got), _bits(want)
    assert g.shape == w.shape, (what, c)
    bad = np.flatnonzero(g.ravel() != w.ravel())
    assert bad.size == 0, f"{what}: {bad.size} of {g.size} differ, case {c}"


@pytest.mark.parametrize("c", _cases(), ids=lambda c: f"case{c['i']}")
def test_attention_random_shape(c):
    print(f"case {c}", flush=True)
    B, S, Hq, Hkv, window, s_v = c["B"], c["S"], c["Hq"], c["Hkv"], c["window"], c["s_v"]
    g = np.random.default_rng(1000 + c["i"])
    Q = (g.standard_normal((B, S, Hq, D)) * c["scale"]).astype(np.float32)
    K = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    V = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    dO = (g.standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    q, k, v, go = (torch.from_numpy(t).cuda() for t in (Q, K, V, dO))
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    logits = brl.attn_logits_buffer(B, S, Hq, window) if c["keep"] else None
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats, logits=logits)
    dQ = brl.attn_bwd_dq(q, k, v, O, go, stats, window, s_v, logits=logits)
    dK, dV = brl.attn_bwd_dkdv(q, k, v, O, go, stats, window, s_v, logits=logits)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy()
    _same(Oh, oracle.attn_fwd(Q, K, V, window, s_v), "O", c)
    _same(dQ, oracle.attn_bwd_dq(Q, K, V, Oh, dO, window, s_v), "dQ", c)
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, Oh, dO, window, s_v)
    _same(dK, wk, "dK", c)
    _same(dV, wv, "dV", c)
