"""GPU parity of attn_fwd (int8 P.V attention) against the CPU oracle, bit
for bit: ragged sequence lengths, sliding windows shorter and longer than the
query block, full causal attention, grouped-query head counts, column slices
of a QKV projection output as Q/K/V, and a row-stride-only O view."""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import oracle

pytestmark = pytest.mark.gpu

D = 128


def _bits(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def assert_bitwise(got, want, what):
    g, w = _bits(got), _bits(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.flatnonzero(g.ravel() != w.ravel())
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at flat {i} "
                             f"(index {np.unravel_index(i, g.shape)}): got {g.ravel()[i]:#010x} "
                             f"want {w.ravel()[i]:#010x}")


def _inputs(B, S, Hq, Hkv, seed, scale=1.0):
    g = np.random.default_rng(seed)
    Q = (g.standard_normal((B, S, Hq, D)) * scale).astype(np.float32)
    K = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    V = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    return Q, K, V


CASES = [
    # B, S, Hq, Hkv, window, s_v
    (1, 1, 1, 1, 0, 0.05),
    (1, 64, 2, 1, 0, 0.05),
    (2, 200, 4, 2, 0, 0.05),
    (2, 200, 4, 2, 64, 0.05),
    (1, 130, 8, 1, 37, 0.0371),
    (1, 150, 4, 4, 1, 0.05),
    (1, 100, 4, 2, 500, 0.05),        # window longer than the sequence
    (1, 333, 16, 4, 130, 0.05),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,window,s_v", CASES)
def test_attention_parity(B, S, Hq, Hkv, window, s_v):
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=S + 7 * Hq + window, scale=0.3)
    O = brl.attn_fwd(torch.from_numpy(Q).cuda(), torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(),
                     window, s_v)
    torch.cuda.synchronize()
    assert_bitwise(O, oracle.attn_fwd(Q, K, V, window, s_v), f"O (B={B} S={S} Hq={Hq} Hkv={Hkv} w={window})")


def test_attention_on_qkv_projection_slices():
    """Q, K, V as column slices of one [B*S, (Hq + 2 Hkv) * D] buffer (the
    QKV projection's output), O written into a wider buffer."""
    B, S, Hq, Hkv, window, s_v = 2, 190, 4, 1, 96, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=3, scale=0.3)
    Y = np.concatenate([Q.reshape(B * S, -1), K.reshape(B * S, -1), V.reshape(B * S, -1)], axis=1)
    Yd = torch.from_numpy(np.ascontiguousarray(Y)).cuda()
    q = Yd[:, :Hq * D].view(B, S, Hq, D)
    k = Yd[:, Hq * D:(Hq + Hkv) * D].view(B, S, Hkv, D)
    v = Yd[:, (Hq + Hkv) * D:].view(B, S, Hkv, D)
    wide = torch.full((B * S, Hq * D + 64), 7.0, device="cuda")
    O = wide[:, :Hq * D].view(B, S, Hq, D)
    brl.attn_fwd(q, k, v, window, s_v, O=O)
    torch.cuda.synchronize()
    assert_bitwise(O, oracle.attn_fwd(Q, K, V, window, s_v), "O (QKV slices)")
    assert torch.all(wide[:, Hq * D:] == 7.0)


def test_attention_large_logits_and_repeat():
    """Logits spread over tens of units (most p underflow to small values or
    +0) and two calls give the same bits."""
    B, S, Hq, Hkv, window, s_v = 1, 257, 4, 2, 0, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=9, scale=2.0)
    args = [torch.from_numpy(t).cuda() for t in (Q, K, V)]
    O1 = brl.attn_fwd(*args, window, s_v)
    O2 = brl.attn_fwd(*args, window, s_v)
    torch.cuda.synchronize()
    want = oracle.attn_fwd(Q, K, V, window, s_v)
    assert_bitwise(O1, want, "O (large logits)")
    assert_bitwise(O2, want, "O (repeat)")


DQ_CASES = [
    # B, S, Hq, Hkv, window, s_v
    (1, 1, 1, 1, 0, 0.05),
    (1, 64, 2, 1, 0, 0.05),
    (2, 150, 4, 2, 0, 0.05),
    (1, 200, 4, 2, 64, 0.0371),
    (1, 333, 16, 4, 130, 0.05),
    (1, 100, 4, 4, 1, 0.05),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,window,s_v", DQ_CASES)
def test_attention_dq_parity(B, S, Hq, Hkv, window, s_v):
    """dQ with 64-bit fixed-point accumulation, bit for bit, from the
    forward's own O and (m, l) statistics."""
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=3 * S + Hq + window, scale=0.3)
    dO = (np.random.default_rng(S + window).standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    q, k, v = (torch.from_numpy(t).cuda() for t in (Q, K, V))
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    dQ = brl.attn_bwd_dq(q, k, v, O, torch.from_numpy(dO).cuda(), stats, window, s_v)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy()
    assert_bitwise(Oh, oracle.attn_fwd(Q, K, V, window, s_v), "O")
    assert_bitwise(dQ, oracle.attn_bwd_dq(Q, K, V, Oh, dO, window, s_v), f"dQ (S={S} w={window})")


@pytest.mark.parametrize("window", [0, 40])
def test_attention_equal_and_near_equal_logits(window):
    """Equal and near-equal logits: Q = 0 (all logits 0) and keys that differ
    by a few ulp, so the row maximum is a tie or a near tie among many keys
    (the case that made every key a candidate of the earlier approximate
    first pass)."""
    B, S, Hq, Hkv, s_v = 1, 150, 4, 2, 0.05
    g = np.random.default_rng(window)
    V = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    base = g.standard_normal(D).astype(np.float32)
    K = np.tile(base, (B, S, Hkv, 1)).astype(np.float32)
    K += (g.integers(-3, 4, K.shape) * np.spacing(np.abs(K))).astype(np.float32)
    for Q in (np.zeros((B, S, Hq, D), np.float32), g.standard_normal((B, S, Hq, D)).astype(np.float32)):
        O = brl.attn_fwd(*(torch.from_numpy(t).cuda() for t in (Q, K, V)), window, s_v)
        torch.cuda.synchronize()
        assert_bitwise(O, oracle.attn_fwd(Q, K, V, window, s_v), f"O (near-equal logits, window {window})")


@pytest.mark.parametrize("q_scale,k_scale", [(1e-20, 1e19), (3e17, 1e-18), (1.0, 40.0)])
def test_attention_extreme_scales(q_scale, k_scale):
    """Q and K of very different magnitudes (squared norms far outside
    binary32's range on one side), and logits spread over hundreds of units
    (the cases that stressed the earlier approximate pass's error bound)."""
    B, S, Hq, Hkv, window, s_v = 1, 130, 4, 2, 50, 0.05
    g = np.random.default_rng(int(abs(np.log10(q_scale))) + 1)
    Q = (g.standard_normal((B, S, Hq, D)) * q_scale).astype(np.float32)
    K = (g.standard_normal((B, S, Hkv, D)) * k_scale).astype(np.float32)
    V = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    O = brl.attn_fwd(*(torch.from_numpy(t).cuda() for t in (Q, K, V)), window, s_v)
    torch.cuda.synchronize()
    assert_bitwise(O, oracle.attn_fwd(Q, K, V, window, s_v), f"O (scales {q_scale}, {k_scale})")


KV_CASES = [
    # B, S, Hq, Hkv, window, s_v
    (1, 1, 1, 1, 0, 0.05),
    (1, 64, 2, 1, 0, 0.05),
    (2, 150, 4, 2, 0, 0.05),
    (1, 200, 4, 2, 64, 0.0371),
    (1, 333, 16, 4, 130, 0.05),
    (1, 100, 4, 4, 1, 0.05),
    (1, 190, 8, 2, 500, 0.05),        # window longer than the sequence
    (2, 129, 8, 1, 70, 0.05),         # eight query heads per KV head
]


@pytest.mark.parametrize("B,S,Hq,Hkv,window,s_v", KV_CASES)
def test_attention_dkdv_parity(B, S, Hq, Hkv, window, s_v):
    """dK and dV with 64-bit fixed-point accumulation, bit for bit, from the
    forward's own O and (m, l) statistics; a few V entries outside the
    quantiser's range get +0."""
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=5 * S + Hq + window, scale=0.3)
    V.reshape(-1)[::977] = 7.5                 # 150 steps at s_v = 0.05: clamped
    dO = (np.random.default_rng(S + window + 1).standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    q, k, v = (torch.from_numpy(t).cuda() for t in (Q, K, V))
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    dK, dV = brl.attn_bwd_dkdv(q, k, v, O, torch.from_numpy(dO).cuda(), stats, window, s_v)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy()
    assert_bitwise(Oh, oracle.attn_fwd(Q, K, V, window, s_v), "O")
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, Oh, dO, window, s_v)
    assert_bitwise(dK, wk, f"dK (S={S} w={window})")
    assert_bitwise(dV, wv, f"dV (S={S} w={window})")


def test_attention_dkdv_into_qkv_gradient_slices():
    """Q, K, V as column slices of the QKV projection output and dK, dV
    written as column slices of one [B*S, (Hq + 2 Hkv) * D] gradient buffer;
    the dQ columns stay untouched."""
    B, S, Hq, Hkv, window, s_v = 2, 170, 4, 1, 96, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=11, scale=0.3)
    dO = (np.random.default_rng(12).standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    Y = np.concatenate([Q.reshape(B * S, -1), K.reshape(B * S, -1), V.reshape(B * S, -1)], axis=1)
    Yd = torch.from_numpy(np.ascontiguousarray(Y)).cuda()
    q = Yd[:, :Hq * D].view(B, S, Hq, D)
    k = Yd[:, Hq * D:(Hq + Hkv) * D].view(B, S, Hkv, D)
    v = Yd[:, (Hq + Hkv) * D:].view(B, S, Hkv, D)
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    G = torch.full((B * S, (Hq + 2 * Hkv) * D), 3.0, device="cuda")
    dK = G[:, Hq * D:(Hq + Hkv) * D].view(B, S, Hkv, D)
    dV = G[:, (Hq + Hkv) * D:].view(B, S, Hkv, D)
    brl.attn_bwd_dkdv(q, k, v, O, torch.from_numpy(dO).cuda(), stats, window, s_v, dK=dK, dV=dV)
    torch.cuda.synchronize()
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, O.cpu().numpy(), dO, window, s_v)
    assert_bitwise(dK, wk, "dK (slices)")
    assert_bitwise(dV, wv, "dV (slices)")
    assert torch.all(G[:, :Hq * D] == 3.0)


def test_attention_dkdv_repeat_and_zero_gradient():
    """Two calls give the same bits; dO = 0 gives +0 everywhere."""
    B, S, Hq, Hkv, window, s_v = 1, 257, 4, 2, 0, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=13, scale=2.0)
    dO = (np.random.default_rng(14).standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    q, k, v, g = (torch.from_numpy(t).cuda() for t in (Q, K, V, dO))
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    k1, v1 = brl.attn_bwd_dkdv(q, k, v, O, g, stats, window, s_v)
    k2, v2 = brl.attn_bwd_dkdv(q, k, v, O, g, stats, window, s_v)
    k0, v0 = brl.attn_bwd_dkdv(q, k, v, O, torch.zeros_like(g), stats, window, s_v)
    torch.cuda.synchronize()
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, O.cpu().numpy(), dO, window, s_v)
    for t, w, n in ((k1, wk, "dK"), (v1, wv, "dV"), (k2, wk, "dK repeat"), (v2, wv, "dV repeat")):
        assert_bitwise(t, w, n)
    assert np.all(_bits(k0) == 0) and np.all(_bits(v0) == 0)


def test_attention_backward_with_subnormal_inputs():
    """1% of the entries of Q, K, V and dO at subnormal magnitudes (read as
    zero by every binary32 operation) and some exact zeros: the forward, dQ,
    dK and dV stay bit-identical to the oracle."""
    B, S, Hq, Hkv, window, s_v = 1, 140, 4, 2, 60, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=17, scale=0.3)
    g = np.random.default_rng(18)
    dO = (g.standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    for t in (Q, K, V, dO):
        flat = t.reshape(-1)
        idx = g.choice(flat.size, flat.size // 100, replace=False)
        flat[idx] = (g.choice([-1.0, 1.0], idx.size) * g.uniform(1e-45, 1e-38, idx.size)).astype(np.float32)
        flat[g.choice(flat.size, flat.size // 200, replace=False)] = 0.0
    q, k, v, go = (torch.from_numpy(t).cuda() for t in (Q, K, V, dO))
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    dQ = brl.attn_bwd_dq(q, k, v, O, go, stats, window, s_v)
    dK, dV = brl.attn_bwd_dkdv(q, k, v, O, go, stats, window, s_v)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy()
    assert_bitwise(Oh, oracle.attn_fwd(Q, K, V, window, s_v), "O (subnormal inputs)")
    assert_bitwise(dQ, oracle.attn_bwd_dq(Q, K, V, Oh, dO, window, s_v), "dQ (subnormal inputs)")
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, Oh, dO, window, s_v)
    assert_bitwise(dK, wk, "dK (subnormal inputs)")
    assert_bitwise(dV, wv, "dV (subnormal inputs)")


def test_attention_backward_binding_rejects_bad_outputs():
    """The binding refuses dK/dV of the wrong shape, only one of the two, or
    with different row strides, before anything is launched."""
    B, S, Hq, Hkv, window, s_v = 1, 64, 4, 2, 0, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=19)
    q, k, v = (torch.from_numpy(t).cuda() for t in (Q, K, V))
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    go = torch.zeros_like(O)
    with pytest.raises(ValueError):
        brl.attn_bwd_dkdv(q, k, v, O, go, stats, window, s_v, dK=torch.empty_like(k))
    with pytest.raises(ValueError):
        brl.attn_bwd_dkdv(q, k, v, O, go, stats, window, s_v, dK=torch.empty_like(q), dV=torch.empty_like(q))
    wide = torch.empty((B * S, 3 * Hkv * D), device="cuda")
    with pytest.raises(ValueError):
        brl.attn_bwd_dkdv(q, k, v, O, go, stats, window, s_v, dK=torch.empty_like(k),
                          dV=wide[:, :Hkv * D].view(B, S, Hkv, D))
    with pytest.raises(ValueError):
        brl.attn_bwd_dkdv(q, k, v, O, go, stats[..., :1], window, s_v)
    torch.cuda.synchronize()


def test_attention_kernels_repeat_ten_times_bit_identically():
    """Ten runs of each attention kernel on one input agree bit for bit (the
    forward's row maxima come from an integer atomic maximum, and the
    gradients from exact int64 sums, so no run may differ)."""
    B, S, Hq, Hkv, window, s_v = 2, 300, 8, 2, 100, 0.05
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=23, scale=0.5)
    dO = (np.random.default_rng(24).standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    q, k, v, go = (torch.from_numpy(t).cuda() for t in (Q, K, V, dO))
    first = None
    for _ in range(10):
        stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
        O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
        dQ = brl.attn_bwd_dq(q, k, v, O, go, stats, window, s_v)
        dK, dV = brl.attn_bwd_dkdv(q, k, v, O, go, stats, window, s_v)
        cur = [t.view(torch.int32).clone() for t in (O, stats, dQ, dK, dV)]
        if first is None:
            first = cur
        else:
            for name, a, b in zip(["O", "stats", "dQ", "dK", "dV"], first, cur):
                assert torch.equal(a, b), f"{name} differs between runs"
    torch.cuda.synchronize()
    assert_bitwise(first[0].view(torch.float32), oracle.attn_fwd(Q, K, V, window, s_v), "O")


# ---- keys of unequal norm: the row maximum must be the exact one ----
def _witness_inputs(S=160):
    """Every query is all ones.  Keys 5, 40 and 70 are the high-norm key l
    (bf16 operands 64(1+2^-7) and -64: approximate logit 2.83, exact 0.011,
    bound 11.4); keys 7, 30 and 60 are 0.125 everywhere (exact logit 1.414,
    the rows' maximum, bound 0.022); the other keys are small.  Pairs sit in
    one key tile, in the other order, and across a tile boundary."""
    g = np.random.default_rng(77)
    Q = np.ones((1, S, 1, D), np.float32)
    K = (g.standard_normal((1, S, 1, D)) * 1e-3).astype(np.float32)
    hi = np.float32(64.0 * (1 + 2.0 ** -8 + 2.0 ** -16))
    lo = np.float32(-64.0 * (1 + 2.0 ** -8 - 2.0 ** -16))
    kl = np.where(np.arange(D) % 2 == 0, hi, lo).astype(np.float32)
    for j in (5, 40, 70):
        K[0, j, 0] = kl
    for j in (7, 30, 60):
        K[0, j, 0] = 0.125
    V = g.standard_normal((1, S, 1, D)).astype(np.float32)
    dO = (g.standard_normal((1, S, 1, D)) * 1e-2).astype(np.float32)
    return Q, K, V, dO


def _full_check(Q, K, V, dO, window, s_v, what, O_bwd=None):
    """Forward (O and its statistics) and the three gradients against the
    oracle; the gradients take the forward's O, or O_bwd when given."""
    q, k, v = (torch.from_numpy(t).cuda() for t in (Q, K, V))
    B, S, Hq, _ = Q.shape
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    g = torch.from_numpy(dO).cuda()
    Ob = O if O_bwd is None else torch.from_numpy(O_bwd).cuda()
    dQ = brl.attn_bwd_dq(q, k, v, Ob, g, stats, window, s_v)
    dK, dV = brl.attn_bwd_dkdv(q, k, v, Ob, g, stats, window, s_v)
    torch.cuda.synchronize()
    assert_bitwise(O, oracle.attn_fwd(Q, K, V, window, s_v), f"O ({what})")
    Oh = Ob.cpu().numpy()
    assert_bitwise(dQ, oracle.attn_bwd_dq(Q, K, V, Oh, dO, window, s_v), f"dQ ({what})")
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, Oh, dO, window, s_v)
    assert_bitwise(dK, wk, f"dK ({what})")
    assert_bitwise(dV, wv, f"dV ({what})")
    return stats.cpu().numpy()


@pytest.mark.parametrize("window", [0, 64])
def test_attention_keys_of_unequal_norm_witness(window):
    """O, (m, l), dQ, dK and dV on the witness row: m_i is the exact logit of
    the 0.125 key (16 c) for every row that attends one, never the key whose
    bf16 logit is larger (the witness that defeated the earlier pruning
    rule)."""
    Q, K, V, dO = _witness_inputs()
    st = _full_check(Q, K, V, dO, window, 0.05, f"witness w={window}")
    c = np.float32(np.float32(1.0) / np.sqrt(np.float32(D)))
    m_j = np.float32(np.float32(16.0) * c)      # 128 products 0.125 summed exactly, times c
    for i in range(Q.shape[1]):
        lo = max(0, i - window + 1) if window > 0 else 0
        if any(lo <= j <= i for j in (7, 30, 60)):
            assert _bits(st[0, i, 0, 0]) == _bits(m_j), (i, st[0, i, 0, 0])


@pytest.mark.parametrize("window", [0, 64])
def test_attention_keys_with_spread_norms(window):
    """Per-key norms spread over 1e-2 .. 1e2 within every row, GQA 4/2."""
    g = np.random.default_rng(300 + window)
    B, S, Hq, Hkv, s_v = 1, 200, 4, 2, 0.05
    Q = (g.standard_normal((B, S, Hq, D)) * 0.3).astype(np.float32)
    K = (g.standard_normal((B, S, Hkv, D)) * 10.0 ** g.uniform(-2, 2, (B, S, Hkv, 1))).astype(np.float32)
    V = g.standard_normal((B, S, Hkv, D)).astype(np.float32)
    dO = (g.standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    _full_check(Q, K, V, dO, window, s_v, f"spread norms w={window}")


def test_attention_fixed_point_ties_on_device():
    """The crafted inputs of the CPU pins of the fixed-point format (tile sums
    at exact ties of the 2^-40 grid, terms in both 32-halves of a 64-tile and
    on both sides of position 64), with the pins' O = 0 given to the
    gradients: the kernels give the oracle's bits."""
    from tests.test_oracle_order_pins import _case_a, WIN
    Q, K, V, O, dO, _, _ = _case_a()
    _full_check(Q, K, V, dO, WIN, 1.0, "fixed-point ties, Q = 0", O_bwd=O)
    # the same with K = 0 and Q carrying the terms (the dK pin's layout)
    Q2 = np.zeros_like(Q)
    Q2[0, 63, 0, 1] = Q2[0, 64, 0, 1] = np.float32(2.0 ** -35)
    Q2[0, 80, 0, 2] = Q2[0, 100, 0, 2] = np.float32(2.0 ** -35)
    Q2[0, 64, 0, 3] = np.float32(3 * 2.0 ** -35)
    dO2 = np.zeros_like(dO)
    for i in (63, 64, 80, 100):
        dO2[0, i, 0, 0] = 1.0
    V2 = np.zeros_like(V)
    V2[0, 40, 0, 0] = V2[0, 64, 0, 0] = 1.0
    _full_check(Q2, np.zeros_like(K), V2, dO2, WIN, 1.0, "fixed-point ties, K = 0", O_bwd=np.zeros_like(O))


def test_attention_workgroups_walk_several_items():
    """The forward runs a persistent grid of at most 512 workgroups, each
    walking (batch, query head, query block) items and reusing one slot of
    the workspace for every item's stored logits.  2 x 16 heads x 18 query
    blocks = 576 items, so some workgroups take two items of different
    lengths (last blocks first); every output and statistic must still be
    the oracle's."""
    B, S, Hq, Hkv, window, s_v = 2, 1100, 16, 4, 100, 0.05
    assert B * Hq * ((S + 63) // 64) > 512
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=41, scale=0.3)
    dO = (np.random.default_rng(43).standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    q, k, v = (torch.from_numpy(t).cuda() for t in (Q, K, V))
    stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
    # dQ reads the statistics (m, l) the forward wrote for every row
    rows = np.arange(0, B * S * Hq, 97)
    dQ = brl.attn_bwd_dq(q, k, v, O, torch.from_numpy(dO).cuda(), stats, window, s_v)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy()
    assert_bitwise(Oh, oracle.attn_fwd(Q, K, V, window, s_v), "O (several items per workgroup)")
    want = oracle.attn_bwd_dq(Q, K, V, Oh, dO, window, s_v, rows=rows)
    got = dQ.cpu().numpy().reshape(B * S * Hq, D)[rows]
    assert_bitwise(got, np.asarray(want).reshape(got.shape), "dQ rows (several items per workgroup)")


KEEP_CASES = [
    # B, S, Hq, Hkv, window, s_v
    (1, 1, 1, 1, 0, 0.05),
    (2, 150, 4, 2, 0, 0.05),
    (1, 200, 4, 2, 64, 0.0371),
    (1, 333, 16, 4, 130, 0.05),
    (1, 190, 8, 2, 500, 0.05),        # window longer than the sequence
    (2, 129, 8, 1, 70, 0.05),
    (1, 100, 4, 4, 1, 0.05),
]


def _oracle_logit(Q, K, b, i, h, j, hk):
    """s_ij = CanonSum_d(q_id * k_jd) * c with the oracle's CanonSum and
    binary32 products and multiply (inputs are normal numbers)."""
    prods = (Q[b, i, h].astype(np.float32) * K[b, j, hk].astype(np.float32)).astype(np.float32)
    c = np.float32(1.0 / float(np.float32(np.sqrt(np.float64(D)))))
    return oracle.mul(oracle.canon_sum(prods), c)


@pytest.mark.parametrize("B,S,Hq,Hkv,window,s_v", KEEP_CASES)
def test_attention_kept_logits(B, S, Hq, Hkv, window, s_v):
    """The forward that keeps its logits gives O and (m, l) bit for bit as
    the plain forward and the oracle; the kept logits are the oracle's s_ij on
    sampled allowed positions; dQ, dK and dV read from them equal the
    oracle's bit for bit."""
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=11 * S + Hq + window, scale=0.3)
    V.reshape(-1)[::977] = 7.5
    dO = (np.random.default_rng(S + window + 3).standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)
    q, k, v = (torch.from_numpy(t).cuda() for t in (Q, K, V))
    g = torch.from_numpy(dO).cuda()
    st0 = torch.empty((B, S, Hq, 2), dtype=torch.float32, device="cuda")
    st1 = torch.empty_like(st0)
    O0 = brl.attn_fwd(q, k, v, window, s_v, stats=st0)
    logits = brl.attn_logits_buffer(B, S, Hq, window)
    logits.fill_(float("nan"))
    O1 = brl.attn_fwd(q, k, v, window, s_v, stats=st1, logits=logits)
    dQ = brl.attn_bwd_dq(q, k, v, O1, g, st1, window, s_v, logits=logits)
    dK, dV = brl.attn_bwd_dkdv(q, k, v, O1, g, st1, window, s_v, logits=logits)
    torch.cuda.synchronize()
    assert_bitwise(O1, O0, "O (kept logits) vs O")
    assert_bitwise(st1, st0, "stats (kept logits) vs stats")
    Oh = O1.cpu().numpy()
    assert_bitwise(Oh, oracle.attn_fwd(Q, K, V, window, s_v), "O")
    assert_bitwise(dQ, oracle.attn_bwd_dq(Q, K, V, Oh, dO, window, s_v), f"dQ from kept logits (S={S} w={window})")
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, Oh, dO, window, s_v)
    assert_bitwise(dK, wk, f"dK from kept logits (S={S} w={window})")
    assert_bitwise(dV, wv, f"dV from kept logits (S={S} w={window})")
    # the kept slots: slot (nqb - 1 - qb) * B*Hq + b*Hq + h, tiles from the block's first key tile
    lg = logits.cpu().numpy()
    nqb = (S + 63) // 64
    tiles = max(((min(qb * 64 + 63, S - 1)) // 64 - (max(0, qb * 64 - window + 1) if window > 0 else 0) // 64 + 1)
                for qb in range(nqb))
    assert lg.size * 4 == brl.attn_logits_bytes(B, S, Hq, window) == nqb * B * Hq * tiles * 64 * 64 * 4
    rng = np.random.default_rng(S)
    for _ in range(40):
        b, h, i = int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(S))
        lo = max(0, i - window + 1) if window > 0 else 0
        j = int(rng.integers(lo, i + 1))
        qb = i // 64
        kt0 = (max(0, qb * 64 - window + 1) if window > 0 else 0) // 64
        slot = (nqb - 1 - qb) * B * Hq + b * Hq + h
        got = lg[(slot * tiles + j // 64 - kt0) * 4096 + (i % 64) * 64 + j % 64]
        want = _oracle_logit(Q, K, b, i, h, j, h // (Hq // Hkv))
        assert np.float32(got).view(np.uint32) == np.float32(want).view(np.uint32), (b, h, i, j, got, want)


def test_attention_kept_logits_rejects_a_short_buffer():
    B, S, Hq, Hkv = 1, 130, 4, 2
    Q, K, V = _inputs(B, S, Hq, Hkv, seed=1)
    q, k, v = (torch.from_numpy(t).cuda() for t in (Q, K, V))
    short = torch.empty(brl.attn_logits_bytes(B, S, Hq, 64) // 4 - 64, dtype=torch.float32, device="cuda")
    with pytest.raises(brl.BrlError):
        brl.attn_fwd(q, k, v, 64, 0.05, logits=short)
