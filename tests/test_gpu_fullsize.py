"""Parity at the full workload sizes, in the launch configuration bench.py
times, against the oracle: every element of the forward's outputs (Y, and
Ypre with the SwiGLU activation), one row of dX in every 64-row tile (the
rows at tile, workgroup and microbatch edges included) and one row of dW in
every 64-row tile of W -- and for the replay, every element.

Workloads (seeded, synthetic; shapes of the Open-1B recipe on the onedev.kr
summary, "Use" and "Limits": 16,384 tokens per GPU microbatch, GQA with 16
query and 4 KV heads, SwiGLU gate+up as one GEMM, 6x8 replay mesh):
  qkv             X [16384,2048], W [3072,2048], dY [16384,3072]
  swiglu_gate_up  X [16384,2048], W [11264,2048] (gate rows 0..5631, up rows
                  5632..11263), dA [16384,5632]
  down_proj       H [16384,5632] ~ SiLU(a)*b, W [2048,5632], dY [16384,2048],
                  dW accumulated over 4 microbatches of 4096 rows
  replay_6x8      48 partials of 201,326,592 fp32 ~ N(0, 1e-4)
Tolerance 0 ULP everywhere.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


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
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at flat {i}: "
                             f"got {g.ravel()[i]:#010x} want {w.ravel()[i]:#010x}")


def _sample(n, edges, k, seed):
    g = np.random.default_rng(seed)
    s = set(e for e in edges if 0 <= e < n)
    s.update(int(x) for x in g.choice(n, k, replace=False))
    return np.array(sorted(s), np.int64)


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


TILE_EDGES_M = [0, 1, 63, 64, 255, 256, 4095, 4096, 8191, 8192, 12287, 12288, 16383]


def _per_tile(n, edges, seed, tile=64):
    """One row in every `tile` rows (its position varying from tile to tile)
    plus the given edge rows."""
    g = np.random.default_rng(seed)
    s = set(e for e in edges if 0 <= e < n)
    for t0 in range(0, n, tile):
        s.add(int(t0 + g.integers(0, min(tile, n - t0))))
    return np.array(sorted(s), np.int64)


def _all_rows(case):
    return np.arange(case.M, dtype=np.int64)


def test_qkv_full_size():
    case = synth.CASES["qkv"]
    inp = synth.linear_inputs(case)
    X, W, dY = _cuda(inp.X), _cuda(inp.W), _cuda(inp.dY)
    Y, _, s_w = brl.qat_linear_fwd(X, W, case.s_x)
    dX, dW = brl.qat_linear_bwd(dY, X, W, case.s_x)
    torch.cuda.synchronize()
    w_sw = oracle.weight_scale(inp.W)
    assert_bitwise(s_w, np.array([w_sw]), "s_w")
    assert_bitwise(Y, oracle.fwd_rows(inp.X, inp.W, case.s_x, rows=_all_rows(case), s_w=w_sw), "Y (every row)")
    rows = _per_tile(case.M, TILE_EDGES_M, 1)
    assert_bitwise(dX[rows], oracle.dx_rows(inp.dY[rows], inp.X, inp.W, case.s_x, rows, s_w=w_sw), "dX rows")
    wr = _per_tile(case.N, [0, 1, 2047, 2048, 2559, 2560, 3071], 2)
    want = oracle.dw_rows(np.ascontiguousarray(inp.dY[:, wr].T), inp.X, inp.W, case.s_x, wr, s_w=w_sw)
    assert_bitwise(dW[wr], want, "dW rows")


def test_swiglu_gate_up_full_size():
    case = synth.CASES["swiglu_gate_up"]
    inp = synth.linear_inputs(case)
    H = case.N // 2
    X, W, dA = _cuda(inp.X), _cuda(inp.W), _cuda(inp.dY)
    A, Ypre, s_w = brl.qat_linear_fwd(X, W, case.s_x, epilogue=brl.EPILOGUE_SWIGLU)
    dX, dW = brl.qat_linear_bwd(dA, X, W, case.s_x, Ypre=Ypre, epilogue=brl.EPILOGUE_SWIGLU)
    torch.cuda.synchronize()
    w_sw = oracle.weight_scale(inp.W)
    assert_bitwise(s_w, np.array([w_sw]), "s_w")
    wA, wPre = oracle.fwd_rows(inp.X, inp.W, case.s_x, rows=_all_rows(case), epilogue=1, s_w=w_sw)
    assert_bitwise(Ypre, wPre, "Ypre (every row)")
    assert_bitwise(A, wA, "SwiGLU activation (every row)")
    rows = _per_tile(case.M, TILE_EDGES_M, 3)
    G_rows = oracle.swiglu_bwd(wPre[rows], inp.dY[rows])
    assert_bitwise(dX[rows], oracle.dx_rows(G_rows, inp.X, inp.W, case.s_x, rows, s_w=w_sw), "dX rows")
    # dW rows n and n + H need the gate and up columns j = n of the
    # pre-activation over all M rows (the oracle's own, from above)
    js = _per_tile(H, [0, 63, 64, 5631], 4)
    cols = np.concatenate([js, js + H])
    pair_cols = np.ascontiguousarray(wPre[:, cols])                    # [M, 2J]: gate cols, then up cols
    dY_cols = []
    G_gate, G_up = [], []
    for t, j in enumerate(js):
        pair = np.ascontiguousarray(np.stack([pair_cols[:, t], pair_cols[:, t + len(js)]], axis=1))   # (g, u)
        d = oracle.swiglu_bwd(pair, np.ascontiguousarray(inp.dY[:, j:j + 1]))
        G_gate.append(d[:, 0].copy())
        G_up.append(d[:, 1].copy())
    dY_cols = np.stack(G_gate + G_up)
    want = oracle.dw_rows(dY_cols, inp.X, inp.W, case.s_x, cols, s_w=w_sw)
    assert_bitwise(dW[cols], want, "dW rows (gate and up)")


def test_down_proj_full_size_microbatches():
    case = synth.CASES["down_proj"]
    inp = synth.linear_inputs(case)
    X, W, dY = _cuda(inp.X), _cuda(inp.W), _cuda(inp.dY)
    B = case.microbatches
    mb = case.M // B
    Y, _, s_w = brl.qat_linear_fwd(X, W, case.s_x)
    dX = torch.empty_like(X)
    dW = None
    for b in range(B):
        sl = slice(b * mb, (b + 1) * mb)
        dXb, dW = brl.qat_linear_bwd(dY[sl], X[sl], W, case.s_x, dX=dX[sl], dW=dW, dW_accumulate=b > 0)
    torch.cuda.synchronize()
    w_sw = oracle.weight_scale(inp.W)
    assert (np.abs(inp.X / case.s_x) > 127).any(), "some activations should clip"
    assert_bitwise(Y, oracle.fwd_rows(inp.X, inp.W, case.s_x, rows=_all_rows(case), s_w=w_sw), "Y (every row)")
    rows = _per_tile(case.M, TILE_EDGES_M, 5)
    assert_bitwise(dX[rows], oracle.dx_rows(inp.dY[rows], inp.X, inp.W, case.s_x, rows, s_w=w_sw), "dX rows")
    wr = _per_tile(case.N, [0, 1, 2047], 6)
    want = oracle.dw_rows(np.ascontiguousarray(inp.dY[:, wr].T), inp.X, inp.W, case.s_x, wr, mb=mb, s_w=w_sw)
    assert_bitwise(dW[wr], want, "dW rows (4 microbatches)")


@pytest.mark.parametrize("resident", [False, True])
def test_replay_full_size(resident):
    """All 48 ranks at 201,326,592 elements; every element of the clipped
    TreeFold, the norm and the running sums A_0..A_4 are compared.  The
    partials arrive one call at a time, either released after each call or
    (resident) kept per replica until its last shard's call, which then
    forms the replica's running sum in one pass."""
    rc = synth.REPLAY
    R, S, L = rc.replicas, rc.shards, rc.length
    st = brl.ReduceState(R, S, L, device=DEV, replica_resident=resident)
    out = torch.empty(L, dtype=torch.float32, device=DEV)
    A = [np.empty(L, np.float32) for _ in range(R)]
    host = np.empty(L, np.float32)
    kept = []
    for v in range(R * S):
        G = synth.replay_partial(rc, v, device=DEV)
        brl.ordered_reduce(st, G, out=out)
        torch.cuda.synchronize()
        host[:] = G.cpu().numpy()
        r, s = divmod(v, S)
        oracle.replay_accumulate(A[r], host, first=(s == 0))
        if resident:
            kept.append(G)
            if s == S - 1:
                kept.clear()       # the replica's last call has run (synchronised above)
        del G
    nu = brl.grad_l2norm_clip(out, rc.max_norm)
    torch.cuda.synchronize()
    T = oracle.treefold(A)
    wnu = oracle.l2norm(T)
    oracle.clip(T, wnu, rc.max_norm, 0.0)
    assert_bitwise(nu, np.array([wnu]), "nu")
    assert float(wnu) > 1.0
    assert_bitwise(out, T, "clipped TreeFold")
    for r in range(R - 1):
        assert_bitwise(st.acc[r], A[r], f"A_{r}")


@pytest.mark.parametrize("name", ["attn_window", "attn_causal"])
def test_attention_full_size(name):
    """One Open-1B layer's attention at the microbatch (4 x 4096 tokens, 16/4
    heads): rows at the sequence start, at query-tile and window edges and
    at the end, plus random rows, for several heads of both KV groups' ends."""
    case = synth.ATTENTION_CASES[name]
    Q, K, V = synth.attention_inputs(case)
    O = brl.attn_fwd(_cuda(Q), _cuda(K), _cuda(V), case.window, case.s_v)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy().reshape(-1, 128)
    edges = [0, 1, 63, 64, 65, 511, 512, 513, 1023, 2048, case.S - 1]
    rows = []
    for b, h in [(0, 0), (1, 3), (2, 4), (3, 15)]:
        for i in _sample(case.S, edges, 6, seed=b * 16 + h):
            rows.append((b * case.S + int(i)) * case.Hq + h)
    rows = np.array(rows, np.int64)
    want = oracle.attn_fwd_rows(Q, K, V, case.window, case.s_v, rows)
    assert_bitwise(Oh[rows], want, f"O rows ({name})")


@pytest.mark.parametrize("name", ["attn_window", "attn_causal"])
def test_attention_dq_full_size(name):
    """dQ (64-bit fixed-point accumulation) at one Open-1B layer, on sampled
    rows, from the forward's own O and statistics; dO ~ N(0, 1e-3)."""
    case = synth.ATTENTION_CASES[name]
    Q, K, V = synth.attention_inputs(case)
    dO = synth.normal(case.seed, "dY", Q.shape, 1e-3)
    q, k, v = _cuda(Q), _cuda(K), _cuda(V)
    stats = torch.empty((case.B, case.S, case.Hq, 2), dtype=torch.float32, device=DEV)
    O = brl.attn_fwd(q, k, v, case.window, case.s_v, stats=stats)
    dQ = brl.attn_bwd_dq(q, k, v, O, _cuda(dO), stats, case.window, case.s_v)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy()
    dQh = dQ.cpu().numpy().reshape(-1, 128)
    edges = [0, 1, 63, 64, 511, 512, 2048, case.S - 1]
    rows = []
    for b, h in [(0, 0), (3, 15)]:
        for i in _sample(case.S, edges, 3, seed=b * 16 + h + 1):
            rows.append((b * case.S + int(i)) * case.Hq + h)
    rows = np.array(rows, np.int64)
    want = oracle.attn_bwd_dq(Q, K, V, Oh, dO, case.window, case.s_v, rows=rows)
    assert_bitwise(dQh[rows], want, f"dQ rows ({name})")


@pytest.mark.parametrize("name", ["attn_window", "attn_causal"])
def test_attention_dkdv_full_size(name):
    """dK and dV (64-bit fixed-point accumulation) at one Open-1B layer, on
    sampled key rows of one KV head per case (the first and the last), from
    the forward's own O and statistics; dO ~ N(0, 1e-3)."""
    case = synth.ATTENTION_CASES[name]
    Q, K, V = synth.attention_inputs(case)
    dO = synth.normal(case.seed, "dY", Q.shape, 1e-3)
    q, k, v = _cuda(Q), _cuda(K), _cuda(V)
    stats = torch.empty((case.B, case.S, case.Hq, 2), dtype=torch.float32, device=DEV)
    O = brl.attn_fwd(q, k, v, case.window, case.s_v, stats=stats)
    dK, dV = brl.attn_bwd_dkdv(q, k, v, O, _cuda(dO), stats, case.window, case.s_v)
    torch.cuda.synchronize()
    Oh = O.cpu().numpy()
    dKh = dK.cpu().numpy().reshape(-1, 128)
    dVh = dV.cpu().numpy().reshape(-1, 128)
    b, hk = (0, 0) if name == "attn_window" else (case.B - 1, case.Hkv - 1)
    edges = [0, 63, 64, 511, 512, case.S - 65, case.S - 1] if name == "attn_window" else \
        [2048, 3071, 4031, 4032, case.S - 1]
    rows = np.array([(b * case.S + int(j)) * case.Hkv + hk
                     for j in _sample(case.S, edges, 2, seed=7 + hk) if name == "attn_window" or j >= 2048],
                    np.int64)
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, Oh, dO, case.window, case.s_v, rows=rows)
    assert_bitwise(dKh[rows], wk, f"dK rows ({name})")
    assert_bitwise(dVh[rows], wv, f"dV rows ({name})")


@pytest.mark.parametrize("name", ["attn_window", "attn_causal"])
def test_attention_kept_logits_full_size(name):
    """The training path at one Open-1B layer: the forward keeping its
    logits and dQ, dK, dV read from them equal the path that forms them
    again, every element, and the oracle on sampled rows."""
    case = synth.ATTENTION_CASES[name]
    Q, K, V = synth.attention_inputs(case)
    dO = synth.normal(case.seed, "dY", Q.shape, 1e-3)
    q, k, v, g = _cuda(Q), _cuda(K), _cuda(V), _cuda(dO)
    st0 = torch.empty((case.B, case.S, case.Hq, 2), dtype=torch.float32, device=DEV)
    st1 = torch.empty_like(st0)
    O0 = brl.attn_fwd(q, k, v, case.window, case.s_v, stats=st0)
    dQ0 = brl.attn_bwd_dq(q, k, v, O0, g, st0, case.window, case.s_v)
    dK0, dV0 = brl.attn_bwd_dkdv(q, k, v, O0, g, st0, case.window, case.s_v)
    L = brl.attn_logits_buffer(case.B, case.S, case.Hq, case.window, DEV)
    O1 = brl.attn_fwd(q, k, v, case.window, case.s_v, stats=st1, logits=L)
    dQ1 = brl.attn_bwd_dq(q, k, v, O1, g, st1, case.window, case.s_v, logits=L)
    dK1, dV1 = brl.attn_bwd_dkdv(q, k, v, O1, g, st1, case.window, case.s_v, logits=L)
    torch.cuda.synchronize()
    del L
    for got, want, what in ((O1, O0, "O"), (st1, st0, "stats"), (dQ1, dQ0, "dQ"), (dK1, dK0, "dK"), (dV1, dV0, "dV")):
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"{what} (kept logits, {name})"
    Oh = O1.cpu().numpy()
    rows = np.array([(b * case.S + i) * case.Hq + h for b, h, i in [(0, 0, 0), (1, 5, 600), (3, 15, case.S - 1)]],
                    np.int64)
    assert_bitwise(dQ1.cpu().numpy().reshape(-1, 128)[rows],
                   oracle.attn_bwd_dq(Q, K, V, Oh, dO, case.window, case.s_v, rows=rows), f"dQ rows ({name})")
    krows = np.array([(b * case.S + j) * case.Hkv + hk for b, hk, j in [(0, 0, 4095), (3, 3, 4032)]], np.int64)
    wk, wv = oracle.attn_bwd_dkdv(Q, K, V, Oh, dO, case.window, case.s_v, rows=krows)
    assert_bitwise(dK1.cpu().numpy().reshape(-1, 128)[krows], wk, f"dK rows ({name})")
    assert_bitwise(dV1.cpu().numpy().reshape(-1, 128)[krows], wv, f"dV rows ({name})")
