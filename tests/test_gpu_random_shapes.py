"""A seeded sweep of the linear layer over random shapes and launch options
against the oracle, every output bit for bit: M, K, N drawn over [1, 320] x
[1, 700] x [2, 320], with the SwiGLU epilogue on a third of the cases, an
addend on some plain ones, dY with or without subnormal entries, the
forward's preparation in one launch or in separate ones, the backward on
either engine at the default or a random chunk depth, and dW accumulated
onto a previous result on some.  The draws are fixed (seed 2026): the same
cases run every time."""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import oracle
import synth

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=2026):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        swiglu = i % 3 == 0
        M = int(g.integers(1, 321))
        K = int(g.integers(1, 701))
        N = int(g.integers(2, 321))
        if swiglu:
            N += N % 2
        out.append(dict(i=i, M=M, K=K, N=N, swiglu=swiglu,
                        addend=(not swiglu) and i % 4 == 1,
                        sub=0.01 if i % 2 else 0.0,
                        fwd_prep=int(g.integers(1, 3)), engine=int(g.integers(1, 3)),
                        chunk=int(g.integers(1, 8)) if i % 3 == 1 else 0,
                        acc=i % 5 == 2))
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


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("c", _cases(), ids=lambda c: f"case{c['i']}")
def test_linear_random_shape(c):
    print(f"case {c}", flush=True)
    M, K, N = c["M"], c["K"], c["N"]
    inp = synth.linear_inputs(synth.small_case(f"r{c['i']}", 5000 + c["i"], M, K, N,
                                               subnormal_frac=c["sub"], swiglu=c["swiglu"]))
    epi = brl.EPILOGUE_SWIGLU if c["swiglu"] else brl.EPILOGUE_NONE
    add = None
    if c["addend"]:
        add = np.random.default_rng(c["i"]).standard_normal((M, N)).astype(np.float32)
    X, W = _cuda(inp.X), _cuda(inp.W)
    Y, Ypre, s_w = brl.qat_linear_fwd(X, W, synth.S_X, addend=None if add is None else _cuda(add),
                                      epilogue=epi, tune=brl.Tuning(fwd_prep=c["fwd_prep"]))
    _same(s_w, np.array([oracle.weight_scale(inp.W)]), "s_w", c)
    if c["swiglu"]:
        wY, wPre = oracle.linear_fwd(inp.X, inp.W, synth.S_X, epilogue=1)
        _same(Ypre, wPre, "Ypre", c)
        G = oracle.swiglu_bwd(wPre, inp.dY)
    else:
        wY = oracle.linear_fwd(inp.X, inp.W, synth.S_X, addend=add)
        G = inp.dY
    _same(Y, wY, "Y", c)

    tune = brl.Tuning(bwd_engine=c["engine"], bwd_chunk_log2=c["chunk"])
    dY = _cuda(inp.dY)
    wX, wW = oracle.linear_bwd(G, inp.X, inp.W, synth.S_X)
    dX, dW = brl.qat_linear_bwd(dY, X, W, synth.S_X, Ypre=Ypre, epilogue=epi, tune=tune)
    _same(dX, wX, "dX", c)
    _same(dW, wW, "dW", c)
    if c["acc"]:
        # the running sum: dW + dW is one binary32 add per element
        brl.qat_linear_bwd(dY, X, W, synth.S_X, Ypre=Ypre, epilogue=epi, need_dX=False, dW=dW,
                           dW_accumulate=True, tune=tune)
        _same(dW, np.float32(wW + wW), "dW accumulated", c)
