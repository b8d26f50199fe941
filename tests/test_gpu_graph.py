"""The library's calls are kernels only (no allocation, copy, fill or host
synchronisation inside), so a HIP graph can capture them.  One graph holds
the linear forward and backward and the attention forward with its three
gradients.  It is replayed three times, with eager work between the replays
that overwrites its outputs and runs the forward on other inputs (with a
workspace of its own: the binding takes one per call, and the graph keeps
the ones it captured), and every replay must equal the eager results bit
for bit."""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import synth

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def test_linear_and_attention_replay_in_a_hip_graph():
    dev = "cuda"
    case = synth.small_case("graph", 5, 192, 160, 96)
    inp = synth.linear_inputs(case)
    X, W, dY = (torch.from_numpy(np.ascontiguousarray(t)).to(dev) for t in (inp.X, inp.W, inp.dY))
    g = np.random.default_rng(6)
    B, S, Hq, Hkv, D, window, s_v = 1, 90, 4, 2, 128, 40, 0.05
    q = torch.from_numpy((g.standard_normal((B, S, Hq, D)) * 0.3).astype(np.float32)).to(dev)
    k = torch.from_numpy(g.standard_normal((B, S, Hkv, D)).astype(np.float32)).to(dev)
    v = torch.from_numpy(g.standard_normal((B, S, Hkv, D)).astype(np.float32)).to(dev)
    go = torch.from_numpy((g.standard_normal((B, S, Hq, D)) * 1e-2).astype(np.float32)).to(dev)

    def run():
        Y, _, _ = brl.qat_linear_fwd(X, W, synth.S_X)
        dX, dW = brl.qat_linear_bwd(dY, X, W, synth.S_X)
        stats = torch.empty((B, S, Hq, 2), dtype=torch.float32, device=dev)
        O = brl.attn_fwd(q, k, v, window, s_v, stats=stats)
        dQ = brl.attn_bwd_dq(q, k, v, O, go, stats, window, s_v)
        dK, dV = brl.attn_bwd_dkdv(q, k, v, O, go, stats, window, s_v)
        return [Y, dX, dW, O, dQ, dK, dV]

    eager = [_bits(t) for t in run()]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    torch.cuda.synchronize()

    other = synth.linear_inputs(synth.small_case("graph_other", 9, 192, 160, 96))
    Xo = torch.from_numpy(np.ascontiguousarray(other.X)).to(dev)
    Wo = torch.from_numpy(np.ascontiguousarray(other.W)).to(dev)
    for rep in range(3):
        for t in outs:
            t.fill_(7.0)
        brl.qat_linear_fwd(Xo, Wo, synth.S_X)          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, want in zip(["Y", "dX", "dW", "O", "dQ", "dK", "dV"], outs, eager):
            got = _bits(t)
            assert np.array_equal(got, want), f"replay {rep}: {name} differs from the eager result"
