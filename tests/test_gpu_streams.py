"""Calls on two streams at once.  The library keeps no state between calls
and every call takes a workspace of its own, so two forward + backward
sequences of different layers issued on two streams without any
synchronisation between them must each give the oracle's bits."""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import oracle
import synth

pytestmark = pytest.mark.gpu


def _bits(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def test_forward_backward_on_two_streams_at_once():
    dev = "cuda"
    cases = [synth.small_case("stream_a", 21, 768, 256, 384), synth.small_case("stream_b", 22, 640, 192, 512)]
    inps = [synth.linear_inputs(c) for c in cases]
    want = []
    for inp in inps:
        Y = oracle.linear_fwd(inp.X, inp.W, synth.S_X)
        dX, dW = oracle.linear_bwd(inp.dY, inp.X, inp.W, synth.S_X)
        want.append((Y, dX, dW))
    dev_in = [[torch.from_numpy(np.ascontiguousarray(t)).to(dev) for t in (inp.X, inp.W, inp.dY)] for inp in inps]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = [[], []]
    # interleave the issue of the two sequences, several rounds, no waits between the streams
    for rnd in range(3):
        for i in (0, 1):
            X, W, dY = dev_in[i]
            s = streams[i]
            with torch.cuda.stream(s):
                Y, _, _ = brl.qat_linear_fwd(X, W, synth.S_X, stream=s)
                dX, dW = brl.qat_linear_bwd(dY, X, W, synth.S_X, stream=s)
            outs[i].append((Y, dX, dW))
    torch.cuda.synchronize()
    for i in (0, 1):
        for rnd, (Y, dX, dW) in enumerate(outs[i]):
            for name, got, w in zip(("Y", "dX", "dW"), (Y, dX, dW), want[i]):
                assert np.array_equal(_bits(got), _bits(w)), f"stream {i} round {rnd}: {name} differs"
