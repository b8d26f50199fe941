"""grad_l2norm_clip_noalloc (the norm and clip for callers that cannot
allocate) against grad_l2norm_clip with a caller workspace, through the C
ABI: the clipped gradient and the norm bit for bit, on several calls in a
row on one device (the library's scratch array keeps the previous call's
contents), each later call smaller than the one before, with the clip active
and inactive, lengths with a ragged tail, and one length whose CanonSum
takes an extra coalesced pass before its tail pass."""
import ctypes as C

import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _pair(n, scale, seed, max_norm=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(n, generator=g, device="cuda") * scale
    a, b = x.clone(), x.clone()
    nu_ref = brl.grad_l2norm_clip(a, max_norm)
    nu = brl.grad_l2norm_clip_noalloc(b, max_norm)
    torch.cuda.synchronize()
    return a, nu_ref, b, nu


@pytest.mark.parametrize("sizes", [[5_000_003, 100_003], [2 ** 27 + 12_345, 64 * 32 * 2401 + 35, 1]])
def test_noalloc_matches_workspace_entry_point(sizes):
    for k, n in enumerate(sizes):
        # first call: the clip is active; later calls: alternately inactive
        scale = 1e-2 if k % 2 == 0 else 1e-7
        a, nu_ref, b, nu = _pair(n, scale, seed=1000 + k + n % 97)
        assert np.array_equal(_bits(nu), _bits(nu_ref)), (n, nu.item(), nu_ref.item())
        assert np.array_equal(_bits(b), _bits(a)), f"clipped gradient differs at n={n}"
        if k == 0:
            assert nu_ref.item() > 1.0          # the first call clips


def test_noalloc_rejects_lengths_beyond_its_scratch():
    L = brl.lib()
    g = torch.zeros(16, device="cuda")
    nu = torch.zeros(1, device="cuda")
    st = L.grad_l2norm_clip_noalloc(C.c_void_p(g.data_ptr()), brl.NOALLOC_NORM_MAX_LEN + 1, 1.0, 0.0,
                                    C.c_void_p(nu.data_ptr()), None, None)
    assert st == brl.BRL_ESHAPE
    assert b"scratch" in L.brl_last_error()
    # nothing ran: the buffers are untouched
    torch.cuda.synchronize()
    assert torch.all(g == 0) and torch.all(nu == 0)
