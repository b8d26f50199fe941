"""Device counter-based draws (brl_philox_u32) against the oracle's
Philox4x32-10: every value is a pure function of (key, stream, position), so
any window of positions, any alignment and any launch gives the same words."""
import json
import os

import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
from oracle import datastream as ds

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _draws(key, stream, first, n):
    t = brl.philox_u32(key, stream, first, n)
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint32)


def test_known_answer_block():
    kat = json.load(open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")))["vectors"][0]
    assert list(_draws(0, 0, 0, 4)) == [int(x, 16) for x in kat["out"]]


@pytest.mark.parametrize("key,stream,first,n", [
    (0x0123456789ABCDEF, 0, 0, 1000),
    (7, 0x6D6978, 3, 517),                 # unaligned start and end
    (2 ** 64 - 1, 5, 2 ** 34 + 1, 300),    # positions past 2^32 blocks
    (42, 1, 1, 1),
])
def test_draws_match_the_oracle(key, stream, first, n):
    got = _draws(key, stream, first, n)
    want = np.array([ds.u32(key, stream, first + k) for k in range(n)], np.uint32)
    assert np.array_equal(got, want)


def test_windows_agree_with_one_long_launch():
    key, stream = 99, 3
    whole = _draws(key, stream, 0, 1 << 20)
    for first, n in [(0, 5), (13, 1000), (4096, 4096), ((1 << 20) - 7, 7)]:
        assert np.array_equal(_draws(key, stream, first, n), whole[first:first + n])
    out = torch.empty(1001, dtype=torch.int32, device="cuda")
    brl.philox_u32(key, stream, 10, 1000, out=out[1:])        # 4-byte but not 16-byte aligned
    torch.cuda.synchronize()
    assert np.array_equal(out[1:].cpu().numpy().view(np.uint32), whole[10:1010])
