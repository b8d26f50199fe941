"""GPU parity of brl_state_hash against the hashlib-based oracle: leaf and
tail boundaries, several tensors (and more than one leaf launch), empty
tensors, 4-byte-aligned sources, multi-level trees, and a state of several
GB.  Every digest must equal the oracle's bytes."""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
from oracle import state_hash as sh

pytestmark = pytest.mark.gpu


def _dev_bytes(n, seed):
    g = np.random.default_rng(seed)
    host = g.integers(0, 256, n, dtype=np.uint8)
    return host, torch.from_numpy(host).cuda()


def _digest(ts):
    d = brl.state_hash(ts)
    torch.cuda.synchronize()
    return bytes(d.cpu().numpy().tobytes())


SIZES = [0, 1, 3, 4, 55, 56, 63, 64, 65, 119, 120, 4095, 4096, 4097, 16384, 17 * 4096 + 77, (1 << 20) + 12345]


@pytest.mark.parametrize("n", SIZES)
def test_single_tensor(n):
    host, dev = _dev_bytes(n, n)
    assert _digest([dev]) == sh.state_hash([host])


def test_several_tensors_with_empty_ones():
    parts = [_dev_bytes(n, 100 + i) for i, n in enumerate([100, 0, 4096, 5, 0, 40000, 64])]
    assert _digest([d for _, d in parts]) == sh.state_hash([h for h, _ in parts])


def test_more_tensors_than_one_leaf_launch():
    g = np.random.default_rng(7)
    sizes = [int(v) for v in g.integers(0, 20000, 150)]
    parts = [_dev_bytes(n, 1000 + i) for i, n in enumerate(sizes)]
    assert _digest([d for _, d in parts]) == sh.state_hash([h for h, _ in parts])


def test_four_byte_aligned_sources_hash_the_same():
    host, dev = _dev_bytes(200004, 11)
    view = dev[4:]                      # 4-byte but not 16-byte aligned
    assert view.data_ptr() % 16 != 0
    assert _digest([view]) == sh.state_hash([host[4:]])
    assert _digest([view, dev[:4]]) == sh.state_hash([host[4:], host[:4]])


def test_float_tensors_hash_their_raw_bytes():
    x = torch.randn(3000, 77, device="cuda")
    y = torch.randn(5, dtype=torch.float64, device="cuda")
    assert _digest([x, y]) == sh.state_hash([x.cpu().numpy(), y.cpu().numpy()])


def test_deep_tree():
    # 512 MiB + 1 byte: 131073 leaves -> 8193 -> 513 -> 33 -> 3 -> 1 -> root
    host, dev = _dev_bytes((1 << 29) + 1, 21)
    assert _digest([dev]) == sh.state_hash([host])


def test_repeat_and_stream_independence():
    host, dev = _dev_bytes(1 << 22, 31)
    want = sh.state_hash([host])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d = brl.state_hash([dev])
    s.synchronize()
    assert bytes(d.cpu().numpy().tobytes()) == want
    assert _digest([dev]) == want
