"""Pins of the state-hash oracle (oracle/state_hash.py) -- CPU only.

The tree is pinned against its special cases that reduce to plain SHA-256
of a spelled-out message (one leaf; two leaves under one node; 17 leaves
under two levels), and against sensitivity: any changed byte, a byte moved
between tensors, the tensor order, an appended empty tensor all change the
root."""
import hashlib
import struct

import numpy as np
import pytest

from oracle import state_hash as sh


def H(b):
    return hashlib.sha256(b).digest()


def tail(lens):
    return struct.pack("<q", len(lens)) + b"".join(struct.pack("<q", n) for n in lens) + b"\x02"


@pytest.mark.parametrize("n", [0, 1, 55, 56, 63, 64, 1000, 4096])
def test_single_leaf_state(n):
    data = bytes((7 * i + 3) & 0xFF for i in range(n))
    assert sh.state_hash([data]) == H(H(data + b"\x00") + tail([n]))


def test_two_leaves_one_node():
    data = bytes(np.random.default_rng(1).integers(0, 256, 4097, dtype=np.uint8))
    l0, l1 = H(data[:4096] + b"\x00"), H(data[4096:] + b"\x00")
    assert sh.state_hash([data]) == H(H(l0 + l1 + b"\x01") + tail([4097]))


def test_leaves_of_several_tensors_in_order():
    a, b = b"\x01" * 100, b"\x02" * 4096 * 2
    la = H(a + b"\x00")
    lb0, lb1 = H(b[:4096] + b"\x00"), H(b[4096:] + b"\x00")
    assert sh.state_hash([a, b]) == H(H(la + lb0 + lb1 + b"\x01") + tail([100, 8192]))


def test_two_levels_for_17_leaves():
    data = bytes(np.random.default_rng(2).integers(0, 256, 17 * 4096 - 5, dtype=np.uint8))
    leaves = [H(data[o:o + 4096] + b"\x00") for o in range(0, len(data), 4096)]
    assert len(leaves) == 17
    n0 = H(b"".join(leaves[:16]) + b"\x01")
    n1 = H(leaves[16] + b"\x01")
    assert sh.state_hash([data]) == H(H(n0 + n1 + b"\x01") + tail([len(data)]))


def test_sensitivity():
    g = np.random.default_rng(3)
    a = bytearray(g.integers(0, 256, 40000, dtype=np.uint8).tobytes())
    b = bytearray(g.integers(0, 256, 5000, dtype=np.uint8).tobytes())
    base = sh.state_hash([bytes(a), bytes(b)])
    seen = {base}
    for pos in list(g.integers(0, len(a), 24)) + [0, len(a) - 1, 4095, 4096, 32768]:
        m = bytearray(a)
        m[pos] ^= 1 << int(g.integers(0, 8))
        d = sh.state_hash([bytes(m), bytes(b)])
        assert d not in seen
        seen.add(d)
    assert sh.state_hash([bytes(a[:-1]), bytes(a[-1:] + b)]) != base      # a byte moved across tensors
    assert sh.state_hash([bytes(b), bytes(a)]) != base                     # order
    assert sh.state_hash([bytes(a), bytes(b), b""]) != base                # an extra empty tensor


def test_numpy_arrays_hash_as_their_bytes():
    x = np.arange(5000, dtype=np.float32)
    assert sh.state_hash([x]) == sh.state_hash([x.tobytes()])
