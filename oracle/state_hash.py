"""CPU oracle of the per-step state hash (TEST INFRASTRUCTURE ONLY: used by
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg).

The pages fix that a hash of the training state is stored after every step,
that a replayed step must reproduce it (rit.work article body; onedev.kr
summary, section "Use"), and that hashing on the host costs about 6 s per
step, with on-device hashing named as the way to remove that cost (onedev.kr,
section "Limits", limitations paragraph).  They do not name the function
(SHA-256 is named only for hashing data-source names, section "How", data
stream paragraph).  Reading taken here: SHA-256 (FIPS 180-4, Python's
``hashlib``) arranged as a tree so that a GPU can hash in parallel:

* the state is an ordered list of tensors, each taken as its raw bytes
  (little-endian, row-major);
* each tensor is cut into consecutive 4 KiB leaves (the last may be shorter;
  an empty tensor has one empty leaf); leaf digest = SHA-256(bytes || 0x00);
* the leaf digests of all tensors, tensor after tensor, form level 0; each
  higher level hashes consecutive groups of 16 digests (512 bytes) as
  SHA-256(digests || 0x01) until one digest remains;
* state hash = SHA-256(top || le64(tensor count) || le64(byte length of each
  tensor, in order) || 0x02).

Written level by level from that description; nothing here is shared with the
GPU code.
"""
from __future__ import annotations

import hashlib
import struct
from typing import Iterable, List

LEAF_BYTES = 4096
FAN_IN = 16


def _sha(data: bytes) -> bytes:
    return hashlib.sha256(data).digest()


def _leaf(chunk) -> bytes:
    h = hashlib.sha256(chunk)
    h.update(b"\x00")
    return h.digest()


def leaf_digests(tensor: memoryview) -> List[bytes]:
    """SHA-256(chunk || 0x00) of each 4 KiB chunk of one tensor's bytes."""
    if len(tensor) == 0:
        return [_leaf(b"")]
    return [_leaf(tensor[o:o + LEAF_BYTES]) for o in range(0, len(tensor), LEAF_BYTES)]


def tree_top(level: List[bytes]) -> bytes:
    """Hash groups of FAN_IN digests (|| 0x01) until one digest remains."""
    while len(level) > 1:
        level = [_sha(b"".join(level[o:o + FAN_IN]) + b"\x01") for o in range(0, len(level), FAN_IN)]
    return level[0]


def state_hash(tensors: Iterable) -> bytes:
    """The state hash of an ordered list of tensors (bytes-like or numpy arrays)."""
    blobs = [memoryview(t).cast("B") for t in tensors]
    if not blobs:
        raise ValueError("the state has at least one tensor")
    level = []
    for b in blobs:
        level.extend(leaf_digests(b))
    top = tree_top(level)
    tail = struct.pack("<q", len(blobs)) + b"".join(struct.pack("<q", len(b)) for b in blobs) + b"\x02"
    return _sha(top + tail)
