"""Topology-invariant data stream (oracle; TEST INFRASTRUCTURE ONLY -- the
product path never imports this module).

Follows the Open-1B summary on onedev.kr, section "How" (counter-based
random numbers: each value a pure function of the seed and a fixed logical
position, Philox) and section "What differs" (the data stream):
  * one canonical stream, independent of world size, rank and node count;
  * three generators: source interleaving from a global mix generator seeded
    by the training seed alone; shard order seeded by (seed, SHA-256 of the
    source name, epoch); document order seeded by (seed, SHA-256 of the
    source name, epoch, shard);
  * selected documents joined with a separator token into one flat token
    buffer, cut from the front into windows of 4,097 tokens (inputs + labels);
  * data parallelism after the stream: rank r of R owns windows m with
    m mod R = r; the global batch must be a multiple of R;
  * a rank-independent resume record: documents consumed per source, epoch
    counters, the mix generator's state, the partial window in the packing
    buffer.
Where the pages stop, this module takes its own readings, stated where they
are used: how a tuple becomes a Philox key, how draws become bounded
integers and permutations, how sources are weighted.

Philox4x32-10 is written from its published definition (Salmon, Moraes, Dror
and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds
of two 32x32->64 multiplies by 0xD2511F53 and 0xCD9E8D57 with the key bumped
by the Weyl constants 0x9E3779B9, 0xBB67AE85 between rounds.
"""
from __future__ import annotations

import functools
import hashlib
import struct
from dataclasses import dataclass, field

WINDOW = 4097
MASK = 0xFFFFFFFF
_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
MIX_STREAM = 0x6D6978          # "mix"


def philox4x32(ctr, key, rounds: int = 10):
    """One Philox4x32 block: 4 counter words and 2 key words -> 4 words."""
    c0, c1, c2, c3 = ctr
    k0, k1 = key
    for r in range(rounds):
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK, p1 & MASK, ((p0 >> 32) ^ c3 ^ k1) & MASK, p0 & MASK
        if r < rounds - 1:
            k0, k1 = (k0 + _W0) & MASK, (k1 + _W1) & MASK
    return c0, c1, c2, c3


def u32(key: int, stream: int, i: int) -> int:
    """32-bit draw at logical position i of (key, stream): word i mod 4 of
    the block with counter (i div 4 as 64 bits, stream, 0)."""
    blk = i >> 2
    out = philox4x32((blk & MASK, (blk >> 32) & MASK, stream & MASK, 0), (key & MASK, (key >> 32) & MASK))
    return out[i & 3]


def bounded(x: int, n: int) -> int:
    """Integer in [0, n) from a 32-bit draw: (x * n) >> 32 (no rejection;
    the bias is below n / 2^32)."""
    return (x * n) >> 32


@functools.lru_cache(maxsize=4096)
def permutation(key: int, n: int):
    """Fisher-Yates from the top: draw t (t = 0 .. n-2) swaps position
    k = n-1-t with bounded(draw, k+1)."""
    p = list(range(n))
    for t in range(n - 1):
        k = n - 1 - t
        j = bounded(u32(key, 0, t), k + 1)
        p[k], p[j] = p[j], p[k]
    return tuple(p)


def _le64(x: int) -> bytes:
    return struct.pack("<Q", x & 0xFFFFFFFFFFFFFFFF)


def source_digest(name: str) -> bytes:
    return hashlib.sha256(name.encode("utf-8")).digest()


def shard_key(seed: int, name: str, epoch: int) -> int:
    h = hashlib.sha256(b"shard" + _le64(seed) + source_digest(name) + _le64(epoch)).digest()
    return struct.unpack("<Q", h[:8])[0]


def doc_key(seed: int, name: str, epoch: int, shard: int) -> int:
    h = hashlib.sha256(b"doc" + _le64(seed) + source_digest(name) + _le64(epoch) + _le64(shard)).digest()
    return struct.unpack("<Q", h[:8])[0]


@dataclass
class Source:
    name: str
    weight: int
    shards: list            # shards[k] = list of documents (each a list/array of token ids)


@dataclass
class SourceState:
    epoch: int = 0
    shard_pos: int = 0
    doc_pos: int = 0
    consumed: int = 0


@dataclass
class Record:
    """Rank-independent resume record."""
    window: int = 0                     # index of the next window to emit
    mix_draws: int = 0                  # draws taken from the mix generator
    sources: list = field(default_factory=list)   # SourceState per source
    buffer: list = field(default_factory=list)    # packed tokens not yet in a window


class Stream:
    def __init__(self, seed: int, sources, separator: int, record: Record | None = None):
        self.seed, self.sources, self.sep = seed, sources, separator
        self.cum = []
        t = 0
        for s in sources:
            t += s.weight
            self.cum.append(t)
        self.total = t
        if t <= 0:
            raise ValueError("the source weights must add up to a positive number")
        for src in sources:
            if src.weight < 0 or (src.weight > 0 and not any(len(d) for d in src.shards)):
                raise ValueError(f"source {src.name}: negative weight or no documents")
        self.rec = record if record is not None else Record(sources=[SourceState() for _ in sources])

    def _pick_source(self) -> int:
        r = bounded(u32(self.seed, MIX_STREAM, self.rec.mix_draws), self.total)
        self.rec.mix_draws += 1
        for k, c in enumerate(self.cum):
            if r < c:
                return k
        raise AssertionError("unreachable")

    def _next_document(self, k: int):
        src, st = self.sources[k], self.rec.sources[k]
        while True:
            if st.shard_pos == len(src.shards):
                st.epoch += 1
                st.shard_pos = 0
            shard = permutation(shard_key(self.seed, src.name, st.epoch), len(src.shards))[st.shard_pos]
            docs = src.shards[shard]
            if st.doc_pos < len(docs):
                doc = permutation(doc_key(self.seed, src.name, st.epoch, shard), len(docs))[st.doc_pos]
                st.doc_pos += 1
                st.consumed += 1
                if st.doc_pos == len(docs):
                    st.doc_pos, st.shard_pos = 0, st.shard_pos + 1
                return docs[doc]
            st.doc_pos, st.shard_pos = 0, st.shard_pos + 1

    def next_window(self):
        """The next window of the global stream: (index m, WINDOW tokens)."""
        while len(self.rec.buffer) < WINDOW:
            k = self._pick_source()
            self.rec.buffer.extend(int(x) for x in self._next_document(k))
            self.rec.buffer.append(self.sep)
        w = self.rec.buffer[:WINDOW]
        del self.rec.buffer[:WINDOW]
        m = self.rec.window
        self.rec.window += 1
        return m, w

    def step(self, global_batch: int, ranks: int, rank: int):
        """Advance by one global batch; return rank's windows (m mod R == rank)."""
        if global_batch % ranks:
            raise ValueError("the global batch must be a multiple of the rank count")
        out = []
        for _ in range(global_batch):
            m, w = self.next_window()
            if m % ranks == rank:
                out.append(w)
        return out

    def record(self) -> Record:
        r = self.rec
        return Record(r.window, r.mix_draws, [SourceState(s.epoch, s.shard_pos, s.doc_pos, s.consumed)
                                             for s in r.sources], list(r.buffer))
