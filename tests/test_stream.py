"""The library's data stream (host code behind the C ABI) against the
oracle, token for token: windows, rank shares, resume records; plus argument
checks.  Runs on the CPU (no device calls)."""
import struct

import numpy as np
import pytest

import bitwise_reproducible_lsq_amd as brl
import synth
from oracle import datastream as ds


def _both(seed, scale=1):
    corpus = synth.corpus(7, scale)
    lib = brl.DataStream(seed, synth.SEPARATOR, corpus)
    orc = ds.Stream(seed, [ds.Source(n, w, sh) for n, w, sh in corpus], synth.SEPARATOR)
    return lib, orc, corpus


@pytest.mark.parametrize("seed", [0, 11, 2 ** 40 + 3])
def test_windows_match_the_oracle(seed):
    lib, orc, _ = _both(seed)
    first, got = lib.next(25)
    assert first == 0
    want = np.array([orc.next_window()[1] for _ in range(25)], np.int32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("ranks", [1, 2, 3, 4])
def test_rank_shares_match_the_oracle(ranks):
    for rank in range(ranks):
        lib, orc, _ = _both(5)
        for _ in range(3):
            got = lib.step(4 * ranks, ranks, rank)
            want = np.array(orc.step(4 * ranks, ranks, rank), np.int32)
            assert np.array_equal(got, want)


def test_record_matches_the_oracle_and_resumes():
    lib, orc, corpus = _both(21)
    lib.next(13)
    for _ in range(13):
        orc.next_window()
    rec = lib.save()
    o = orc.record()
    assert rec[:8] == b"BRLSTRM1"
    seed, nsrc, sep, window, mix = struct.unpack_from("<QIiQQ", rec, 8)
    assert (seed, nsrc, sep, window, mix) == (21, len(corpus), synth.SEPARATOR, o.window, o.mix_draws)
    off = 8 + 32
    for k, (name, _, _) in enumerate(corpus):
        assert rec[off:off + 32] == ds.source_digest(name)
        e, sp, dp, cons = struct.unpack_from("<QQQQ", rec, off + 32)
        st = o.sources[k]
        assert (e, sp, dp, cons) == (st.epoch, st.shard_pos, st.doc_pos, st.consumed)
        off += 64
    nbuf = struct.unpack_from("<Q", rec, off)[0]
    assert list(np.frombuffer(rec[off + 8:], "<i4")) == o.buffer and nbuf == len(o.buffer)
    # resume: a fresh stream loaded with the record continues identically
    cont = lib.next(7)[1]
    fresh = brl.DataStream(21, synth.SEPARATOR, corpus)
    fresh.load(rec)
    assert np.array_equal(fresh.next(7)[1], cont)


def test_epochs_roll_over_like_the_oracle():
    """A small corpus drawn far past its size (several epochs per source)."""
    corpus = [(n, w, [sh[:2] for sh in shards]) for n, w, shards in synth.corpus(3)]
    lib = brl.DataStream(4, synth.SEPARATOR, corpus)
    orc = ds.Stream(4, [ds.Source(n, w, sh) for n, w, sh in corpus], synth.SEPARATOR)
    got = lib.next(60)[1]
    want = np.array([orc.next_window()[1] for _ in range(60)], np.int32)
    assert np.array_equal(got, want)
    assert max(s.epoch for s in orc.record().sources) >= 2


def test_bad_arguments():
    corpus = synth.corpus(7)
    with pytest.raises(brl.BrlError):
        brl.DataStream(1, 0, [("x", 1, [[]])])                       # weighted source without documents
    with pytest.raises(brl.BrlError):
        brl.DataStream(1, 0, [(n, 0, sh) for n, _, sh in corpus])     # zero total weight
    s = brl.DataStream(1, 0, corpus)
    with pytest.raises(brl.BrlError):
        s.step(5, 2, 0)                                              # batch not a multiple of ranks
    with pytest.raises(brl.BrlError):
        s.step(4, 2, 2)                                              # rank out of range
    other = brl.DataStream(2, 0, corpus)
    with pytest.raises(brl.BrlError):
        s.load(other.save())                                         # record of another seed
    with pytest.raises(brl.BrlError):
        s.load(b"not a record")


def test_resume_with_a_different_rank_count():
    """Elastic resume: four ranks each walk the global stream for two
    batches of 8 windows and keep windows m with m mod 4 = r; their resume
    records are byte-identical; two ranks loaded with that record continue
    with windows m mod 2 = r of the same global stream."""
    corpus = synth.corpus(7, 1)
    G = 8
    _, ref = brl.DataStream(33, synth.SEPARATOR, corpus).next(5 * G)
    records = []
    for r in range(4):
        st = brl.DataStream(33, synth.SEPARATOR, corpus)
        got = np.concatenate([st.step(G, 4, r) for _ in range(2)])
        assert np.array_equal(got, ref[:2 * G][r::4])
        records.append(st.save())
        st.close()
    assert all(rec == records[0] for rec in records)
    for r in range(2):
        st = brl.DataStream(33, synth.SEPARATOR, corpus)
        st.load(records[0])
        got = np.concatenate([st.step(G, 2, r) for _ in range(3)])
        assert np.array_equal(got, ref[2 * G:][r::2])
        st.close()
