"""Pins of the data-stream oracle (onedev.kr summary, "How": counter-based
Philox random numbers; "What differs": the topology-invariant stream, window
assignment m mod R = r, the rank-independent resume record)."""
import json
import os
import itertools

import numpy as np
import pytest

import synth
from oracle import datastream as ds

HERE = os.path.dirname(os.path.abspath(__file__))


def _sources(scale=1):
    return [ds.Source(n, w, shards) for n, w, shards in synth.corpus(7, scale)]


def test_philox_known_answers():
    kat = json.load(open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")))
    for v in kat["vectors"]:
        ctr = tuple(int(x, 16) for x in v["counter"])
        key = tuple(int(x, 16) for x in v["key"])
        assert ds.philox4x32(ctr, key) == tuple(int(x, 16) for x in v["out"])


def test_draws_are_pure_functions_of_the_position():
    key, stream = 0x0123456789ABCDEF, 5
    a = [ds.u32(key, stream, i) for i in range(40)]
    b = [ds.u32(key, stream, i) for i in reversed(range(40))][::-1]
    assert a == b
    blk = ds.philox4x32((2, 0, stream, 0), (key & ds.MASK, key >> 32))
    assert a[8:12] == list(blk)
    assert [ds.u32(key, stream + 1, i) for i in range(8)] != a[:8]


def test_bounded_and_permutations():
    for n in (1, 2, 3, 7, 100):
        for key in range(20):
            p = ds.permutation(key, n)
            assert sorted(p) == list(range(n))
    assert all(0 <= ds.bounded(x, 5) < 5 for x in (0, 1, 2 ** 31, 2 ** 32 - 1))
    # all 24 orders of 4 items appear with about equal frequency over many keys
    counts = {}
    for key in range(24 * 200):
        p = ds.permutation(key * 7919 + 3, 4)
        counts[p] = counts.get(p, 0) + 1
    assert len(counts) == 24
    chi2 = sum((c - 200) ** 2 / 200 for c in counts.values())
    assert chi2 < 60          # 23 degrees of freedom: p < 1e-4 beyond this


def test_windows_are_the_documents_joined_by_the_separator():
    """Re-derive the token stream from the selection rule written out here
    (mix draw -> source, shard and document permutations) and compare."""
    src = _sources()
    st = ds.Stream(11, src, synth.SEPARATOR)
    wins = [st.next_window()[1] for _ in range(12)]
    flat = list(itertools.chain.from_iterable(wins))
    # independent walk
    total = sum(s.weight for s in src)
    pos = [[0, 0, 0] for _ in src]      # epoch, shard_pos, doc_pos
    out, t = [], 0
    while len(out) < len(flat):
        r = (ds.u32(11, ds.MIX_STREAM, t) * total) >> 32
        t += 1
        k = next(i for i, c in enumerate(np.cumsum([s.weight for s in src])) if r < c)
        e, sp, dp = pos[k]
        shards = src[k].shards
        if sp == len(shards):
            e, sp = e + 1, 0
        sh = ds.permutation(ds.shard_key(11, src[k].name, e), len(shards))[sp]
        d = ds.permutation(ds.doc_key(11, src[k].name, e, sh), len(shards[sh]))[dp]
        dp += 1
        if dp == len(shards[sh]):
            dp, sp = 0, sp + 1
        pos[k] = [e, sp, dp]
        out.extend(int(x) for x in shards[sh][d])
        out.append(synth.SEPARATOR)
    assert out[:len(flat)] == flat
    assert all(len(w) == ds.WINDOW for w in wins)


@pytest.mark.parametrize("ranks", [1, 2, 3, 6])
def test_rank_streams_partition_the_global_stream(ranks):
    """Any rank count sees the same windows: rank r gets exactly those with
    m mod R = r, and interleaving the ranks' windows rebuilds the stream."""
    M = 6
    ref = ds.Stream(3, _sources(), synth.SEPARATOR)
    glob = [ref.next_window()[1] for _ in range(2 * M)]
    per_rank = []
    for r in range(ranks):
        st = ds.Stream(3, _sources(), synth.SEPARATOR)
        per_rank.append(st.step(M, ranks, r) + st.step(M, ranks, r))
    for r in range(ranks):
        assert per_rank[r] == [glob[m] for m in range(2 * M) if m % ranks == r]
    with pytest.raises(ValueError):
        ds.Stream(3, _sources(), synth.SEPARATOR).step(M, 4, 0)


def test_resume_record_reproduces_the_rest_of_the_stream():
    st = ds.Stream(5, _sources(), synth.SEPARATOR)
    for _ in range(7):
        st.next_window()
    rec = st.record()
    assert rec.window == 7
    cont = [st.next_window() for _ in range(9)]
    resumed = ds.Stream(5, _sources(), synth.SEPARATOR, record=rec)
    assert [resumed.next_window() for _ in range(9)] == cont


def test_epochs_visit_every_document_once():
    """A source drawn until it wraps: each epoch takes every document exactly
    once, and the next epoch's order differs."""
    rng = np.random.default_rng(1)
    shards = [[rng.integers(1, 100, 5).astype(np.int32) + 1000 * (10 * s + d) for d in range(n)]
              for s, n in enumerate([3, 0, 4, 2])]
    st = ds.Stream(9, [ds.Source("tiny", 1, shards)], synth.SEPARATOR)
    seen = [st._next_document(0)[0] // 1000 for _ in range(18)]
    assert sorted(seen[:9]) == sorted(seen[9:]) == sorted(10 * s + d for s, n in enumerate([3, 0, 4, 2])
                                                          for d in range(n))
    assert seen[:9] != seen[9:]
    # the epoch advances when the next document is drawn (lazily)
    assert (st.rec.sources[0].epoch, st.rec.sources[0].shard_pos, st.rec.sources[0].consumed) == (1, 4, 18)


def test_source_proportions_follow_the_weights():
    src = [ds.Source(f"s{k}", w, [[np.array([k + 1], np.int32)] * 50]) for k, w in enumerate([6, 3, 1])]
    st = ds.Stream(2, src, synth.SEPARATOR)
    counts = np.zeros(3)
    for _ in range(3000):
        counts[st._pick_source()] += 1
    assert np.allclose(counts / 3000, [0.6, 0.3, 0.1], atol=0.03)


def test_orders_depend_on_the_source_name_digest():
    assert ds.shard_key(1, "web", 0) != ds.shard_key(1, "code", 0)
    assert ds.shard_key(1, "web", 0) != ds.shard_key(1, "web", 1)
    assert ds.doc_key(1, "web", 0, 0) != ds.doc_key(1, "web", 0, 1)
    assert ds.shard_key(1, "web", 0) == ds.shard_key(1, "web", 0)
