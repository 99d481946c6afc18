"""Oracle pins: clamps, batch intake, split_simple, split_equal, output_ids.

Expected values come from tests/golden/page_numbers.json (numbers the pages
print, with citations) or from closed forms stated in each test.
"""

import json
import os

import numpy as np
import pytest

from oracle import batching as B
from oracle import OracleEngine, SplitError

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def chunk_calls(n, n_batch):
    return [min(n_batch, n - a) for a in range(0, n, n_batch)]


def test_caller_chunking_and_split_simple_5000():
    g = GOLD["caller_chunking"]
    nb, nub = B.clamp_params(1 << 20, g["n_batch"], g["n_ubatch"])
    calls = chunk_calls(g["n_tokens"], nb)
    assert calls == g["calls"]
    per_call = [len(B.split_batch([{0}] * n, nub, 1)) for n in calls]
    assert per_call == g["ubatches_per_call"]
    assert sum(per_call) == g["forward_passes"]


def test_split_simple_page_examples():
    g = GOLD["split_simple_1000"]
    sizes = [len(s) for (s, _, _) in B.split_batch([{0}] * g["n_tokens"], g["n_ubatch"], 1)]
    assert sizes == g["sizes"]
    g = GOLD["split_simple_1500"]
    parts = B.split_batch([{0}] * g["n_tokens"], g["n_ubatch"], 1)
    assert [len(s) for (s, _, _) in parts] == g["sizes"]
    assert [[s[0], s[-1]] for (s, _, _) in parts] == g["ranges"]


def test_split_simple_ignores_sequence_ids():
    # slots of three sequences interleaved are taken purely in submission order
    sets = [{i % 3} for i in range(10)]
    parts = B.split_batch(sets, 4, 1)
    assert [s for (s, _, _) in parts] == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9]]


def test_clamps():
    g = GOLD["clamp_small_batch"]
    nb, nub = B.clamp_params(4096, g["n_batch"], g["n_ubatch"])
    assert nub == g["effective_n_ubatch"]
    d = GOLD["defaults"]
    assert B.clamp_params(1 << 20, 0, d["n_ubatch"]) == (d["n_batch"], d["n_ubatch"])
    # causal: n_batch limited to the cache capacity; non-causal: not
    assert B.clamp_params(1000, 2048, 512, causal=True) == (1000, 512)
    assert B.clamp_params(1000, 2048, 512, causal=False) == (2048, 512)
    # n_ubatch == 0 falls back to n_batch
    assert B.clamp_params(4096, 1024, 0) == (1024, 1024)
    assert B.clamp_params(100, 2048, 0) == (100, 100)


def test_spec_verify_pass_count_and_no_padding():
    g = GOLD["spec_verify"]
    assert len(B.split_batch([{0}] * g["rows"], g["n_ubatch"], 1)) == g["passes"]
    # a one-token decode is a one-row ubatch, not padded to n_ubatch
    assert [len(s) for (s, _, _) in B.split_batch([{0}], 512, 1)] == [1]


def test_split_equal_decode_then_prompts():
    # 64 single-token sequences plus two long prompts: the first ubatch takes
    # one slot from each of the 66 sets (floor(512/66) = 7 >= 1, but the
    # decoders only have one slot each), then only the prompt sets remain.
    sets = [{k} for k in range(2, 66)] + [{0}] * 300 + [{1}] * 200
    parts = B.split_batch(sets, 512, 8)
    slots, nst, ns = parts[0]
    assert (nst, ns) == (1, 66)
    # ordered by smallest sequence id
    assert [min(sets[i]) for i in slots] == list(range(66))
    # then the two prompts: min(remaining, 512 // 2) each
    slots, nst, ns = parts[1]
    assert (nst, ns) == (199, 2)
    assert [min(sets[i]) for i in slots] == [0] * 199 + [1] * 199
    total = sum(len(s) for (s, _, _) in parts)
    assert total == len(sets)
    flat = sorted(i for (s, _, _) in parts for i in s)
    assert flat == list(range(len(sets)))


def test_split_equal_equal_lengths_and_caps():
    sets = [{0}] * 10 + [{1}] * 3 + [{2}] * 7
    parts = B.split_batch(sets, 512, 4)
    # every ubatch has the same count from each of its sets
    for slots, nst, ns in parts:
        assert len(slots) == nst * ns
        counts = {}
        for i in slots:
            counts[min(sets[i])] = counts.get(min(sets[i]), 0) + 1
        assert set(counts.values()) == {nst}
    assert [(nst, ns) for (_, nst, ns) in parts] == [(3, 3), (4, 2), (3, 1)]
    # n_ubatch caps n_seq_tokens * n_seqs
    parts = B.split_batch([{0}] * 9 + [{1}] * 9, 4, 2)
    assert [(nst, ns) for (_, nst, ns) in parts] == [(2, 2)] * 4 + [(1, 2)]
    # more sets than n_ubatch: stop adopting at n_ubatch sets
    parts = B.split_batch([{k} for k in range(6)], 4, 2)
    assert [(len(s), nst, ns) for (s, nst, ns) in parts] == [(4, 1, 4), (2, 1, 2)]


def test_split_equal_overlapping_sets_wait():
    # slot 1's set {0,1} overlaps the adopted {0}: it waits; {1} alone is
    # then blocked by nothing -- but {0,1} must not share a ubatch with {0}
    sets = [{0}, {0, 1}, {2}, {0}]
    parts = B.split_batch(sets, 512, 2)
    for slots, _, _ in parts:
        members = [frozenset(sets[i]) for i in slots]
        uniq = set(members)
        for a in uniq:
            for b in uniq:
                assert a == b or not (a & b)
    first = parts[0][0]
    assert 1 not in first
    assert sorted(i for (s, _, _) in parts for i in s) == [0, 1, 2, 3]


def test_split_equal_submission_order_within_set():
    sets = [{1}, {0}, {1}, {0}, {1}]
    parts = B.split_batch(sets, 512, 2)
    slots, nst, ns = parts[0]
    assert slots == [1, 3, 0, 2]            # set {0} first, each in submission order
    assert parts[1][0] == [4]


def test_output_ids():
    ids = B.output_ids([0, 1, 0, 1, 1], 8)
    assert ids.tolist() == [-1, 0, -1, 1, 2, -1, -1, -1]


def test_fill_batch_autofill_and_errors():
    p, s, o = B.fill_batch(3, None, None, None, {0: 5}, 1, 1)
    assert p == [5, 6, 7] and s == [(0,)] * 3 and o == [0, 0, 1]
    p, s, o = B.fill_batch(4, None, [[1], [0], [1], [0, 2]], [1, 1, 1, 1], {0: 0, 1: 10}, 4, 1)
    assert p == [10, 0, 11, 1]
    assert s[3] == (0, 2)
    # first listed id stays first (the query masks against it)
    p, s, o = B.fill_batch(1, [0], [[2, 0, 1]], None, {}, 4, 1)
    assert s == [(2, 0, 1)]
    with pytest.raises(SplitError):
        B.fill_batch(1, [0], [[4]], None, {}, 4, 1)        # id out of range
    with pytest.raises(SplitError):
        B.fill_batch(1, [-1], [[0]], None, {}, 4, 1)       # negative position
    with pytest.raises(SplitError):
        B.fill_batch(1, [0], [[]], None, {}, 4, 1)         # no id
    p, s, o = B.fill_batch(1, [0], [[1, 0]], None, {}, 4, 2)   # ids in two streams: accepted
    assert s == [(1, 0)]


def test_separate_copies_of_a_prefix_across_streams():
    """"What does llama.cpp's KV cache actually look like in memory?", "Unified versus non-unified": with one stream per sequence a common
    prefix needs separate copies.  A 6-slot prefix shared by sequences 0..3
    takes 6 cells of the unified cache and 6 cells in each of 4 streams, each
    copy holding only the id of its stream; every sequence's decode query
    then attends exactly as over the unified cache."""
    rng = np.random.default_rng(21)
    P, n_seq, layers = 6, 4, [0]
    k = rng.standard_normal((P, 2 * 16))
    v = rng.standard_normal((P, 2 * 16))
    q = rng.standard_normal((n_seq, 4 * 16))
    kd = rng.standard_normal((n_seq, 2 * 16))
    vd = rng.standard_normal((n_seq, 2 * 16))
    outs = {}
    for n_stream, kv in ((1, 64), (4, 16)):
        eng = OracleEngine(1, 4, 2, 16, kv_size=kv, n_stream=n_stream, n_seq_max=n_seq, n_batch=64, n_ubatch=64,
                           layers=layers)
        st, ubs, _ = eng.split(P, list(range(P)), [tuple(range(n_seq))] * P, [0] * P)
        assert st == 0 and len(ubs) == 1
        ub = ubs[0]
        eng.commit(ub, build_mask=False)
        eng.store(ub, 0, k, v)
        assert len(ub.copies) == P * (n_stream - 1)
        used = [int((eng.cells.pos[s] >= 0).sum()) for s in range(n_stream)]
        assert used == [P] * n_stream
        for s in range(n_stream):
            held = eng.cells.member[s][eng.cells.pos[s] >= 0]
            want = [q_ for q_ in range(n_seq) if q_ % n_stream == s]
            assert all(sorted(np.nonzero(h)[0].tolist()) == want for h in held)
        st, ubs, _ = eng.split(n_seq, [P] * n_seq, [(i,) for i in range(n_seq)], [1] * n_seq)
        ub = ubs[0] if len(ubs) == 1 else None
        res = np.zeros((n_seq, 4 * 16))
        for u in ubs:
            eng.commit(u, build_mask=True)
            eng.store(u, 0, kd[u.src], vd[u.src])
            res[u.src] = eng.attend(u, 0, q[u.src])
        outs[n_stream] = res
    assert np.allclose(outs[1], outs[4], rtol=0, atol=1e-12)


def test_engine_rejects_batch_larger_than_n_batch():
    eng = OracleEngine(1, 2, 1, 16, kv_size=64, n_batch=16, n_ubatch=8)
    with pytest.raises(SplitError):
        eng.split(17)
    st, ubs, ids = eng.split(16)
    assert st == 0 and [u.n_tokens for u in ubs] == [8, 8]


def test_split_seq_one_set_per_ubatch():
    """split_seq ("Batch、Ubatch 与解码主循环", Part C item 3): every ubatch holds the tokens of one
    sequence set; different sequences are never mixed.  Interleaved decode
    slots of three sequences, a prefix-shared slot {0, 1} and a cap of 2."""
    sets = [{0}, {1}, {0}, {1}, {2}, {0}, {0, 1}, {0}]
    parts = B.split_batch(sets, 2, 1, mode="seq")
    assert [p[0] for p in parts] == [[0, 2], [1, 3], [4], [5, 7], [6]]
    assert all(p[2] == 1 and p[1] == len(p[0]) for p in parts)
    # invariants: a partition of the batch, one set per ubatch, at most
    # n_ubatch slots, submission order inside a ubatch
    for n_ubatch in (1, 2, 3, 8):
        parts = B.split_batch(sets, n_ubatch, 1, mode="seq")
        flat = sorted(i for p in parts for i in p[0])
        assert flat == list(range(len(sets)))
        for slots, _, _ in parts:
            assert len({frozenset(sets[i]) for i in slots}) == 1
            assert 0 < len(slots) <= n_ubatch and slots == sorted(slots)


def test_split_seq_long_sequence_is_cut_at_n_ubatch():
    sets = [{3}] * 1000
    parts = B.split_batch(sets, 512, 4, mode="seq")
    assert [len(p[0]) for p in parts] == [512, 488]


def test_split_modes_auto_matches_init_batch_choice():
    rng = np.random.default_rng(5)
    sets = [{int(s)} for s in rng.integers(0, 4, size=40)]
    assert B.split_batch(sets, 8, 1) == B.split_batch(sets, 8, 1, mode="simple")
    assert B.split_batch(sets, 8, 3) == B.split_batch(sets, 8, 3, mode="equal")
    with pytest.raises(SplitError):
        B.split_batch(sets, 8, 1, mode="nope")
