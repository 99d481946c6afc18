"""Pins for the oracle's sequence-state save / restore (oracle/seqstate.py).

* "What does llama.cpp's KV cache actually look like in memory?", "Opening the .bin dump" (tests/golden/page_numbers.json, state_dump):
  seven cells of the Qwen3-0.6B shape serialize to 803,596 bytes = 802,816
  payload + 780 metadata; the first K record starts at byte 108, its 12-byte
  header puts the first K value at byte 120, where the page's eight bytes
  decode to its four printed values; K records of layers 0..27 come before
  the V records;
* the blob records positions, not cells: two engines that placed the same
  sequence in different cells save identical bytes;
* restore is the inverse of save (positions, rows and attention), replaces
  what the destination held, shares nothing with other sequences, and
  leaves everything untouched when it does not fit or the blob does not
  match the context.
"""

import json
import os
import struct

import numpy as np
import pytest

from oracle import OracleEngine, f16_round
from oracle import seqstate as S

GOLD = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_numbers.json")))


def engine(n_layer=2, n_head=4, n_head_kv=2, head_dim=16, kv_size=64, n_stream=1, n_seq_max=4, order=None):
    return OracleEngine(n_layer, n_head, n_head_kv, head_dim, kv_size, n_stream, n_seq_max, n_batch=64,
                        n_ubatch=64, cell_order=order)


def run(eng, pos, seqs, rng):
    st, ubs, _ = eng.split(len(pos), pos, seqs, None)
    assert st == 0
    for ub in ubs:
        eng.commit(ub, build_mask=True)
        for l in eng.layers:
            eng.store(ub, l, rng.standard_normal((ub.n_tokens, eng.E)), rng.standard_normal((ub.n_tokens, eng.E)))
    return ubs


def test_page_sizes_and_offsets():
    d = GOLD["state_dump"]
    eng = engine(n_layer=28, n_head=16, n_head_kv=8, head_dim=128, kv_size=64, n_seq_max=2)
    rng = np.random.default_rng(5)
    run(eng, list(range(d["cells"])), [(0,)] * d["cells"], rng)
    # the page's first four K values in layer 0's row of position 0
    s, cells, pos = S.sequence_cells(eng, 0)
    first = np.frombuffer(bytes.fromhex(d["first_bytes_hex"].replace(" ", "")), "<f2")
    eng.K[0][s, cells[0], :4] = first
    blob = S.save(eng, 0)
    assert len(blob) == d["file_bytes"] == d["payload_bytes"] + d["metadata_bytes"]
    assert S.record_offset(28, 8, 128, 7, 0, 0) == d["first_k_record"]
    assert d["first_k_record"] + d["record_header_bytes"] == d["first_k_value"]
    assert blob[d["first_k_value"]:d["first_k_value"] + 8].hex(" ") == d["first_bytes_hex"]
    vals = struct.unpack_from("<4e", blob, d["first_k_value"])
    assert [round(v, 4) for v in vals] == d["first_values_4dp"]
    # metadata = leading bytes + one header per record; payload = rows
    assert d["first_k_record"] + 56 * d["record_header_bytes"] == d["metadata_bytes"]
    assert 56 * 7 * 2048 == d["payload_bytes"]
    # all K records, then all V records, each row the cell's full row
    row = 2048
    for kind, cache in enumerate((eng.K, eng.V)):
        for layer in range(28):
            off = S.record_offset(28, 8, 128, 7, kind, layer)
            assert off == 108 + (kind * 28 + layer) * (12 + 7 * row)
            assert struct.unpack_from("<IQ", blob, off) == (S.TYPE_F16, row)
            for i, c in enumerate(cells):
                got = np.frombuffer(blob, "<f2", count=1024, offset=off + 12 + i * row)
                assert np.array_equal(got.view(np.uint16), cache[layer][s, c].view(np.uint16))
    assert struct.unpack_from("<7i", blob, 80) == tuple(range(7))


def test_blob_records_positions_not_cells():
    rng_cells = np.random.default_rng(11).permutation(64)
    blobs = []
    for order in (None, rng_cells):
        eng = engine(order=order)
        rng = np.random.default_rng(3)
        run(eng, list(range(10)), [(0, 1)] * 10, rng)          # shared prefix
        run(eng, [10, 11, 10], [(0,), (0,), (1,)], rng)
        blobs.append((S.save(eng, 0), S.save(eng, 1), S.sequence_cells(eng, 0)[1]))
    assert blobs[0][0] == blobs[1][0] and blobs[0][1] == blobs[1][1]
    assert blobs[0][2] != blobs[1][2]                            # different cells, same bytes
    n0 = struct.unpack_from("<I", blobs[0][0], 20)[0]
    assert n0 == 12 and struct.unpack_from("<12i", blobs[0][0], 80) == tuple(range(12))


def test_round_trip_into_another_engine_and_sequence():
    src = engine()
    rng = np.random.default_rng(7)
    run(src, list(range(6)), [(0, 1)] * 6, rng)
    run(src, [6, 7, 6], [(0,), (0,), (1,)], rng)
    blob = S.save(src, 0)
    dst = engine(order=np.random.default_rng(2).permutation(64))
    run(dst, [0, 1, 2], [(3,)] * 3, np.random.default_rng(9))   # something else lives there
    cells = S.load(dst, 2, blob)
    s, dcells, dpos = S.sequence_cells(dst, 2)
    assert sorted(dcells) == sorted(cells) and dpos == list(range(8))
    assert all(dst.cells.member[s, c].sum() == 1 for c in dcells)   # a private copy
    _, scells, _ = S.sequence_cells(src, 0)
    for layer in range(2):
        for a, b in zip(scells, dcells):
            assert np.array_equal(src.K[layer][0, a], dst.K[layer][0, b])
            assert np.array_equal(src.V[layer][0, a], dst.V[layer][0, b])
    assert S.save(dst, 2) == blob
    # the same query attends identically over the original and the copy
    q = np.random.default_rng(1).standard_normal((1, 4 * 16))
    outs = []
    for e, seq in ((src, 0), (dst, 2)):
        _, ubs, _ = e.split(1, [8], [(seq,)], [1])
        e.commit(ubs[0], build_mask=True)
        for layer in range(2):
            e.store(ubs[0], layer, np.zeros((1, e.E)), np.zeros((1, e.E)))
        outs.append(e.attend(ubs[0], 1, q))
    assert np.allclose(outs[0], outs[1], rtol=0, atol=1e-12)


def test_restore_replaces_and_all_or_nothing():
    src = engine(kv_size=16)
    run(src, list(range(9)), [(0,)] * 9, np.random.default_rng(4))
    blob = S.save(src, 0)
    dst = engine(kv_size=16)
    run(dst, list(range(5)), [(1,)] * 5, np.random.default_rng(5))
    run(dst, list(range(4)), [(2,)] * 4, np.random.default_rng(6))
    before = (dst.cells.pos.copy(), dst.cells.member.copy())
    with pytest.raises(S.StateError):
        S.load(dst, 3, blob)                  # 7 free cells < 9
    assert np.array_equal(before[0], dst.cells.pos) and np.array_equal(before[1], dst.cells.member)
    S.load(dst, 1, blob)                      # 7 free + sequence 1's own 5 >= 9: replaced
    _, _, pos1 = S.sequence_cells(dst, 1)
    assert pos1 == list(range(9))
    assert S.sequence_cells(dst, 2)[2] == list(range(4))


def test_blob_validation():
    src = engine()
    run(src, list(range(3)), [(0,)] * 3, np.random.default_rng(8))
    blob = S.save(src, 0)
    with pytest.raises(S.StateError):
        S.load(engine(head_dim=32), 0, blob)
    with pytest.raises(S.StateError):
        S.load(engine(n_layer=3), 0, blob)
    bad = bytearray(blob)
    bad[S.record_offset(2, 2, 16, 3, 1, 0)] = 2          # V record of layer 0 claims another type
    with pytest.raises(S.StateError):
        S.load(engine(), 0, bytes(bad))
    with pytest.raises(S.StateError):
        S.load(engine(), 0, blob[:-1])
    empty = S.save(engine(), 0)
    assert len(empty) == S.state_bytes(2, 2, 16, 0) == 80 + 2 * 2 * 12
    e = engine()
    assert S.load(e, 0, empty) == [] and S.sequence_cells(e, 0)[1] == []


def test_f16_rows_are_the_stored_rounding():
    eng = engine(n_layer=1)
    x = np.random.default_rng(12).standard_normal((4, eng.E))
    st, ubs, _ = eng.split(4, [0, 1, 2, 3], [(0,)] * 4, None)
    eng.commit(ubs[0], build_mask=False)
    eng.store(ubs[0], 0, x, -x)
    blob = S.save(eng, 0)
    off = S.record_offset(1, 2, 16, 4, 0, 0) + 12
    rows = np.frombuffer(blob, "<f2", count=4 * eng.E, offset=off).reshape(4, eng.E)
    assert np.array_equal(rows.view(np.uint16), f16_round(x).view(np.uint16))
