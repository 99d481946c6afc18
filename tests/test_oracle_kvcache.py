"""Oracle pins: cache sizes and addresses, F16 encoding, n_kv, placement, mask."""

import json
import os

import numpy as np
import pytest

from oracle import (CellTable, OracleEngine, f16_round, row_bytes, cache_bytes, k_elem_offset)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))
KIB, MIB, GIB = 1024, 1024 ** 2, 1024 ** 3


def test_row_and_token_sizes():
    g = GOLD["kv_row"]
    assert row_bytes(g["n_head_kv"], g["head_dim"]) == g["row_bytes"]
    per_token = cache_bytes(g["n_layer"], g["n_head_kv"], g["head_dim"], kv_size=1)
    assert per_token == g["per_token_kv_bytes"] == 112 * KIB
    assert cache_bytes(g["n_layer"], g["n_head_kv"], g["head_dim"], kv_size=8) == g["eight_tokens_bytes"]


def test_allocation_448_mib_unified_and_not():
    g = GOLD["kv_allocation"]
    total = cache_bytes(28, 8, 128, g["kv_size"])
    assert total == g["total_mib"] * MIB
    assert total // 2 == g["k_mib"] * MIB == g["v_mib"] * MIB
    n = GOLD["non_unified"]
    assert cache_bytes(28, 8, 128, n["total_cells"] // n["n_seq"], n_stream=n["n_seq"]) == n["total_mib"] * MIB


def test_strides_and_address_example():
    g = GOLD["k_tensor_dims"]
    ne0, ne1, ne2 = g["ne"]
    rb = row_bytes(8, 128)
    assert [2, rb, ne1 * rb] == g["nb"]
    ex = g["example"]
    assert k_elem_offset(ex["cell"], ex["head"], ex["elem"], 8, 128) == ex["offset"]
    # stream slabs start at s * nb[2]
    assert k_elem_offset(0, 0, 0, 8, 128, stream=1, kv_size=ne1) == g["nb"][2]


def test_state_dump_payload_arithmetic():
    g = GOLD["state_dump"]
    payload = cache_bytes(28, 8, 128, kv_size=g["cells"])
    assert payload == g["payload_bytes"]
    # metadata, then 56 records of 12-byte header + rows
    assert g["first_k_record"] + 56 * g["record_header_bytes"] == g["metadata_bytes"]
    assert g["metadata_bytes"] + payload == g["file_bytes"]
    assert g["first_k_record"] + g["record_header_bytes"] == g["first_k_value"]


def test_f16_bytes_decode_and_roundtrip():
    g = GOLD["state_dump"]
    raw = bytes.fromhex(g["first_bytes_hex"].replace(" ", ""))
    vals = np.frombuffer(raw, dtype="<f2")
    assert [round(float(v), 4) for v in vals] == g["first_values_4dp"]
    assert float(vals[0]) == 0.449462890625            # 0x3731 = (1 + 817/1024) / 4
    # the store rounding reproduces the stored bit patterns from nearby fp32 values
    assert f16_round(np.float32(0.4495)).tobytes() == raw[:2]
    assert f16_round(vals.astype(np.float32)).tobytes() == raw


def test_f16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = 2.0 ** -10                                    # F16 spacing at 1.0
    assert float(f16_round(one + ulp / 2)) == 1.0       # tie -> even (1.0)
    assert float(f16_round(one + 3 * ulp / 2)) == 1.0 + 2 * ulp   # tie -> even
    assert float(f16_round(one + 0.51 * ulp)) == 1.0 + ulp
    assert float(f16_round(np.float32(70000.0))) == np.inf        # overflow
    assert float(f16_round(np.float32(-2.0 ** -25))) == 0.0       # underflow to -0
    assert np.signbit(f16_round(np.float32(-2.0 ** -25)))


def test_cache_budget_page4():
    g = GOLD["cache_budget"]
    m = g["mha"]
    per_tok = 2 * m["n_layer"] * m["width"] * m["bytes_per_value"]
    assert per_tok == m["per_token_kib"] * KIB
    assert per_tok * m["ctx"] == m["ctx_gib"] * GIB
    q = g["gqa"]
    per_tok = cache_bytes(q["n_layer"], q["n_head_kv"], q["head_dim"], kv_size=1)
    assert per_tok == q["per_token_kib"] * KIB
    assert per_tok * q["ctx"] == q["ctx_mib"] * MIB


def fill(table, n, stream=0, seq=0):
    cells = table.reserve([stream] * n)
    base = table.seq_pos_max(seq) + 1
    table.commit([stream] * n, cells, list(range(base, base + n)), [(seq,)] * n)
    return cells


def test_n_kv_page_example():
    g = GOLD["n_kv_padding"]
    t = CellTable(4096)
    assert t.n_kv() == g["quantum"]                     # empty cache still reports 256
    fill(t, g["live"])
    assert t.n_kv() == g["reported"]
    # stays constant as decode proceeds until cell index 768 is occupied
    seen = set()
    for step in range(g["reported"] - g["live"]):
        seen.add(t.n_kv())
        fill(t, 1)
    assert seen == {g["reported"]}
    assert t.used_max_p1(0) == g["reported"]
    assert t.n_kv() == g["reported"]
    fill(t, 1)                                          # cell 768, the 769th cell
    assert t.n_kv() == g["reported"] + g["quantum"]
    # and is then constant for the next 255 steps
    vals = set()
    for step in range(g["constant_steps"] - 1):
        vals.add(t.n_kv())
        fill(t, 1)
    assert vals == {1024}
    assert t.n_kv() == 1024


def test_n_kv_small_cache_and_streams():
    t = CellTable(64)
    assert t.n_kv() == 64                               # min(kv_size, ...) clause
    t = CellTable(1024, n_stream=3, n_seq_max=3)
    fill(t, 10, stream=0, seq=0)
    fill(t, 300, stream=2, seq=2)
    assert t.n_kv() == 512                              # largest over streams


def test_placement_order_all_or_nothing_and_reuse():
    order = np.array([[5, 3, 7, 0, 1, 2, 4, 6]])
    t = CellTable(8, order=order)
    assert t.reserve([0, 0, 0]) == [5, 3, 7]
    t.release([0, 0, 0], [5, 3, 7])
    cells = t.reserve([0] * 8)
    assert cells == order[0].tolist()
    t.release([0] * 8, cells)
    fill(t, 6)
    before = (t.pos.copy(), t.member.copy(), t.reserved.copy())
    assert t.reserve([0, 0, 0]) is None                 # only 2 left: nothing reserved
    assert np.array_equal(before[2], t.reserved)
    # a freed cell returns with its original rank
    t.seq_rm(0, 2, 3)                                   # frees the cell holding pos 2 (cell 7)
    assert t.reserve([0]) == [7]


def test_seq_rm_multi_sequence_cells():
    t = CellTable(16, n_seq_max=3)
    cells = t.reserve([0, 0])
    t.commit([0, 0], cells, [0, 1], [(0, 1, 2), (0, 1, 2)])
    t.seq_rm(1, -1, -1)
    assert (t.pos[0, cells] == [0, 1]).all()            # still held by 0 and 2
    assert not t.member[0, cells, 1].any()
    t.seq_rm(0, 1, -1)
    t.seq_rm(2, 1, -1)
    assert t.pos[0, cells[1]] == -1 and t.pos[0, cells[0]] == 0
    t.seq_rm(-1, -1, -1)
    assert (t.pos < 0).all()


def test_mask_prefix_sharing_page_example():
    g = GOLD["prefix_sharing"]
    eng = OracleEngine(1, 2, 1, 16, kv_size=64, n_seq_max=3)
    st, ubs, _ = eng.split(2, g["prefill"]["pos"], [g["prefill"]["seq_ids"]] * 2)
    eng.commit(ubs[0])
    dec = g["decode"]
    st, ubs, _ = eng.split(3, [d["pos"] for d in dec], [[d["seq"]] for d in dec])
    ub = ubs[0]
    m = eng.commit(ub)
    assert ub.cells == [2, 3, 4]
    for r, d in enumerate(dec):
        visible = set(np.nonzero(m[r] == 0)[0].tolist())
        assert visible == {0, 1, ub.cells[r]}           # shared prefix + own cell only
    assert m.dtype == np.float16 and m.shape == (3, 64)        # n_kv capped by kv_size
    assert set(np.unique(m.view(np.uint16)).tolist()) == {0x0000, 0xFC00}


def test_mask_uses_first_sequence_id_only():
    eng = OracleEngine(1, 2, 1, 16, kv_size=64, n_seq_max=3)
    st, ubs, _ = eng.split(3, [0, 0, 0], [[0], [1], [2]])
    eng.commit(ubs[0])
    st, ubs, _ = eng.split(1, [1], [[0, 1, 2]])
    m = eng.commit(ubs[0])
    # the query belongs to {0,1,2} but masks as sequence 0: sees cell 0 and itself
    assert set(np.nonzero(m[0] == 0)[0].tolist()) == {0, 3}


def test_mask_causal_and_empty_cells_and_noncausal():
    eng = OracleEngine(1, 2, 1, 16, kv_size=64, n_seq_max=1)
    st, ubs, _ = eng.split(4, [0, 1, 2, 3], [[0]] * 4)
    m = eng.commit(ubs[0])
    vis = (m == 0)
    assert np.array_equal(vis[:, :4], np.tril(np.ones((4, 4), bool)))
    assert not vis[:, 4:].any()                          # empty cells
    eng = OracleEngine(1, 2, 1, 16, kv_size=64, n_seq_max=1, causal=False)
    st, ubs, _ = eng.split(4, [0, 1, 2, 3], [[0]] * 4)
    m = eng.commit(ubs[0])
    assert (m[:, :4] == 0).all() and (m[:, 4:] != 0).all()


def test_later_ubatch_invisible_until_committed():
    eng = OracleEngine(1, 2, 1, 16, kv_size=64, n_ubatch=2)
    st, ubs, _ = eng.split(4, [0, 1, 2, 3], [[0]] * 4)
    assert len(ubs) == 2
    m0 = eng.commit(ubs[0])
    assert set(np.nonzero(m0[1] == 0)[0].tolist()) == {0, 1}
    m1 = eng.commit(ubs[1])
    assert set(np.nonzero(m1[1] == 0)[0].tolist()) == {0, 1, 2, 3}


def test_cache_full_returns_1():
    eng = OracleEngine(1, 2, 1, 16, kv_size=8)
    st, ubs, _ = eng.split(6)
    for u in ubs:
        eng.commit(u)
    st, ubs, ids = eng.split(3)
    assert st == 1 and ubs == []
    assert (eng.cells.pos >= 0).sum() == 6
