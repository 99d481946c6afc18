"""Oracle pins for the attention step.

* brute force: explicit loops over the token history (no cells, no n_kv, no
  mask) on the Tiny workload and on a small multi-sequence case;
* library special case: one sequence in contiguous cells equals torch's
  scaled_dot_product_attention(is_causal=True) on the CPU in fp64 with the KV
  heads repeated for GQA;
* closed forms: one visible key returns its value; equal keys average the
  values; a row with nothing visible is zero;
* needles: a dominant key planted in a visible cell takes over the output,
  the same key in a hidden cell (other sequence / future / beyond n_kv)
  changes nothing;
* invariances: isolation from unrelated sequences, slot order, ubatch size,
  free-cell order.
"""

import math

import numpy as np
import pytest

from oracle import OracleEngine, brute_force_attention, f16_round, masked_attention
from synthetic import workloads as W


def run_oracle(wl, cell_order="auto", n_ubatch=None, layers=None):
    """Drive the oracle through every batch; returns {(batch, layer): out
    rows in batch order} for measured batches and the engine."""
    order = wl.cell_order if cell_order == "auto" else cell_order
    eng = OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size,
                       wl.n_stream, wl.n_seq_max, wl.n_batch,
                       wl.n_ubatch if n_ubatch is None else n_ubatch, wl.causal,
                       cell_order=order, layers=layers, swa=wl.swa)
    layers = eng.layers
    outs = {}
    for b, bt in enumerate(wl.batches):
        st, ubs, _ = eng.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0
        ks = {l: wl.tensor(b, l, W.KIND_K) for l in layers}
        vs = {l: wl.tensor(b, l, W.KIND_V) for l in layers}
        qs = {l: wl.tensor(b, l, W.KIND_Q) for l in layers} if bt.measured else None
        res = {l: np.zeros((bt.n_tokens, wl.n_head * wl.head_dim)) for l in layers}
        for ub in ubs:
            eng.commit(ub)
            for l in layers:
                eng.store(ub, l, ks[l][ub.src], vs[l][ub.src])
                if bt.measured:
                    res[l][ub.src] = eng.attend(ub, l, qs[l][ub.src])
        if bt.measured:
            for l in layers:
                outs[(b, l)] = res[l]
    return outs, eng


def brute(wl, layer=0):
    """Brute force over the submitted token history, batch by batch, ubatch
    boundaries ignored except that a query sees tokens of its own batch up to
    its position (which is what causal + committed-before means here)."""
    hist = []
    outs = {}
    for b, bt in enumerate(wl.batches):
        k = f16_round(wl.tensor(b, layer, W.KIND_K))
        v = f16_round(wl.tensor(b, layer, W.KIND_V))
        for i in range(bt.n_tokens):
            hist.append((int(bt.pos[i]), set(bt.seq_ids[i]), k[i], v[i]))
        if bt.measured:
            q = wl.tensor(b, layer, W.KIND_Q)
            queries = [(int(bt.pos[i]), bt.seq_ids[i][0], q[i]) for i in range(bt.n_tokens)]
            outs[(b, layer)] = np.array(brute_force_attention(
                queries, hist, wl.n_head, wl.n_head_kv, wl.head_dim, wl.causal, swa=wl.swa))
    return outs


def test_tiny_matches_brute_force():
    wl = W.tiny()
    got, _ = run_oracle(wl)
    ref = brute(wl)
    assert set(got) == set(ref)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-12)


def test_multi_sequence_prefix_matches_brute_force():
    wl = W.prefix_decode(n_seq=3, prefix=5, private=4, n_layer=1, kv_size=64)
    wl.n_head, wl.n_head_kv, wl.head_dim = 4, 2, 8
    for bt in wl.batches:
        bt.measured = True
    got, _ = run_oracle(wl)
    ref = brute(wl)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-12)


def test_single_sequence_equals_torch_sdpa():
    torch = pytest.importorskip("torch")
    wl = W.qwen_prefill(n_prompt=200, n_layer=1, kv_size=256, n_batch=128, n_ubatch=48)
    wl.n_head, wl.n_head_kv, wl.head_dim = 8, 2, 32
    got, eng = run_oracle(wl)
    L = wl.n_head * wl.head_dim
    q = np.concatenate([wl.tensor(b, 0, W.KIND_Q) for b in range(len(wl.batches))])
    k = np.concatenate([f16_round(wl.tensor(b, 0, W.KIND_K)) for b in range(len(wl.batches))])
    v = np.concatenate([f16_round(wl.tensor(b, 0, W.KIND_V)) for b in range(len(wl.batches))])
    T, d, H, Hk = q.shape[0], wl.head_dim, wl.n_head, wl.n_head_kv
    qt = torch.tensor(q, dtype=torch.float64).view(T, H, d).transpose(0, 1)
    kt = torch.tensor(k.astype(np.float64)).view(T, Hk, d).transpose(0, 1)
    vt = torch.tensor(v.astype(np.float64)).view(T, Hk, d).transpose(0, 1)
    kt = kt.repeat_interleave(H // Hk, dim=0)
    vt = vt.repeat_interleave(H // Hk, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref.transpose(0, 1).reshape(T, L).numpy()
    mine = np.concatenate([got[(b, 0)] for b in range(len(wl.batches))])
    np.testing.assert_allclose(mine, ref, rtol=1e-10, atol=1e-12)


def small_engine(**kw):
    args = dict(n_layer=1, n_head=4, n_head_kv=2, head_dim=8, kv_size=64, n_seq_max=4)
    args.update(kw)
    return OracleEngine(**args)


def test_closed_forms():
    rng = np.random.default_rng(7)
    eng = small_engine()
    # one token: its own value, for every head of its group
    st, ubs, _ = eng.split(1, [0], [[0]])
    ub = ubs[0]
    eng.commit(ub)
    k = rng.standard_normal((1, 16)).astype(np.float32)
    v = rng.standard_normal((1, 16)).astype(np.float32)
    eng.store(ub, 0, k, v)
    o = eng.attend(ub, 0, rng.standard_normal((1, 32)).astype(np.float32))
    v16 = f16_round(v).astype(np.float64)[0]
    expect = np.concatenate([v16[0:8], v16[0:8], v16[8:16], v16[8:16]])
    np.testing.assert_array_equal(o[0], expect)
    # equal keys: uniform weights -> mean of the values
    eng = small_engine()
    st, ubs, _ = eng.split(5, list(range(5)), [[1]] * 5)
    ub = ubs[0]
    eng.commit(ub)
    kk = np.tile(rng.standard_normal((1, 16)).astype(np.float32), (5, 1))
    vv = rng.standard_normal((5, 16)).astype(np.float32)
    eng.store(ub, 0, kk, vv)
    o = eng.attend(ub, 0, rng.standard_normal((5, 32)).astype(np.float32))
    v16 = f16_round(vv).astype(np.float64)
    np.testing.assert_allclose(o[4, 0:8], v16[:, 0:8].mean(axis=0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o[4, 24:32], v16[:, 8:16].mean(axis=0), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o[1, 8:16], v16[:2, 0:8].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_fully_masked_row_is_zero():
    eng = small_engine()
    st, ubs, _ = eng.split(1, [0], [[0]])
    ub = ubs[0]
    eng.commit(ub)
    mask = np.full_like(ub.mask, np.float16(-np.inf))
    o = masked_attention(np.ones((1, 32), np.float32), eng.K[0], eng.V[0], [0], mask, 4, 2)
    assert (o == 0).all()


def needle_setup(where):
    """Sequence 0 has 40 tokens; sequence 1 has 10.  A query of sequence 0 at
    position 20.  The needle key points along q for head 0 (kv head 0)."""
    rng = np.random.default_rng(11)
    eng = small_engine(kv_size=300)
    d = 8
    q = rng.standard_normal((1, 32)).astype(np.float32)
    qhat = q[0, 0:d] / np.linalg.norm(q[0, 0:d])
    st, ubs, _ = eng.split(40, list(range(40)), [[0]] * 40)
    ub0 = ubs[0]
    eng.commit(ub0)
    k0 = rng.standard_normal((40, 16)).astype(np.float32) * 0.1
    v0 = rng.standard_normal((40, 16)).astype(np.float32)
    st, ubs, _ = eng.split(10, list(range(10)), [[1]] * 10)
    ub1 = ubs[0]
    eng.commit(ub1)
    k1 = rng.standard_normal((10, 16)).astype(np.float32) * 0.1
    v1 = rng.standard_normal((10, 16)).astype(np.float32)
    needle_v = np.full(16, 7.0, np.float32)
    if where == "visible":
        k0[5, 0:d] = 50 * qhat
        v0[5] = needle_v
    elif where == "future":
        k0[30, 0:d] = 50 * qhat
        v0[30] = needle_v
    elif where == "other_seq":
        k1[3, 0:d] = 50 * qhat
        v1[3] = needle_v
    eng.store(ub0, 0, k0, v0)
    eng.store(ub1, 0, k1, v1)
    if where == "beyond_nkv":
        # a stale row beyond n_kv (cell 290) must never be read
        eng.K[0][0, 290, 0:d] = f16_round(50 * qhat)
        eng.V[0][0, 290] = f16_round(needle_v)
    st, ubs, _ = eng.split(1, [20], [[0]])
    ub = ubs[0]
    eng.commit(ub)
    eng.store(ub, 0, rng.standard_normal((1, 16)).astype(np.float32) * 0.1,
              rng.standard_normal((1, 16)).astype(np.float32))
    return eng.attend(ub, 0, q), ub


def test_needles():
    base, _ = needle_setup("none")
    o, _ = needle_setup("visible")
    np.testing.assert_allclose(o[0, 0:8], 7.0, rtol=1e-6)          # head 0 locks onto the needle
    assert np.abs(o[0, 0:8] - base[0, 0:8]).max() > 1.0
    for where in ("future", "other_seq", "beyond_nkv"):
        o, ub = needle_setup(where)
        np.testing.assert_array_equal(o, base)
    assert ub.n_kv == 256


def test_isolation_from_unrelated_sequence():
    rng = np.random.default_rng(3)
    outs = []
    for with_b in (False, True):
        eng = small_engine()
        rows = [(p, 0) for p in range(6)]
        if with_b:
            rows = [(0, 1), (0, 0), (1, 1), (1, 0), (2, 0), (2, 1), (3, 0), (4, 0), (5, 0)]
        st, ubs, _ = eng.split(len(rows), [p for p, _ in rows], [[s] for _, s in rows])
        ub = ubs[0]
        eng.commit(ub)
        kv_rng = {s: np.random.default_rng(100 + s) for s in (0, 1)}
        k = np.zeros((len(rows), 16), np.float32)
        v = np.zeros((len(rows), 16), np.float32)
        q = np.zeros((len(rows), 32), np.float32)
        for r, (p, s) in enumerate(rows):
            g = np.random.default_rng(1000 * s + p)
            k[r], v[r], q[r] = g.standard_normal(16), g.standard_normal(16), g.standard_normal(32)
        eng.store(ub, 0, k, v)
        o = eng.attend(ub, 0, q)
        outs.append({(p, s): o[r] for r, (p, s) in enumerate(rows)})
    for key, val in outs[0].items():
        np.testing.assert_array_equal(val, outs[1][key])


def test_row_order_invariance():
    wl = W.mixed(n_prompt_seq=2, n_decoders=3, prompt_range=(5, 9), ctx_range=(4, 12),
                 n_layer=1, n_stream=1, kv_size=128, n_batch=64, n_ubatch=64)
    wl.n_seq_max = 5
    got, _ = run_oracle(wl)
    # permute the slots of every batch: outputs permute with them
    rng = np.random.default_rng(5)
    perms = [rng.permutation(bt.n_tokens) for bt in wl.batches]
    wl2 = W.mixed(n_prompt_seq=2, n_decoders=3, prompt_range=(5, 9), ctx_range=(4, 12),
                  n_layer=1, n_stream=1, kv_size=128, n_batch=64, n_ubatch=64)
    wl2.n_seq_max = 5
    base_tensor = wl.tensor
    for bt, pm in zip(wl2.batches, perms):
        bt.pos = bt.pos[pm]
        bt.seq_ids = [bt.seq_ids[i] for i in pm]
        bt.output = bt.output[pm]
    wl2.tensor = lambda b, l, kind: base_tensor(b, l, kind)[perms[b]]
    got2, _ = run_oracle(wl2)
    for (b, l), val in got.items():
        np.testing.assert_allclose(got2[(b, l)], val[perms[b]], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("n_ubatch", [64, 7, 1])
def test_split_invariance(n_ubatch):
    wl = W.qwen_prefill(n_prompt=150, n_layer=1, kv_size=512, n_batch=100, n_ubatch=512)
    wl.n_head, wl.n_head_kv, wl.head_dim = 4, 2, 16
    ref, eng_ref = run_oracle(wl)
    got, eng = run_oracle(wl, n_ubatch=n_ubatch)
    assert np.array_equal(eng.cells.pos, eng_ref.cells.pos)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-13)


def test_cell_permutation_invariance():
    wl = W.cb_decode(n_seq=6, lengths=(3, 9, 17, 30), n_layer=1, kv_size=128)
    wl.n_head, wl.n_head_kv, wl.head_dim = 4, 2, 16
    a, ea = run_oracle(wl)
    b, eb = run_oracle(wl, cell_order=None)
    assert not np.array_equal(ea.cells.pos, eb.cells.pos)
    for key in a:
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-13)


def test_workload_context_total_matches_page4_duty_cycle():
    wl = W.cb_decode(n_layer=1)
    measured = wl.batches[-1]
    # eight lengths 64..2048 hold 5568 useful positions; 64 sequences = 8 x that
    assert int(measured.pos.sum()) == 8 * 5568
    assert 5568 / (8 * 2048) == pytest.approx(0.34, abs=0.005)
    assert (20 + 2000) / (2 * 2000) == pytest.approx(0.505)


def test_single_ubatch_noncausal_equals_torch_sdpa():
    """Non-causal attention ("llama.cpp and the ubatch", "The mask is doing
    the work": the position test applies only under causal attention): one
    sequence stored as one ubatch sees every one of its cells, which is
    torch's scaled_dot_product_attention without a mask."""
    import dataclasses
    torch = pytest.importorskip("torch")
    wl = W.qwen_prefill(n_prompt=150, n_layer=1, kv_size=256, n_batch=256, n_ubatch=256)
    wl = dataclasses.replace(wl, causal=False)
    wl.n_head, wl.n_head_kv, wl.head_dim = 8, 2, 32
    got, _ = run_oracle(wl)
    assert len(wl.batches) == 1
    q = wl.tensor(0, 0, W.KIND_Q)
    k = f16_round(wl.tensor(0, 0, W.KIND_K)).astype(np.float64)
    v = f16_round(wl.tensor(0, 0, W.KIND_V)).astype(np.float64)
    T, d, H, Hk = q.shape[0], wl.head_dim, wl.n_head, wl.n_head_kv
    qt = torch.tensor(q, dtype=torch.float64).view(T, H, d).transpose(0, 1)
    kt = torch.tensor(k).view(T, Hk, d).transpose(0, 1).repeat_interleave(H // Hk, dim=0)
    vt = torch.tensor(v).view(T, Hk, d).transpose(0, 1).repeat_interleave(H // Hk, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=False)
    ref = ref.transpose(0, 1).reshape(T, H * d).numpy()
    np.testing.assert_allclose(got[(0, 0)], ref, rtol=1e-10, atol=1e-12)


def test_noncausal_multi_sequence_matches_brute_force():
    """Non-causal, several sequences, one ubatch per call: every query sees
    all cells of its sequence stored so far, its own call included."""
    import dataclasses
    wl = W.prefix_decode(n_seq=3, prefix=5, private=4, n_layer=1, kv_size=64)
    wl = dataclasses.replace(wl, causal=False)
    wl.n_head, wl.n_head_kv, wl.head_dim = 4, 2, 8
    for bt in wl.batches:
        bt.measured = True
    got, _ = run_oracle(wl)
    ref = brute(wl)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-12)


# -- sliding window ("llama.cpp and the ubatch", "The mask is doing the work":
# the window rule is elided; reading: a key is outside the window when the
# query's position minus the key's is at least the window)

def _swa(wl, w):
    import dataclasses
    wl = dataclasses.replace(wl, swa=w)
    for bt in wl.batches:
        bt.measured = True
    return wl


@pytest.mark.parametrize("w", [1, 3, 6])
def test_swa_matches_brute_force(w):
    for wl in (W.tiny(), W.prefix_decode(n_seq=3, prefix=5, private=4, n_layer=1, kv_size=64)):
        wl = _swa(wl, w)
        wl.n_head, wl.n_head_kv, wl.head_dim = (2, 1, 16) if wl.name == "tiny" else (4, 2, 8)
        got, _ = run_oracle(wl)
        ref = brute(wl)
        for key in ref:
            np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-12)


def test_swa_wider_than_the_history_is_causal():
    wl = W.tiny()
    base, _ = run_oracle(_swa(wl, 0))
    wide, _ = run_oracle(_swa(W.tiny(), 15))          # positions 0..14: every key within 15
    narrow, _ = run_oracle(_swa(W.tiny(), 14))
    for key in base:
        np.testing.assert_array_equal(wide[key], base[key])
    assert any(not np.array_equal(narrow[key], base[key]) for key in base)


def test_swa_window_of_one_returns_the_own_value():
    wl = _swa(W.tiny(), 1)
    got, _ = run_oracle(wl)
    for b, bt in enumerate(wl.batches):
        v = f16_round(wl.tensor(b, 0, W.KIND_V)).astype(np.float64)
        G, d = wl.n_head // wl.n_head_kv, wl.head_dim              # head h reads KV head h // G
        want = np.concatenate([v[:, (h // G) * d:(h // G + 1) * d] for h in range(wl.n_head)], axis=1)
        np.testing.assert_allclose(got[(b, 0)], want, rtol=0, atol=1e-12)


def test_swa_needle_at_the_window_edge():
    """A dominant key one position inside the window takes over the output;
    the same key one position further back changes nothing."""
    H, Hk, d, w = 2, 1, 16, 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal(H * d)
    base_k = rng.standard_normal((10, Hk * d)) * 0.1
    base_v = rng.standard_normal((10, Hk * d))
    def run(needle_pos):
        eng = OracleEngine(1, H, Hk, d, kv_size=64, swa=w)
        k, v = base_k.copy(), base_v.copy()
        if needle_pos is not None:
            k[needle_pos] = 50.0 * q[:d] / np.linalg.norm(q[:d])
            v[needle_pos] = 7.0
        st, ubs, _ = eng.split(10, list(range(10)), [(0,)] * 10, [1] * 10)
        eng.commit(ubs[0])
        eng.store(ubs[0], 0, k, v)
        return eng.attend(ubs[0], 0, np.tile(q, (10, 1)))[9]
    plain = run(None)
    assert np.allclose(run(9 - w), plain, atol=1e-12)          # just outside: no effect
    inside = run(9 - w + 1)
    assert np.allclose(inside[:d], 7.0, atol=1e-3)                # just inside: takes over
