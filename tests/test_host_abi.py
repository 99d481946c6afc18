"""The C ABI on the CPU (no GPU needed).

* libkvattn.so loads and exports every function include/kvattn.h declares;
* the host half -- batch intake, split_simple / split_equal, placement,
  commit, n_kv, output_ids, seq_rm, error codes -- matches the oracle bit for
  bit on every workload shape (reduced sizes) and on edge cases.
"""

import os
import re
import subprocess

import numpy as np
import pytest

from oracle import OracleEngine, SplitError
from synthetic import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
K = pytest.importorskip("ubatch_attention_paged_amd")


def declared_functions():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvattn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 23
    lib = K.load()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kvattn_\w+)", out))
    assert set(names) <= exported
    # nothing else leaks into the C namespace
    assert exported == set(names)


def host_ctx(wl, order="auto", n_ubatch=None):
    order = wl.cell_order if order == "auto" else order
    return K.Context(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                     wl.n_seq_max, wl.n_batch, wl.n_ubatch if n_ubatch is None else n_ubatch,
                     wl.causal, cell_order=order, split_mode=wl.split_mode)


def oracle_for(wl, order="auto", n_ubatch=None):
    order = wl.cell_order if order == "auto" else order
    return OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                        wl.n_seq_max, wl.n_batch, wl.n_ubatch if n_ubatch is None else n_ubatch,
                        wl.causal, cell_order=order, layers=[], split_mode=wl.split_mode)


def compare_split(ctx, eng, n, pos, seqs, out):
    st, ubs, ids = ctx.split(n, pos, seqs, out, with_ids=True)
    rst, rubs, rids = eng.split(n, pos, seqs, out)
    assert st == rst
    if st:
        return ubs, rubs
    assert len(ubs) == len(rubs)
    for u, r in zip(ubs, rubs):
        assert u.src.tolist() == r.src
        assert u.pos.tolist() == r.pos
        assert u.seq_ids == [tuple(s) for s in r.seq_ids]
        assert u.output.tolist() == r.output
        assert (u.n_seq_tokens, u.n_seqs) == (r.n_seq_tokens, r.n_seqs)
        assert u.stream.tolist() == r.streams
        assert u.cells.tolist() == r.cells
        assert u.copies == [tuple(c) for c in r.copies]
        assert u.n_tokens == u.n_seq_tokens * u.n_seqs
        assert u.seq_id_unq.tolist() == sorted({s for ss in r.seq_ids for s in ss})
    assert np.array_equal(ids, rids)
    return ubs, rubs


def commit_all(ctx, eng, ubs, rubs):
    for u, r in zip(ubs, rubs):
        ctx.store(u, 0, [], [])
        eng.commit(r, build_mask=False)
        assert ctx.n_kv() == eng.cells.n_kv() == r.n_kv


def compare_tables(ctx, eng):
    for s in range(eng.n_stream):
        pos, mask = ctx.cells(s)
        assert np.array_equal(pos, eng.cells.pos[s])
        member = K.seqset_members(mask, K.MAX_SEQ)
        assert np.array_equal(member[:, :eng.n_seq_max], eng.cells.member[s])
        assert not member[:, eng.n_seq_max:].any()


def shrink(wl, layers=1):
    wl.n_layer = layers
    return wl


WORKLOADS = [
    lambda: W.tiny(),
    lambda: shrink(W.qwen_prefill(n_prompt=1300, n_layer=1, kv_size=2048, n_batch=1024, n_ubatch=256)),
    lambda: shrink(W.cb_decode(n_seq=16, lengths=(5, 9, 70, 130), n_layer=1, kv_size=2048)),
    lambda: shrink(W.mixed(n_prompt_seq=4, n_decoders=12, prompt_range=(20, 90), ctx_range=(10, 60),
                           n_layer=1, n_stream=4, kv_size=512, n_batch=128, n_ubatch=32)),
    lambda: shrink(W.prefix_decode(n_seq=8, prefix=300, private=40, n_layer=1, kv_size=1024)),
    lambda: shrink(W.prefix_decode(n_seq=8, prefix=300, private=40, n_layer=1, kv_size=512, n_stream=4)),
]


WL_IDS = ["tiny", "prefill", "cb_decode", "mixed", "prefix", "prefix_streams"]


@pytest.mark.parametrize("make", WORKLOADS, ids=WL_IDS)
def test_host_split_placement_matches_oracle(make):
    wl = make()
    ctx, eng = host_ctx(wl), oracle_for(wl)
    for bt in wl.batches:
        ubs, rubs = compare_split(ctx, eng, bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        commit_all(ctx, eng, ubs, rubs)
    compare_tables(ctx, eng)


@pytest.mark.parametrize("mode", ["simple", "equal", "seq"])
@pytest.mark.parametrize("make", WORKLOADS, ids=WL_IDS)
def test_host_split_modes_match_oracle(make, mode):
    """Each split strategy requested explicitly, on every workload shape."""
    import dataclasses
    wl = dataclasses.replace(make(), split_mode=mode)
    ctx, eng = host_ctx(wl), oracle_for(wl)
    for bt in wl.batches:
        ubs, rubs = compare_split(ctx, eng, bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        if mode == "seq":
            for u in ubs:
                assert u.n_seqs == 1 and len(set(u.seq_ids)) == 1
        commit_all(ctx, eng, ubs, rubs)
    compare_tables(ctx, eng)


def test_full_size_config_splits_match_oracle():
    # the caller calls and ubatches of the full Qwen3 prefill and the
    # full-size decode workloads (placement only, no tensors)
    for wl in (W.qwen_prefill(n_layer=1), W.cb_decode(n_layer=1), W.prefix_decode(n_layer=1)):
        ctx, eng = host_ctx(wl), oracle_for(wl)
        for bt in wl.batches:
            ubs, rubs = compare_split(ctx, eng, bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
            commit_all(ctx, eng, ubs, rubs)
        compare_tables(ctx, eng)
    pre = W.qwen_prefill(n_layer=1)
    assert [b.n_tokens for b in pre.batches] == [2048, 952]


def test_mixed_full_size_split_equal_matches_oracle():
    wl = W.mixed(n_layer=1)
    ctx, eng = host_ctx(wl), oracle_for(wl)
    first = True
    for bt in wl.batches:
        ubs, rubs = compare_split(ctx, eng, bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        if bt.measured and first:
            # one decode token per decoder plus the prompts that fit: one
            # slot from every sequence set in the first ubatch
            n_sets = len({s for s in bt.seq_ids})
            assert n_sets > 56
            assert (ubs[0].n_seqs, ubs[0].n_seq_tokens) == (n_sets, 1)
            first = False
        commit_all(ctx, eng, ubs, rubs)
    compare_tables(ctx, eng)


def test_autofill_and_defaults_match_oracle():
    ctx = K.Context(1, 2, 1, 16, kv_size=64, n_seq_max=4)
    eng = OracleEngine(1, 2, 1, 16, kv_size=64, n_seq_max=4, layers=[])
    ubs, rubs = compare_split(ctx, eng, 5, None, None, None)
    commit_all(ctx, eng, ubs, rubs)
    ubs, rubs = compare_split(ctx, eng, 4, None, [[1], [0], [1, 3], [0]], [1, 0, 0, 1])
    commit_all(ctx, eng, ubs, rubs)
    assert [u.pos.tolist() for u in ubs] == [[0, 5, 1, 6]]
    compare_tables(ctx, eng)
    assert K.kvattn_seq_pos_max(ctx.ctx, 0) == eng.cells.seq_pos_max(0) == 6
    assert K.kvattn_seq_pos_max(ctx.ctx, 2) == -1


@pytest.mark.parametrize("kv_size,n_stream,n_batch,causal", [(64, 1, 0, True), (64, 2, 100, True),
                                                             (4096, 1, 3000, True), (64, 1, 100, False)])
def test_output_ids_sized_by_library_clamp(kv_size, n_stream, n_batch, causal):
    """The binding sizes output_ids from kvattn_get_params (the library's
    clamp, "llama.cpp and the ubatch", "Three things called batch"), not from
    arithmetic of its own; the oracle's clamp must agree with it."""
    from oracle.batching import clamp_params
    ctx = K.Context(1, 2, 1, 16, kv_size=kv_size, n_stream=n_stream, n_seq_max=2, n_batch=n_batch,
                    n_ubatch=0, causal=causal)
    nb = K.kvattn_get_params(ctx.ctx).n_batch
    assert nb == clamp_params(kv_size * n_stream, n_batch, 0, causal)[0]
    assert ctx.n_batch() == nb
    st, ubs, ids = ctx.split(3, [0, 1, 2], [[0], [1], [0]], [1, 0, 1], with_ids=True)
    assert st == 0 and ids.shape == (nb,)
    assert ids[:3].tolist() == [0, -1, 1] and (ids[3:] == -1).all()


def test_seq_rm_and_reuse_match_oracle():
    wl = W.cb_decode(n_seq=6, lengths=(4, 9, 15), n_layer=1, kv_size=64)
    ctx, eng = host_ctx(wl), oracle_for(wl)
    for bt in wl.batches:
        ubs, rubs = compare_split(ctx, eng, bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        commit_all(ctx, eng, ubs, rubs)
    for args in ((2, -1, -1), (4, 3, 7), (-1, 10, -1)):
        ctx.seq_rm(*args)
        eng.seq_rm(*args)
        compare_tables(ctx, eng)
    ubs, rubs = compare_split(ctx, eng, 3, [20, 21, 22], [[1], [2], [3]], None)
    commit_all(ctx, eng, ubs, rubs)
    compare_tables(ctx, eng)


def test_split_invariance_of_placement():
    for nub in (512, 64, 7, 1):
        wl = W.qwen_prefill(n_prompt=150, n_layer=1, kv_size=512, n_batch=100, n_ubatch=nub)
        ctx = host_ctx(wl)
        for bt in wl.batches:
            st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
            assert [u.n_tokens for u in ubs] == [min(nub, bt.n_tokens - a) for a in range(0, bt.n_tokens, nub)]
            for u in ubs:
                ctx.store(u, 0, [], [])
        pos, _ = ctx.cells(0)
        assert pos[:150].tolist() == list(range(150)) and (pos[150:] == -1).all()


def test_error_codes():
    ctx = K.Context(1, 2, 1, 16, kv_size=8, n_seq_max=3, n_batch=6, n_ubatch=4)
    with pytest.raises(K.KvattnError) as e:
        ctx.split(7)                                      # more than n_batch
    assert e.value.code == K.KVATTN_EINVAL
    for pos, seqs in (([0], [[3]]), ([-1], [[0]]), ([0], [[]])):
        with pytest.raises(K.KvattnError) as e:
            ctx.split(1, pos, seqs)
        assert e.value.code == K.KVATTN_EINVAL
    st, ubs, _ = ctx.split(6)
    assert st == 0 and [u.n_tokens for u in ubs] == [4, 2]
    with pytest.raises(K.KvattnError) as e:
        ctx.store(ubs[1], 0, [], [])                      # out of order
    assert e.value.code == K.KVATTN_ESTATE
    ctx.store(ubs[0], 0, [], [])
    ctx.store(ubs[1], 0, [], [])
    before = ctx.cells(0)
    st, ubs2, _ = ctx.split(3)                            # 2 cells left: nothing reserved
    assert st == K.KVATTN_NO_SLOT and ubs2 == []
    after = ctx.cells(0)
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    st, ubs3, _ = ctx.split(2)
    assert st == 0 and ubs3[0].cells.tolist() == [6, 7]
    with pytest.raises(K.KvattnError) as e:
        ctx.store(ubs[0], 0, [], [])                      # stale handle from an earlier split
    assert e.value.code == K.KVATTN_ESTATE
    # a device call on a host-only context
    with pytest.raises(K.KvattnError) as e:
        ctx.attend(ubs3[0], 0, [], [])
    assert e.value.code == K.KVATTN_ENODEV
    # streams: a slot whose ids live in two streams is stored in both
    c2 = K.Context(1, 2, 1, 16, kv_size=8, n_stream=2, n_seq_max=4)
    st, ubs, _ = c2.split(2, [0, 1], [[1, 0, 2], [3]])
    assert st == 0 and ubs[0].copies == [(0, 0, 0)] and ubs[0].stream.tolist() == [1, 1]
    assert ubs[0].cells.tolist() == [0, 1]
    # bad parameters
    with pytest.raises(K.KvattnError):
        K.Context(1, 3, 2, 16, kv_size=8)                 # n_head not a multiple
    with pytest.raises(K.KvattnError):
        K.Context(1, 2, 1, 24, kv_size=8)                 # unsupported head_dim
    with pytest.raises(K.KvattnError):
        K.Context(1, 2, 1, 16, kv_size=8, n_seq_max=257)   # more than 256 sequences
    with pytest.raises(K.KvattnError):
        K.Context(1, 2, 1, 16, kv_size=4, cell_order=[0, 1, 1, 2])


def test_time_next_attend_arguments():
    """Kernel timing is armed per context and checked on the host: unknown
    kinds and NULL events are refused; a failing attend call disarms it."""
    ctx = K.Context(1, 2, 1, 16, kv_size=8, n_ubatch=4)
    for kind, e0, e1 in ((3, 1, 2), (K.KVATTN_KERNEL_MFMA, 0, 2), (K.KVATTN_KERNEL_VALU, 1, 0)):
        with pytest.raises(K.KvattnError) as e:
            K.kvattn_time_next_attend(ctx.ctx, kind, e0, e1)
        assert e.value.code == K.KVATTN_EINVAL
    K.kvattn_time_next_attend(ctx.ctx, -1, 0, 0)          # disarm: always accepted
    # armed with stand-in handles: the host-only attend fails before any
    # launch, so the handles are never used, and the call clears them
    K.kvattn_time_next_attend(ctx.ctx, K.KVATTN_KERNEL_MERGE, 1, 2)
    st, ubs, _ = ctx.split(2)
    ctx.store(ubs[0], 0, [], [])
    with pytest.raises(K.KvattnError) as e:
        ctx.attend(ubs[0], 0, [], [])
    assert e.value.code == K.KVATTN_ENODEV


def test_probe_arguments_refused_on_the_host():
    """The ceiling probes check their arguments before any launch."""
    for args in ((0, 10, 1, 10, 1, 4), (1, 0, 1, 10, 1, 4), (1, 10, 0, 10, 1, 4), (1, 10, 1, 10, 0, 4),
                 (1, 10, 1, 10, 1, 0), (1, 10, 1, -1, 1, 4)):
        with pytest.raises(K.KvattnError) as e:
            K.kvattn_probe_gather(*args)
        assert e.value.code == K.KVATTN_EINVAL
    for args in ((0, 1, 4, 10), (1, 0, 4, 10), (1, 1, 0, 10), (1, 1, 4, -1)):
        with pytest.raises(K.KvattnError) as e:
            K.kvattn_probe_mfma(*args)
        assert e.value.code == K.KVATTN_EINVAL


def test_empty_batch_and_uncommitted_release():
    ctx = K.Context(1, 2, 1, 16, kv_size=8, n_ubatch=4)
    st, ubs, _ = ctx.split(0)
    assert st == 0 and ubs == []
    st, ubs, _ = ctx.split(8)
    assert st == 0 and len(ubs) == 2
    ctx.store(ubs[0], 0, [], [])
    # a new split releases the never-stored second ubatch's cells
    st, ubs, _ = ctx.split(4)
    assert st == 0 and ubs[0].cells.tolist() == [4, 5, 6, 7]


def test_workspace_and_cache_bytes():
    p = K.kvattn_params()
    p.n_layer, p.n_head, p.n_head_kv, p.head_dim, p.kv_size = 28, 16, 8, 128, 4096
    p.n_stream, p.n_seq_max, p.n_ubatch = 1, 1, 512
    assert K.kvattn_cache_bytes(p) == 448 * 2 ** 20
    ws = K.kvattn_workspace_bytes(p)
    assert 0 < ws < 512 * 2 ** 20
    p.head_dim = 24
    assert K.kvattn_workspace_bytes(p) == 0


@pytest.mark.parametrize("kw", [dict(head_dim=48), dict(n_head=3, n_head_kv=2), dict(n_head=32, n_head_kv=2),
                                dict(n_seq_max=257), dict(kv_size=0), dict(split_mode=4), dict(split_mode=-1), dict(swa_window=-1),
                                # one layer's K tensor at 2 GiB: 2^20 cells x 8 heads x 128 x 2 B
                                dict(kv_size=1 << 20, n_head=8, n_head_kv=8, head_dim=128)])
def test_create_rejects_bad_geometry(kw):
    args = dict(n_layer=1, n_head=2, n_head_kv=1, head_dim=16, kv_size=64, n_seq_max=1)
    args.update(kw)
    with pytest.raises(K.KvattnError) as e:
        K.Context(args.pop("n_layer"), args.pop("n_head"), args.pop("n_head_kv"), args.pop("head_dim"), **args)
    assert e.value.code == K.KVATTN_EINVAL


def test_create_accepts_largest_layer_tensor():
    # just below 2 GiB per layer tensor: (2^20 - 64) cells x 1024 numbers x 2 B
    ctx = K.Context(1, 8, 8, 128, kv_size=(1 << 20) - 64, n_seq_max=1)
    assert 0 < ctx.n_kv() <= (1 << 20) - 64


def test_seq_state_size_matches_oracle():
    from oracle import seqstate as S
    wl = W.prefix_decode(n_seq=4, prefix=20, private=5, n_layer=2, kv_size=128)
    ctx, eng = host_ctx(wl), oracle_for(wl)
    for bt in wl.batches:
        ubs, rubs = compare_split(ctx, eng, bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        commit_all(ctx, eng, ubs, rubs)
    ctx.seq_rm(2, 22, -1)
    eng.seq_rm(2, 22, -1)
    for seq in range(wl.n_seq_max):
        n = len(S.sequence_cells(eng, seq)[1])
        assert ctx.state_size(seq) == S.state_bytes(wl.n_layer, wl.n_head_kv, wl.head_dim, n)
    n0 = 20 + 5 + 1                            # shared prefix, private cells, the decode token
    assert ctx.state_size(0) == 80 + 4 * n0 + 2 * 2 * (12 + n0 * wl.E * 2)
    with pytest.raises(K.KvattnError):
        ctx.state_size(wl.n_seq_max)
    # save / load need the GPU
    with pytest.raises(K.KvattnError) as e:
        K.kvattn_seq_state_save(ctx.ctx, 0, 4096, 1 << 20)
    assert e.value.code == K.KVATTN_ENODEV
    with pytest.raises(K.KvattnError) as e:
        K.kvattn_seq_state_load(ctx.ctx, 0, 4096, 1 << 20)
    assert e.value.code == K.KVATTN_ENODEV


@pytest.mark.parametrize("seed", range(200))
def test_random_batches_match_oracle(seed):
    """Differential check on random inputs: batches of random sequence-id sets
    (shared prefixes, ids spanning streams), random positions and output
    flags or auto-fill, every split strategy, one to four streams, shuffled
    free lists, partially stored splits (the unstored ubatches' cells are
    released by the next split), retirements and full caches; half of the
    seeds map the sequences to ids spread over [0, 256).  Every ubatch's
    slots, positions, cells and copies, the status, output_ids and the
    committed cell table must equal the oracle's after every step."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 77]))
    irng = np.random.default_rng(np.random.SeedSequence([seed, 78]))
    n_stream = int(rng.choice([1, 2, 4]))
    n_seqs = int(rng.integers(2, 13))
    n_seq_max, idmap = n_seqs, list(range(n_seqs))
    if irng.random() < 0.5:                 # a wide id space
        n_seq_max = int(irng.integers(65, K.MAX_SEQ + 1))
        idmap = [int(x) for x in irng.choice(n_seq_max, size=n_seqs, replace=False)]
    kv_size = int(rng.choice([24, 48, 96]))
    n_batch = int(rng.choice([8, 16, 32]))
    n_ubatch = int(rng.choice([3, 4, 8, 16]))
    mode = str(rng.choice(["auto", "simple", "equal", "seq"]))
    order = (np.stack([rng.permutation(kv_size) for _ in range(n_stream)]).astype(np.int32)
             if rng.random() < 0.5 else None)
    ctx = K.Context(1, 2, 1, 16, kv_size, n_stream, n_seq_max, n_batch, n_ubatch, cell_order=order,
                    split_mode=mode)
    eng = OracleEngine(1, 2, 1, 16, kv_size, n_stream, n_seq_max, n_batch, n_ubatch, cell_order=order,
                       layers=[], split_mode=mode)
    nb = ctx.n_batch()
    next_pos = [0] * n_seqs
    for step in range(12):
        if step and rng.random() < 0.25:
            who = int(rng.integers(-1, n_seqs))
            args = (idmap[who] if who >= 0 else -1, int(rng.integers(-1, 8)), int(rng.integers(-1, 40)))
            ctx.seq_rm(*args)
            eng.seq_rm(*args)
            compare_tables(ctx, eng)
            continue
        n = int(rng.integers(0, nb + 1))
        seqs, pos = [], []
        for _ in range(n):
            first = int(rng.integers(0, n_seqs))
            ids = [first]
            if rng.random() < 0.2:          # a shared slot: extra ids (possibly in other streams)
                extra = rng.choice(n_seqs, size=int(rng.integers(1, min(3, n_seqs) + 1)), replace=False)
                ids += [int(x) for x in extra if int(x) != first]
            seqs.append([idmap[i] for i in ids])
            pos.append(next_pos[first] if rng.random() < 0.8 else int(rng.integers(0, 64)))
            next_pos[first] = pos[-1] + 1
        out = (rng.random(n) < 0.3).astype(np.int8).tolist()
        if rng.random() < 0.15:
            pos_arg, out_arg = None, None       # auto-fill positions and output flags
        else:
            pos_arg, out_arg = pos, out
        ubs, rubs = compare_split(ctx, eng, n, pos_arg, seqs, out_arg)
        if ubs:
            keep = len(ubs) if rng.random() < 0.8 else int(rng.integers(0, len(ubs) + 1))
            commit_all(ctx, eng, ubs[:keep], rubs[:keep])
        compare_tables(ctx, eng)
