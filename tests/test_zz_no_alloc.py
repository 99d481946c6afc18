"""kvattn_attend_noalloc: the allocation-free variant of kvattn_attend.

Its split-K partials live in the library's static device array instead of
the workspace; the kernels and the plan are the same, so its outputs must
equal kvattn_attend's bit for bit.  Two calls in a row on one GPU, the second
with a smaller input (the array still holds the first call's partials), plus
the refusal of a plan whose partial rows per layer exceed the array.
"""

import numpy as np
import pytest

from synthetic import workloads as W
from tests.helpers import assert_parity, batch_tensors, make_ctx

pytestmark = pytest.mark.gpu


def both_entry_points(wl, layers):
    """Store every batch; for the measured one attend over all ``layers`` in
    one call through kvattn_attend and through kvattn_attend_noalloc.
    Returns (plan stats, [(attend, noalloc) float64 per layer])."""
    import torch
    from ubatch_attention_paged_amd.harness import ubatch_rows
    dev = torch.device("cuda:0")
    ctx = make_ctx(wl, attend_layers=len(layers))
    HD = wl.n_head * wl.head_dim
    pairs, stats = [], None
    for b, bt in enumerate(wl.batches):
        t = batch_tensors(wl, b, layers, bt.measured)
        K = [torch.from_numpy(t[(l, W.KIND_K)]).to(dev) for l in layers]
        V = [torch.from_numpy(t[(l, W.KIND_V)]).to(dev) for l in layers]
        st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0
        for ub in ubs:
            ctx.store(ub, layers[0], [ubatch_rows(ub, x) for x in K], [ubatch_rows(ub, x) for x in V])
            if not bt.measured:
                continue
            Q = [ubatch_rows(ub, torch.from_numpy(t[(l, W.KIND_Q)]).to(dev)) for l in layers]
            oa = [torch.full((ub.n_tokens, HD), float("nan"), device=dev) for _ in layers]
            ob = [torch.full((ub.n_tokens, HD), float("nan"), device=dev) for _ in layers]
            ctx.attend(ub, layers[0], Q, oa)
            ctx.attend_noalloc(ub, layers[0], Q, ob)
            torch.cuda.synchronize()
            stats = ctx.plan_stats()
            pairs += [(x.double().cpu().numpy(), y.double().cpu().numpy()) for x, y in zip(oa, ob)]
    ctx.close()
    return stats, pairs


def test_noalloc_matches_attend_twice_second_smaller():
    # first call: 32 sequences sharing a 1024-cell prefix, 28 layers in one
    # attend call -> ~96 partial rows per layer, so the static array (2016
    # rows of this head shape) holds 21 layers per launch: two launches
    big = W.prefix_decode(n_seq=32, prefix=1024, private=128, n_layer=28, kv_size=8192)
    small = W.prefix_decode(n_seq=8, prefix=256, private=64, n_layer=3, kv_size=2048)
    for wl, name in ((big, "first (32 sequences, 28 layers)"), (small, "second (8 sequences, 3 layers)")):
        print(f"no-alloc attend: {name}", flush=True)
        stats, pairs = both_entry_points(wl, list(range(wl.n_layer)))
        assert stats["n_partial_rows"] > 0 and stats["n_reduced"] == wl.batches[-1].n_tokens, stats
        if wl is big:
            assert 2016 // stats["n_partial_rows"] < wl.n_layer, stats
        for l, (a, b) in enumerate(pairs):
            assert np.isfinite(a).all() and np.isfinite(b).all(), (name, l)
            assert_parity(b, a, tag=f"{name} layer {l}")
            assert np.array_equal(a, b), f"{name} layer {l}: same kernels and plan, results must be identical"


def test_noalloc_refuses_partials_beyond_the_array():
    """64 KV heads x 128 with 8 query heads each: one partial row is 264 KiB,
    so the 16 MiB array holds 63 rows.  8 sequences sharing a 65536-cell
    prefix cut into 16 chunks give 136 rows per layer: refused with
    KVATTN_ENOMEM before anything is launched (the output stays untouched),
    while kvattn_attend's workspace holds them."""
    import torch
    import ubatch_attention_paged_amd as K
    dev = torch.device("cuda:0")
    n_seq, prefix, hkv, d, g = 8, 65536, 64, 128, 8
    ctx = K.Context(1, hkv * g, hkv, d, kv_size=prefix + 256, n_seq_max=n_seq, n_batch=2048, n_ubatch=2048,
                    device="cuda:0", attend_layers=1)
    E = hkv * d
    zeros = torch.zeros((2048, E), dtype=torch.float32, device=dev)
    everyone = [tuple(range(n_seq))] * 2048
    for a in range(0, prefix, 2048):
        st, ubs, _ = ctx.split(2048, np.arange(a, a + 2048), everyone, np.zeros(2048, np.int8))
        assert st == 0
        for ub in ubs:
            ctx.store(ub, 0, [zeros[:ub.n_tokens]], [zeros[:ub.n_tokens]])
    st, ubs, _ = ctx.split(n_seq, [prefix] * n_seq, [(i,) for i in range(n_seq)], [1] * n_seq)
    assert st == 0 and len(ubs) == 1
    ub = ubs[0]
    ctx.store(ub, 0, [zeros[:n_seq]], [zeros[:n_seq]])
    rows = ctx.plan_stats()["n_partial_rows"]
    assert rows > 63, rows
    q = torch.zeros((n_seq, hkv * g * d), dtype=torch.float32, device=dev)
    out = torch.full((n_seq, hkv * g * d), 7.0, device=dev)
    with pytest.raises(K.KvattnError) as ei:
        ctx.attend_noalloc(ub, 0, [q], [out])
    assert ei.value.code == K.KVATTN_ENOMEM and "exceed" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    ctx.close()


def test_noalloc_under_hip_graph_capture():
    """The caller it is for: a decode step's attention captured into a HIP
    graph (torch.cuda.graph) and replayed.  Every replay, with eager work and
    synchronisations between replays, equals the eager call bit for bit (the
    captured launches read the plan and partials in place; nothing in the
    call allocates or writes memory outside the kernels)."""
    import torch
    import ubatch_attention_paged_amd as K
    from ubatch_attention_paged_amd.harness import ubatch_rows
    dev = torch.device("cuda:0")
    wl = W.prefix_decode(n_seq=8, prefix=256, private=64, n_layer=3, kv_size=2048)
    layers = list(range(wl.n_layer))
    ctx = make_ctx(wl, attend_layers=len(layers))
    HD = wl.n_head * wl.head_dim
    checked = 0
    for b, bt in enumerate(wl.batches):
        t = batch_tensors(wl, b, layers, bt.measured)
        Kt = [torch.from_numpy(t[(l, W.KIND_K)]).to(dev) for l in layers]
        Vt = [torch.from_numpy(t[(l, W.KIND_V)]).to(dev) for l in layers]
        st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0
        for ub in ubs:
            ctx.store(ub, 0, [ubatch_rows(ub, x) for x in Kt], [ubatch_rows(ub, x) for x in Vt])
            if not bt.measured:
                continue
            Q = [ubatch_rows(ub, torch.from_numpy(t[(l, W.KIND_Q)]).to(dev)) for l in layers]
            ref = [torch.full((ub.n_tokens, HD), float("nan"), device=dev) for _ in layers]
            ctx.attend_noalloc(ub, 0, Q, ref)
            torch.cuda.synchronize()
            assert ctx.plan_stats()["n_reduced"] > 0       # split-K partials in the static array
            out = [torch.full_like(r, float("nan")) for r in ref]
            print("[gpu] capturing kvattn_attend_noalloc into a HIP graph", flush=True)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                ctx.attend_noalloc(ub, 0, Q, out)
            scratch = [torch.full_like(r, float("nan")) for r in ref]
            for rep in range(3):
                for o in out:
                    o.fill_(float("nan"))
                graph.replay()
                torch.cuda.synchronize()
                assert all(torch.equal(a, c) for a, c in zip(ref, out)), f"replay {rep}"
                # eager work between replays: the workspace entry point into other buffers
                ctx.attend(ub, 0, Q, scratch)
                torch.cuda.synchronize()
                assert_parity(scratch[0].double().cpu().numpy(), ref[0].double().cpu().numpy(), tag="eager")
            checked += 1
            del graph
    assert checked == 1
    ctx.close()
