"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Cache bytes, the dense mask and the per-class cell lists must match bit for
bit; attention outputs must satisfy |g - r| <= 2e-3 + 5e-3 |r| elementwise
(and the tighter per-kernel bounds below, which catch a dropped cell that the
tolerance alone would let through).  Sizes here span several 64-cell tiles,
several q-tiles and ragged tails while the oracle stays within seconds.
"""

import numpy as np
import pytest

from synthetic import workloads as W
from tests.helpers import MFMA_BOUND, VALU_BOUND, assert_parity, gpu_run, make_ctx, model_for, oracle_run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
K = pytest.importorskip("ubatch_attention_paged_amd")


def small(name):
    if name == "tiny":
        return W.tiny()
    if name == "prefill":
        return W.qwen_prefill(n_prompt=700, n_layer=2, kv_size=1024, n_batch=512, n_ubatch=256)
    if name == "cb_decode":
        return W.cb_decode(n_seq=16, lengths=(5, 40, 130, 300), n_layer=2, kv_size=4096)
    if name == "mixed":
        return W.mixed(n_prompt_seq=4, n_decoders=12, prompt_range=(30, 200), ctx_range=(20, 300),
                       n_layer=2, n_stream=4, kv_size=2048, n_batch=256, n_ubatch=64)
    if name == "prefix":
        return W.prefix_decode(n_seq=8, prefix=300, private=50, n_layer=2, kv_size=1024)
    if name == "prefix32":
        return W.prefix_decode(n_seq=32, prefix=200, private=20, n_layer=1, kv_size=2048)
    if name == "d64":
        wl = W.mixed(n_prompt_seq=2, n_decoders=5, prompt_range=(40, 150), ctx_range=(10, 90),
                     n_layer=1, n_stream=1, kv_size=1024, n_batch=256, n_ubatch=100)
        wl.n_head, wl.n_head_kv, wl.head_dim = 32, 16, 64      # E = 1024, G = 2, d = 64
        return wl
    raise KeyError(name)


NAMES = ["tiny", "prefill", "cb_decode", "mixed", "prefix", "prefix32", "d64"]


def expected_classes(eng, ub):
    """Cells per (stream, sequence set) that some query of the ubatch sees,
    ascending cell index, classes ordered by (stream, set bitmask)."""
    out = []
    for s in range(eng.n_stream):
        qseqs = {ub.seq_ids[i][0] for i in range(ub.n_tokens) if ub.streams[i] == s}
        if not qseqs:
            continue
        pos = eng.cells.pos[s]
        bits = np.array([sum(1 << int(q) for q in np.nonzero(row)[0]) for row in eng.cells.member[s]], dtype=object)
        occupied = np.nonzero(pos >= 0)[0]
        masks = sorted({bits[j] for j in occupied if any(bits[j] >> q & 1 for q in qseqs)})
        for m in masks:
            out.append((s, m, occupied[bits[occupied] == m]))
    return out


@pytest.mark.parametrize("name", NAMES)
def test_end_to_end_parity(name):
    wl = small(name)
    layers = list(range(wl.n_layer))
    print(f"[gpu] end_to_end {name}: {wl.note}", flush=True)
    eng, ref, masks, meta = oracle_run(wl, layers, keep_masks=True)
    seen = {"mask": 0, "classes": 0}

    def check(ctx, b, ub):
        u = ub_index[b]
        r = meta[(b, u)]
        assert ub.cells.tolist() == r.cells
        m = ctx.mask(ub).cpu().numpy().view(np.uint16)
        assert m.shape == masks[(b, u)].shape
        assert np.array_equal(m, masks[(b, u)].view(np.uint16)), f"mask differs (batch {b}, ubatch {u})"
        seen["mask"] += 1
        ub_index[b] += 1

    ub_index = {b: 0 for b in range(len(wl.batches))}
    ctx, got = gpu_run(wl, layers, on_ubatch=check)
    assert seen["mask"] == len(meta)
    worst, worst_rel = 0.0, 0.0
    for key in ref:
        ma, mr = assert_parity(got[key], ref[key], tag=f"{name} batch {key[0]} layer {key[1]}", **ref.model(key))
        worst, worst_rel = max(worst, ma), max(worst_rel, mr)
    # tighter than the tolerance: the fp32 vector-ALU path (decode-only
    # workloads) agrees to ~1e-6; the MFMA path rounds q and the softmax
    # weights to F16 (relative 2^-11)
    print(f"[gpu] end_to_end {name}: max abs error {worst:.3e}, "
          f"max rel error {worst_rel:.3e} over |ref| >= 1e-2", flush=True)
    if name == "cb_decode":
        assert worst < VALU_BOUND, worst     # fp32 throughout on the vector-ALU path
    # cache bytes: every committed cell row equals the oracle's F16 rounding
    for l in layers:
        gk = ctx.K[l].cpu().numpy().view(np.uint16)
        gv = ctx.V[l].cpu().numpy().view(np.uint16)
        occ = eng.cells.pos >= 0
        assert np.array_equal(gk[occ], eng.K[l][occ].view(np.uint16))
        assert np.array_equal(gv[occ], eng.V[l][occ].view(np.uint16))
    ctx.close()


HEAD_SHAPES = [(d, g) for d in (16, 32, 64, 128) for g in (1, 2, 4, 8)]   # every compiled instance


@pytest.mark.parametrize("swa", [0, 60])
@pytest.mark.parametrize("d,g", HEAD_SHAPES)
def test_mfma_head_shapes(d, g, swa):
    """Every head size and query-head group the matrix-core kernel is built
    for.  Its LDS tile layout differs per head size (row length, segment
    swizzle, and below 32 the zero V columns the transpose reads cover), so
    each runs prompt ubatches long enough for matrix-core work items, with
    ragged tails, against the oracle."""
    wl = W.mixed(n_prompt_seq=2, n_decoders=4, prompt_range=(70, 200), ctx_range=(10, 90), n_layer=1,
                 n_stream=1, kv_size=1024, n_batch=256, n_ubatch=128)
    wl.n_head, wl.n_head_kv, wl.head_dim = 2 * g, 2, d
    wl.swa = swa              # 60 positions: prompts of up to 200 tokens skip their leading tiles
    layers = [0]
    print(f"[gpu] head shape d={d} g={g} window {swa}: {wl.note}", flush=True)
    _, ref, _, _ = oracle_run(wl, layers, keep_masks=False)
    items = {"mfma": 0}

    def count(ctx, b, ub):
        items["mfma"] += ctx.plan_stats()["n_items_mfma"]

    ctx, got = gpu_run(wl, layers, on_ubatch=count)
    worst = 0.0
    for key in ref:
        ma, _ = assert_parity(got[key], ref[key], tag=f"d={d} g={g} window {swa} batch {key[0]}", **ref.model(key))
        worst = max(worst, ma)
    print(f"[gpu] head shape d={d} g={g} window {swa}: max abs error {worst:.3e}", flush=True)
    assert items["mfma"] > 0
    ctx.close()


@pytest.mark.parametrize("d,g,hk", [(128, 1, 8), (128, 4, 8), (64, 1, 16), (64, 4, 16),
                                    (128, 2, 4), (64, 1, 8), (128, 4, 4),
                                    (128, 2, 16), (64, 4, 32), (128, 1, 32), (64, 2, 64)])
def test_valu_head_shapes(d, g, hk):
    """The vector-ALU decode kernel's other (head_dim, group, row width)
    instances (the workloads above run group 2 over 1024-number rows): lanes
    map to KV heads differently per head size, the group sets how many query
    heads each lane's K/V feeds, 512-number rows put two cells in one
    wavefront load (lane halves, merged at the end), and 2048 / 4096-number
    rows split each row between wavefront groups.  Contexts up to 300 cells
    are cut into split-K chunks, so the merge runs too."""
    wl = W.cb_decode(n_seq=16, lengths=(5, 40, 130, 300), n_layer=1, kv_size=4096)
    wl.n_head_kv = hk
    wl.n_head = wl.n_head_kv * g
    wl.head_dim = d
    layers = [0]
    print(f"[gpu] vector-ALU head shape d={d} g={g} kv heads {hk} (row {d * hk})", flush=True)
    _, ref, _, _ = oracle_run(wl, layers)
    items = {"valu": 0}

    def count(ctx, b, ub):
        items["valu"] += ctx.plan_stats()["n_items_valu"]

    ctx, got = gpu_run(wl, layers, on_ubatch=count)
    worst = 0.0
    for key in ref:
        ma, _ = assert_parity(got[key], ref[key], tag=f"d={d} g={g} hk={hk} batch {key[0]}", **ref.model(key))
        worst = max(worst, ma)
    assert items["valu"] > 0
    assert worst < 2e-5, worst      # fp32 throughout on this path
    ctx.close()


@pytest.mark.parametrize("hk", [4, 16])
def test_prefix_sharing_other_row_widths(hk):
    """Shared-prefix decode with 512- and 2048-number rows: the prefix runs
    on the matrix cores, the private tails on the vector ALUs (two cells per
    wavefront load, or a row split between wavefront groups), the merge
    combines them."""
    wl = W.prefix_decode(n_seq=8, prefix=300, private=50, n_layer=1, kv_size=1024)
    wl.n_head_kv = hk
    wl.n_head = 2 * hk
    layers = [0]
    print(f"[gpu] prefix sharing, {hk} KV heads x 128", flush=True)
    _, ref, _, _ = oracle_run(wl, layers)
    kinds = {"valu": 0, "mfma": 0, "red": 0}

    def count(ctx, b, ub):
        st = ctx.plan_stats()
        kinds["valu"] += st["n_items_valu"]
        kinds["mfma"] += st["n_items_mfma"]
        kinds["red"] += st["n_reduced"]

    ctx, got = gpu_run(wl, layers, on_ubatch=count)
    for key in ref:
        assert_parity(got[key], ref[key], tag=f"hk={hk} batch {key[0]}", **ref.model(key))
    assert kinds["valu"] > 0 and kinds["mfma"] > 0 and kinds["red"] > 0, kinds
    ctx.close()


@pytest.mark.parametrize("swa", [0, 4500])
def test_mfma_long_context_items(swa):
    """Matrix-core items longer than 64 tiles: a 5200-token context is stored
    unmeasured, then a 100-token chunk attends over all 5300 cells (83 tiles
    per item, so the causal tile trimming strides lanes more than once and
    the LDS ring turns over 80 times); with a 4500-position sliding window the
    walk starts past the first tiles."""
    batches = (W._prompt_batches((0,), 0, 5200, 1024, measured=False) +
               W._prompt_batches((0,), 5200, 100, 1024, measured=True))
    wl = W.Workload("long_context", 1, 4, 2, 64, kv_size=8192, n_stream=1, n_seq_max=1, seed=2601,
                    batches=batches, n_batch=1024, n_ubatch=512, swa=swa,
                    note=f"5200-token context + 100-token chunk, window {swa}")
    layers = [0]
    print(f"[gpu] long-context items: {wl.note}", flush=True)
    _, ref, _, _ = oracle_run(wl, layers)
    items = {"mfma": 0}

    def count(ctx, b, ub):
        items["mfma"] += ctx.plan_stats()["n_items_mfma"]

    ctx, got = gpu_run(wl, layers, on_ubatch=count)
    assert len(ref) == 1
    for key in ref:
        assert_parity(got[key], ref[key], tag=f"long context, window {swa}", **ref.model(key))
    assert items["mfma"] > 0
    ctx.close()


@pytest.mark.parametrize("name", ["prefill", "cb_decode", "mixed", "prefix32"])
def test_class_lists_bit_exact(name):
    wl = small(name)
    print(f"[gpu] class lists {name}", flush=True)
    eng, _, _, meta = oracle_run(wl, [0], keep_masks=False, sigma=False)
    # replay the placement on the GPU, checking the lists after every commit
    eng2, _, _, _ = None, None, None, None
    from oracle import OracleEngine
    eng2 = OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                        wl.n_seq_max, wl.n_batch, wl.n_ubatch, wl.causal, cell_order=wl.cell_order, layers=[])
    ctx = make_ctx(wl)
    dev = torch.device("cuda:0")
    E = wl.E
    checked = 0
    for b, bt in enumerate(wl.batches):
        st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        _, rubs, _ = eng2.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        zeros = torch.zeros((max(u.n_tokens for u in ubs), E), device=dev)
        for ub, r in zip(ubs, rubs):
            ctx.store(ub, 0, [zeros[:ub.n_tokens]], [zeros[:ub.n_tokens]])
            eng2.commit(r, build_mask=False)
            got = ctx.classes()
            exp = expected_classes(eng2, r)
            assert [(s, m) for s, m, _ in got] == [(s, m) for s, m, _ in exp]
            for (_, _, cg), (_, _, ce) in zip(got, exp):
                assert np.array_equal(cg, ce)
            checked += 1
    assert checked == len(meta)
    ctx.close()


def test_only_outputs_and_layer_chunks():
    wl = small("mixed")
    layers = [0, 1]
    print("[gpu] only_outputs / layer chunks", flush=True)
    _, ref, _, _ = oracle_run(wl, layers)
    _, full = gpu_run(wl, layers, layer_chunk=2)
    _, per_layer = gpu_run(wl, layers, layer_chunk=1)
    _, outs = gpu_run(wl, layers, only_outputs=True)
    for key in ref:
        # items are sized for the layers per call (one layer per call may cut
        # prompt classes into chunks merged by split-K), so the two agree to
        # rounding, and each against the oracle
        assert_parity(per_layer[key], ref[key], tag=f"one layer per call {key}", **ref.model(key))
        assert np.abs(per_layer[key] - full[key]).max() < MFMA_BOUND
        b = key[0]
        flagged = np.nonzero(wl.batches[b].output)[0]
        assert_parity(outs[key], ref[key], rows=flagged, tag=f"only_outputs {key}", **ref.model(key))
        # fewer query rows can move a class from the MFMA kernel to the fp32
        # vector kernel, so the two runs agree to rounding, not bit for bit
        assert np.abs(outs[key][flagged] - full[key][flagged]).max() < MFMA_BOUND


@pytest.mark.parametrize("n_prompt", [700, 1200])
def test_prompt_split_k_one_layer_per_call(n_prompt):
    """One layer per attend call: a prompt ubatch's 128-row matrix-core items
    alone would leave most of the GPU idle, so their cell lists are cut into
    chunks (multiples of the 64-cell tile) whose partial softmax states the
    merge kernel combines -- including chunks wholly in the future of an
    item's queries, which contribute nothing."""
    wl = W.qwen_prefill(n_prompt=n_prompt, n_layer=2, kv_size=2048, n_batch=n_prompt, n_ubatch=512)
    layers = [0, 1]
    print(f"[gpu] prompt split-K, {n_prompt} tokens, one layer per call", flush=True)
    _, ref, _, _ = oracle_run(wl, layers)
    split = {"rows": 0}

    def count(ctx, b, ub):
        split["rows"] = max(split["rows"], ctx.plan_stats()["n_partial_rows"])

    ctx, got = gpu_run(wl, layers, layer_chunk=1, on_ubatch=count)
    assert split["rows"] > 0
    worst = 0.0
    for key in ref:
        ma, _ = assert_parity(got[key], ref[key], tag=f"prompt split-K {n_prompt} {key}", **ref.model(key))
        worst = max(worst, ma)
    print(f"[gpu] prompt split-K {n_prompt}: max abs error {worst:.3e}", flush=True)
    ctx.close()


@pytest.mark.parametrize("n_ubatch", [512, 64, 7])
def test_split_invariance(n_ubatch):
    wl = W.qwen_prefill(n_prompt=300, n_layer=1, kv_size=512, n_batch=256, n_ubatch=512)
    print(f"[gpu] split invariance n_ubatch={n_ubatch}", flush=True)
    _, ref, _, _ = oracle_run(wl, [0])
    _, got = gpu_run(wl, [0], n_ubatch=n_ubatch)
    for key in ref:
        assert_parity(got[key], ref[key], tag=f"n_ubatch {n_ubatch}", **ref.model(key))


def test_repeat_store_attend_is_idempotent():
    wl = small("cb_decode")
    print("[gpu] idempotent replay", flush=True)
    ctx = make_ctx(wl)
    dev = torch.device("cuda:0")
    from tests.helpers import batch_tensors
    for b, bt in enumerate(wl.batches):
        t = batch_tensors(wl, b, [0, 1], bt.measured)
        Kt = [torch.from_numpy(t[(l, W.KIND_K)]).to(dev) for l in (0, 1)]
        Vt = [torch.from_numpy(t[(l, W.KIND_V)]).to(dev) for l in (0, 1)]
        st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert len(ubs) == 1
        ctx.store(ubs[0], 0, Kt, Vt)
        if bt.measured:
            Q = [torch.from_numpy(t[(l, W.KIND_Q)]).to(dev) for l in (0, 1)]
            o1 = [torch.empty_like(q) for q in Q]
            o2 = [torch.empty_like(q) for q in Q]
            ctx.attend(ubs[0], 0, Q, o1)
            for _ in range(3):
                ctx.store(ubs[0], 0, Kt, Vt)
                ctx.attend(ubs[0], 0, Q, o2)
            torch.cuda.synchronize()
            for a, c in zip(o1, o2):
                assert torch.equal(a, c)
    ctx.close()


@pytest.mark.parametrize("name", ["prefix", "cb_decode"])
def test_kernel_timing_events_change_nothing(name):
    """Arming kernel timing (hipExtLaunchKernel start/stop events) leaves the
    results bit-identical (for the shared-prefix plan, timing the matrix-core
    or the vector-ALU kernel turns the combined launch into two); a timed
    kernel's elapsed time is positive and
    within the events around the whole call; a kind the call does not launch
    gets both events back to back (about zero)."""
    wl = small(name)
    print(f"[gpu] kernel timing events {name}", flush=True)
    ctx = make_ctx(wl)
    dev = torch.device("cuda:0")
    from tests.helpers import batch_tensors
    layers = list(range(wl.n_layer))
    checked = 0
    for b, bt in enumerate(wl.batches):
        t = batch_tensors(wl, b, layers, bt.measured)
        Kt = [torch.from_numpy(t[(l, W.KIND_K)]).to(dev) for l in layers]
        Vt = [torch.from_numpy(t[(l, W.KIND_V)]).to(dev) for l in layers]
        st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0 and len(ubs) == 1
        ub = ubs[0]
        ctx.store(ub, 0, Kt, Vt)
        if not bt.measured:
            continue
        Q = [torch.from_numpy(t[(l, W.KIND_Q)]).to(dev) for l in layers]
        ref = [torch.empty_like(q) for q in Q]
        ctx.attend(ub, 0, Q, ref)
        stats = ctx.plan_stats()
        launched = {K.KVATTN_KERNEL_MFMA: stats["n_items_mfma"] > 0, K.KVATTN_KERNEL_VALU: stats["n_items_valu"] > 0,
                    K.KVATTN_KERNEL_MERGE: stats["n_reduced"] > 0}
        for kind, has in launched.items():
            k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0.record()
            k1.record()                        # creates the HIP events
            K.kvattn_time_next_attend(ctx.ctx, kind, k0.cuda_event, k1.cuda_event)
            out = [torch.full_like(q, float("nan")) for q in Q]
            c0.record()
            ctx.attend(ub, 0, Q, out)
            c1.record()
            torch.cuda.synchronize()
            for a, c in zip(ref, out):
                assert torch.equal(a, c)
            kt, ct = k0.elapsed_time(k1), c0.elapsed_time(c1)
            print(f"  kind {kind} launched {has}: kernel {kt:.4f} ms, call {ct:.4f} ms", flush=True)
            if has:
                assert 0 < kt <= ct
            else:
                assert 0 <= kt < 0.05
            checked += 1
        # an untimed call afterwards is unaffected by the earlier arming
        out = [torch.full_like(q, float("nan")) for q in Q]
        ctx.attend(ub, 0, Q, out)
        torch.cuda.synchronize()
        assert all(torch.equal(a, c) for a, c in zip(ref, out))
    assert checked == 3
    ctx.close()


@pytest.mark.parametrize("hk,g,d", [(8, 2, 128), (4, 2, 128), (8, 1, 128), (8, 4, 64), (16, 2, 64), (16, 2, 128)])
def test_combined_launch_matches_separate_launches(hk, g, d):
    """A plan with matrix-core and vector-ALU items (a shared prefix beside
    each sequence's own cells) runs both in one launch where the shape allows
    (one launch of both bodies, the vector-ALU merge in rounds through one
    LDS slot per row slice); timing one kind of kernel runs them as two
    launches.  Both give bit-identical outputs -- the rounds repeat the
    one-round merge's arithmetic in its order -- over rows of 512, 1024 and
    2048 numbers, one to four query heads per KV head, head sizes 64 and
    128 (2048-number rows of 128-number heads take the two launches
    either way)."""
    wl = W.prefix_decode(n_seq=8, prefix=300, private=50, n_layer=2, kv_size=1024)
    wl.n_head_kv, wl.n_head, wl.head_dim = hk, hk * g, d
    print(f"[gpu] combined launch: {hk} KV heads x {d}, group {g}", flush=True)
    ctx = make_ctx(wl)
    dev = torch.device("cuda:0")
    from tests.helpers import batch_tensors
    layers = list(range(wl.n_layer))
    compared = 0
    for b, bt in enumerate(wl.batches):
        t = batch_tensors(wl, b, layers, bt.measured)
        st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0 and len(ubs) == 1
        ub = ubs[0]
        ctx.store(ub, 0, [torch.from_numpy(t[(l, W.KIND_K)]).to(dev) for l in layers],
                  [torch.from_numpy(t[(l, W.KIND_V)]).to(dev) for l in layers])
        if not bt.measured:
            continue
        stats = ctx.plan_stats()
        assert stats["n_items_mfma"] > 0 and stats["n_items_valu"] > 0, stats
        Q = [torch.from_numpy(t[(l, W.KIND_Q)]).to(dev) for l in layers]
        combined = [torch.full_like(q, float("nan")) for q in Q]
        ctx.attend(ub, 0, Q, combined)
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k0.record()
        k1.record()
        K.kvattn_time_next_attend(ctx.ctx, K.KVATTN_KERNEL_VALU, k0.cuda_event, k1.cuda_event)
        separate = [torch.full_like(q, float("nan")) for q in Q]
        ctx.attend(ub, 0, Q, separate)
        torch.cuda.synchronize()
        for a, c in zip(combined, separate):
            assert torch.isfinite(a).all() and torch.equal(a, c)
        compared += 1
    assert compared == 1
    ctx.close()


def test_kernel_timing_across_launches():
    """A call whose layers are cut into several launches (the allocation-free
    entry point holds 21 layers' partials of this plan per launch, so 28
    layers take two): the start event belongs to the timed kernel's first
    launch, the stop event to its last, the outputs stay bit-identical to
    kvattn_attend's."""
    wl = W.prefix_decode(n_seq=32, prefix=1024, private=128, n_layer=28, kv_size=8192)
    print("[gpu] kernel timing across launches", flush=True)
    layers = list(range(wl.n_layer))
    ctx = make_ctx(wl, attend_layers=len(layers))
    dev = torch.device("cuda:0")
    from tests.helpers import batch_tensors
    from ubatch_attention_paged_amd.harness import ubatch_rows
    HD = wl.n_head * wl.head_dim
    done = False
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
            ctx.attend(ub, 0, Q, ref)
            stats = ctx.plan_stats()
            assert stats["n_partial_rows"] * wl.n_layer > 2016 and stats["n_items_mfma"] > 0, stats
            for kind in (K.KVATTN_KERNEL_MFMA, K.KVATTN_KERNEL_VALU, K.KVATTN_KERNEL_MERGE):
                k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                k0.record()
                k1.record()
                K.kvattn_time_next_attend(ctx.ctx, kind, k0.cuda_event, k1.cuda_event)
                out = [torch.full_like(r, float("nan")) for r in ref]
                c0.record()
                ctx.attend_noalloc(ub, 0, Q, out)
                c1.record()
                torch.cuda.synchronize()
                assert all(torch.equal(a, c) for a, c in zip(ref, out))
                kt, ct = k0.elapsed_time(k1), c0.elapsed_time(c1)
                print(f"  kind {kind}: first launch start to last launch end {kt:.4f} ms, call {ct:.4f} ms", flush=True)
                assert 0 < kt <= ct
            done = True
    assert done
    ctx.close()


def test_needles_on_gpu():
    """A dominant key in a visible cell takes over head 0's output; the same
    key planted in a hidden cell (other sequence, future position, stale row
    past n_kv) changes nothing."""
    from ubatch_attention_paged_amd.harness import decode
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(11)
    H, Hk, D = 16, 8, 128
    E = Hk * D

    def run(where):
        ctx = K.Context(1, H, Hk, D, kv_size=1024, n_seq_max=2, device="cuda:0")
        q = np.random.default_rng(11).standard_normal((1, H * D)).astype(np.float32)
        qhat = q[0, :D] / np.linalg.norm(q[0, :D])
        k0 = (np.random.default_rng(1).standard_normal((300, E)) * 0.1).astype(np.float32)
        v0 = np.random.default_rng(2).standard_normal((300, E)).astype(np.float32)
        k1 = (np.random.default_rng(3).standard_normal((40, E)) * 0.1).astype(np.float32)
        v1 = np.random.default_rng(4).standard_normal((40, E)).astype(np.float32)
        needle = np.full(D, 7.0, np.float32)
        if where == "visible":
            k0[77, :D], v0[77, :D] = 50 * qhat, needle
        elif where == "future":
            k0[250, :D], v0[250, :D] = 50 * qhat, needle
        elif where == "other_seq":
            k1[13, :D], v1[13, :D] = 50 * qhat, needle
        T = lambda a: [torch.from_numpy(np.ascontiguousarray(a)).to(dev)]
        decode(ctx, 300, np.arange(300), [[0]] * 300, None, T(k0), T(v0))
        decode(ctx, 40, np.arange(40), [[1]] * 40, None, T(k1), T(v1))
        if where == "beyond_nkv":
            ctx.K[0][0, 900, :D] = torch.from_numpy(50 * qhat).half().to(dev)
            ctx.V[0][0, 900, :D] = torch.from_numpy(needle).half().to(dev)
        kq = (np.random.default_rng(5).standard_normal((1, E)) * 0.1).astype(np.float32)
        vq = np.random.default_rng(6).standard_normal((1, E)).astype(np.float32)
        st, ubs, outs = decode(ctx, 1, [200], [[0]], None, T(kq), T(vq), Q=T(q))
        torch.cuda.synchronize()
        o = outs[0].cpu().numpy()
        ctx.close()
        return o

    base = run("none")
    hit = run("visible")
    np.testing.assert_allclose(hit[0, :D], 7.0, rtol=2e-3)
    for where in ("future", "other_seq", "beyond_nkv"):
        np.testing.assert_array_equal(run(where), base)


def test_cache_full_and_empty_batch_on_gpu():
    ctx = K.Context(1, 16, 8, 128, kv_size=16, device="cuda:0")
    st, ubs, _ = ctx.split(0)
    assert st == 0 and ubs == []
    st, ubs, _ = ctx.split(16)
    z = torch.zeros((16, 1024), device="cuda:0")
    ctx.store(ubs[0], 0, [z], [z])
    st, ubs, _ = ctx.split(1)
    assert st == K.KVATTN_NO_SLOT
    ctx.close()


@pytest.mark.parametrize("needle_pos", [40, 100, 180])
def test_mfma_running_max_jumps(needle_pos):
    """A prompt whose keys are small except one large key at a cell in the
    second 32-cell block of a tile: for the queries aligned with it, that
    block's maximum exceeds the running maximum by far more than the lazy
    rescale slack, after the first block of the same tile was already
    weighted.  Against the oracle on the same inputs (matrix-core path)."""
    from oracle import OracleEngine
    from ubatch_attention_paged_amd.harness import decode
    dev = torch.device("cuda:0")
    H, Hk, D, T = 16, 8, 128, 200
    E = Hk * D
    rng = np.random.default_rng(21)
    q = rng.standard_normal((T, H * D)).astype(np.float32)
    k = (rng.standard_normal((T, E)) * 0.1).astype(np.float32)
    v = rng.standard_normal((T, E)).astype(np.float32)
    u = rng.standard_normal(E).astype(np.float32)
    # each head's slice of the needle has norm ~80: its score is ~N(0, 10^2) in
    # log2 units, so for a good share of queries it jumps past every earlier
    # score by more than 2^8 (the F16 rounding of q moves such a score by
    # ~0.005, well inside the tolerance)
    k[needle_pos] = 226.0 * u / np.linalg.norm(u)
    pos = np.arange(T, dtype=np.int32)
    seqs = [[0]] * T
    ctx = K.Context(1, H, Hk, D, kv_size=512, n_seq_max=1, device="cuda:0")
    Tt = lambda a: [torch.from_numpy(np.ascontiguousarray(a)).to(dev)]
    st, ubs, outs = decode(ctx, T, pos, seqs, None, Tt(k), Tt(v), Q=Tt(q))
    assert st == 0 and len(ubs) == 1
    got = outs[0].cpu().numpy().astype(np.float64)
    ctx.close()
    eng = OracleEngine(1, H, Hk, D, 512, 1, 1, 2048, 2048, True, layers=[0])
    _, oubs, _ = eng.split(T, pos, [tuple(s) for s in seqs], None)
    ref, alt, sig = (np.zeros((T, H * D)) for _ in range(3))
    for ub in oubs:
        eng.commit(ub)
        eng.store(ub, 0, k[ub.src], v[ub.src])
        ref[ub.src] = eng.attend(ub, 0, q[ub.src])
        alt[ub.src], sig[ub.src] = model_for(eng, ub, 0, q[ub.src])
    # the needle's scores are ~30x those of N(0,1) keys, and rounding the
    # scaled q to F16 moves them by up to ~0.01 (log2 units): outputs near the
    # needle's value (|r| ~ 1) move by up to ~2.5e-3, inside the elementwise
    # tolerance 2e-3 + 5e-3 |r| but not always below 2e-3 in absolute terms;
    # the rounding model takes that query rounding into account exactly
    assert_parity(got, ref, tag=f"needle at {needle_pos}", strict_abs=False, alt=alt, sigma=sig)


@pytest.mark.parametrize("needle_pos", [3, 150, 199])
def test_decode_running_max_jumps(needle_pos):
    """The same kind of large key, read by single-token decode queries (the
    fp32 vector-ALU split-K path) against the oracle."""
    from oracle import OracleEngine
    from ubatch_attention_paged_amd.harness import decode
    dev = torch.device("cuda:0")
    H, Hk, D, T, S = 16, 8, 128, 200, 6
    E = Hk * D
    rng = np.random.default_rng(22)
    k = (rng.standard_normal((T + S, E)) * 0.1).astype(np.float32)
    v = rng.standard_normal((T + S, E)).astype(np.float32)
    q = rng.standard_normal((S, H * D)).astype(np.float32)
    u = rng.standard_normal(E).astype(np.float32)
    k[needle_pos] = 226.0 * u / np.linalg.norm(u)
    ctx = K.Context(1, H, Hk, D, kv_size=512, n_seq_max=1, device="cuda:0")
    eng = OracleEngine(1, H, Hk, D, 512, 1, 1, 2048, 2048, True, layers=[0])
    Tt = lambda a: [torch.from_numpy(np.ascontiguousarray(a)).to(dev)]
    decode(ctx, T, np.arange(T), [[0]] * T, None, Tt(k[:T]), Tt(v[:T]))
    _, oubs, _ = eng.split(T, np.arange(T, dtype=np.int32), [(0,)] * T, None)
    for ub in oubs:
        eng.commit(ub, build_mask=False)
        eng.store(ub, 0, k[:T][ub.src], v[:T][ub.src])
    for s in range(S):
        p = T + s
        st, ubs, outs = decode(ctx, 1, [p], [[0]], None, Tt(k[p:p + 1]), Tt(v[p:p + 1]), Q=Tt(q[s:s + 1]))
        got = outs[0].cpu().numpy().astype(np.float64)
        _, oubs, _ = eng.split(1, np.array([p], np.int32), [(0,)], None)
        eng.commit(oubs[0])
        eng.store(oubs[0], 0, k[p:p + 1], v[p:p + 1])
        ref = eng.attend(oubs[0], 0, q[s:s + 1])
        assert_parity(got, ref, tag=f"decode step {s}, needle at {needle_pos}")
    ctx.close()


@pytest.mark.parametrize("name", ["prefill", "cb_decode", "mixed", "prefix"])
def test_noncausal_parity(name):
    """causal = 0: cells at later positions (already stored) are visible too,
    in both attention kernels and the split-K merge."""
    import dataclasses
    wl = dataclasses.replace(small(name), causal=False)
    layers = list(range(wl.n_layer))
    print(f"[gpu] non-causal {name}", flush=True)
    _, ref, _, _ = oracle_run(wl, layers)
    _, got = gpu_run(wl, layers)
    worst = 0.0
    for key in ref:
        ma, _ = assert_parity(got[key], ref[key], tag=f"non-causal {name} {key}", **ref.model(key))
        worst = max(worst, ma)
    print(f"[gpu] non-causal {name}: max abs error {worst:.3e}", flush=True)
    if name == "cb_decode":
        assert worst < VALU_BOUND, worst


@pytest.mark.parametrize("name,mode", [("mixed", "seq"), ("prefix", "seq"), ("prefill", "seq"), ("mixed", "simple")])
def test_split_mode_parity(name, mode):
    """Explicitly requested split strategies end to end: split_seq keeps every
    ubatch to one sequence set; split_simple over several streams mixes
    streams inside a ubatch."""
    import dataclasses
    wl = dataclasses.replace(small(name), split_mode=mode)
    layers = list(range(wl.n_layer))
    print(f"[gpu] split mode {mode} on {name}", flush=True)
    eng, ref, masks, meta = oracle_run(wl, layers, keep_masks=True)
    ub_index = {b: 0 for b in range(len(wl.batches))}

    def check(ctx, b, ub):
        r = meta[(b, ub_index[b])]
        assert ub.cells.tolist() == r.cells
        if mode == "seq":
            assert ub.n_seqs == 1 and len(set(ub.seq_ids)) == 1
        m = ctx.mask(ub).cpu().numpy().view(np.uint16)
        assert np.array_equal(m, masks[(b, ub_index[b])].view(np.uint16))
        ub_index[b] += 1

    _, got = gpu_run(wl, layers, on_ubatch=check)
    for key in ref:
        assert_parity(got[key], ref[key], tag=f"{mode} {name} {key}", **ref.model(key))


def test_prefix_separate_copies_across_streams():
    """A prefix shared by 8 sequences in a 4-stream cache is stored once per
    stream (separate copies written by the store kernel); every sequence's
    decode token attends like the oracle's and like the same workload over
    one unified stream."""
    wl4 = W.prefix_decode(n_seq=8, prefix=200, private=30, n_layer=2, kv_size=512, n_stream=4)
    wl1 = W.prefix_decode(n_seq=8, prefix=200, private=30, n_layer=2, kv_size=2048, n_stream=1)
    layers = [0, 1]
    _, ref, _, _ = oracle_run(wl4, layers)
    ctx4, got4 = gpu_run(wl4, layers)
    ctx1, got1 = gpu_run(wl1, layers)
    for key in ref:
        assert_parity(got4[key], ref[key], tag=f"4 streams {key}", **ref.model(key))
        assert_parity(got4[key], got1[key], tag=f"4 streams vs unified {key}")
    for s in range(4):
        pos, mask = ctx4.cells(s)
        assert int((pos >= 0).sum()) == 200 + 2 * 31       # the prefix copy, 2 sequences x (30 + 1)


@pytest.mark.parametrize("name,w", [("tiny", 3), ("prefill", 100), ("prefill", 300), ("cb_decode", 50),
                                    ("mixed", 64), ("prefix", 200), ("prefix", 1)])
def test_sliding_window_parity(name, w):
    """A sliding window of w positions (reading of the elided window rule: a
    cell is hidden when the query's position minus its position is >= w) in
    the dense diagnostic mask (bit for bit), the matrix-core kernel (masked
    and skipped tiles) and the vector-ALU kernel."""
    import dataclasses
    wl = dataclasses.replace(small(name), swa=w)
    layers = list(range(wl.n_layer))
    print(f"[gpu] sliding window {w} on {name}", flush=True)
    eng, ref, masks, meta = oracle_run(wl, layers, keep_masks=True)
    ub_index = {b: 0 for b in range(len(wl.batches))}

    def check(ctx, b, ub):
        m = ctx.mask(ub).cpu().numpy().view(np.uint16)
        assert np.array_equal(m, masks[(b, ub_index[b])].view(np.uint16))
        ub_index[b] += 1

    _, got = gpu_run(wl, layers, on_ubatch=check)
    for key in ref:
        assert_parity(got[key], ref[key], tag=f"window {w} {name} {key}", **ref.model(key))


@pytest.mark.parametrize("n_shared", [0, 1200])
def test_many_sequences(n_shared):
    """256 live sequences, the widest sequence set: two decode ubatches of 256
    queries over group prefixes (cells holding 8 ids), private prompts and,
    with n_shared, 1200 cells holding 8 random ids each, so one ubatch sees
    288 or ~1500 distinct sets, read by ~40 queries each in the second case.
    Past 1024 classes the tail of the class list is merged
    into one class of the union set, walked with the per-cell membership
    test; when the queries then still need more split-K partial rows than
    the workspace holds (each query gets one per class it reads), the
    planner halves the class cap until they fit.  Cells and dense masks bit
    for bit, the class lists too while nothing is merged, every output
    within tolerance."""
    wl = W.many_sequences(n_shared=n_shared)
    print(f"[gpu] many_sequences: {wl.note}", flush=True)
    eng, ref, masks, meta = oracle_run(wl, [0], keep_masks=True)
    ub_index = {b: 0 for b in range(len(wl.batches))}
    plan_classes = []

    def check(ctx, b, ub):
        u = ub_index[b]
        assert ub.cells.tolist() == meta[(b, u)].cells
        if wl.batches[b].measured:
            m = ctx.mask(ub).cpu().numpy().view(np.uint16)
            assert np.array_equal(m, masks[(b, u)].view(np.uint16)), f"mask differs (batch {b}, ubatch {u})"
            st = ctx.plan_stats()
            plan_classes.append((st["n_classes"], st["n_partial_rows"]))
        ub_index[b] += 1

    ctx, got = gpu_run(wl, [0], on_ubatch=check)
    last = max(meta)
    exp = expected_classes(eng, meta[last])
    n_classes = ctx.plan_stats()["n_classes"]
    if len(exp) <= 1024:
        got_cls = ctx.classes()
        assert n_classes == len(exp) == len(got_cls)
        assert [(s, m) for s, m, _ in got_cls] == [(s, m) for s, m, _ in exp]
        for (_, _, cg), (_, _, ce) in zip(got_cls, exp):
            assert np.array_equal(cg, ce)
    else:
        # 1023 sets of ~8 queries each would need ~8000 partial rows: the cap shrinks
        assert max(c for c, _ in plan_classes) < 1024, plan_classes
    worst = 0.0
    for key in ref:
        ma, _ = assert_parity(got[key], ref[key], tag=f"many_sequences n_shared={n_shared} batch {key[0]}", **ref.model(key))
        worst = max(worst, ma)
    print(f"[gpu] many_sequences n_shared={n_shared}: {len(exp)} sets, (classes, partial rows) per decode ubatch "
          f"{plan_classes}, max abs error {worst:.3e}", flush=True)
    ctx.close()
