"""The native iteration-level batching loop (include/kvsched.h) on the CPU.

Host-only contexts: every batch the loop assembles is split and committed
(store with no layers), so retirement and preemption act on a real cell
table.  Checked bit for bit against the oracle's loop (oracle/scheduler.py),
which is pinned by hand-worked traces in test_oracle_scheduler.py:

* the hand-worked traces themselves;
* seeded request streams under both admission policies, with and without
  chunking, one and several streams, roomy and exhausted caches: every
  iteration's retired / preempted / admitted lists and batch, and the
  context's cell table against the oracle engine's after every iteration;
* parameter and state errors.
"""

import numpy as np
import pytest

from oracle import OracleEngine, seqstate
from oracle.scheduler import OracleScheduler, SchedError
from synthetic.serving import request_stream

from test_oracle_scheduler import CASES, STREAMS

K = pytest.importorskip("ubatch_attention_paged_amd")

KEYS = ("retired", "preempted", "admitted", "swapped_out", "swapped_in", "req", "seq", "pos", "output",
        "n_running", "n_waiting")


def host_ctx(kv_size, n_stream, n_seq_max, n_batch, n_ubatch=0, split_mode="auto"):
    return K.Context(1, 2, 1, 16, kv_size=kv_size, n_stream=n_stream, n_seq_max=n_seq_max,
                     n_batch=n_batch, n_ubatch=n_ubatch or n_batch, split_mode=split_mode)


def run_batch(ctx, sch):
    it = sch.it
    if it.batch.n_tokens == 0:
        return []
    st, ubs, _ = ctx.split_batch(it.batch)
    assert st == 0
    for u in ubs:
        ctx.store(u, 0, [], [])
    return ubs


@pytest.mark.parametrize("name", sorted(CASES))
def test_native_hand_worked_trace(name):
    case = CASES[name]
    p = case["params"]
    budget = int(p["budget"])
    # the swap cases size their blobs for 1 layer of 64-byte rows: 1 KV head of 32
    ctx = K.Context(int(p.get("n_layer", 1)), 2, 1, int(p.get("row_bytes", 32)) // 2, kv_size=int(p["kv_size"]),
                    n_stream=int(p["n_stream"]), n_seq_max=int(p["n_seq_max"]), n_batch=budget, n_ubatch=budget)
    sch = K.Scheduler(ctx, token_budget=budget, max_running=int(p["max_running"]), policy=p["policy"],
                      block_size=int(p["block_size"]), chunked=p["chunked"] == "1", max_requests=16,
                      preempt=p.get("preempt", "recompute"), swap_bytes=int(p.get("swap_bytes", 0)))
    for pr, g in case["reqs"]:
        sch.submit(pr, g)
    for exp in case["its"]:
        sch.step()
        got = sch.record()
        for key in ("retired", "preempted", "admitted", "req", "seq", "pos", "output"):
            assert list(got[key]) == exp[key], (name, exp["k"], key)
        run_batch(ctx, sch)
        sch.advance()
    assert sch.record()["n_running"] == 0 and sch.record()["n_waiting"] == 0


def compare_tables(ctx, eng, n_stream):
    for s in range(n_stream):
        pos, mask = ctx.cells(s)
        rpos = eng.cells.pos[s]
        nq = eng.cells.member.shape[2]
        member = K.seqset_members(mask, K.MAX_SEQ)
        assert np.array_equal(pos, rpos)
        assert np.array_equal(member[:, :nq], eng.cells.member[s])
        assert not member[:, nq:].any()


def drive_both(stream, max_iters=5000, stats=None):
    n_batch = stream.token_budget
    ctx = host_ctx(stream.kv_size, stream.n_stream, stream.n_seq_max, n_batch, stream.n_ubatch, stream.split_mode)
    eng = OracleEngine(1, 2, 1, 16, stream.kv_size, stream.n_stream, stream.n_seq_max, n_batch, stream.n_ubatch,
                       layers=[], split_mode=stream.split_mode)
    hooks = {}
    if stream.preempt == "swap":
        eng = OracleEngine(1, 2, 1, 16, stream.kv_size, stream.n_stream, stream.n_seq_max, n_batch, stream.n_ubatch,
                           split_mode=stream.split_mode)
        hooks = dict(swap_out=lambda q: seqstate.save(eng, q), swap_in=lambda q, b: seqstate.load(eng, q, b))
    kw = stream.sched_kwargs()
    kw.update(n_layer=1, row_bytes=32)          # the host contexts here: 1 layer, 1 KV head of 16
    ref = OracleScheduler(release=lambda q: eng.seq_rm(q), **kw, **hooks)
    sch = K.Scheduler(ctx, token_budget=stream.token_budget, max_running=stream.max_running,
                      policy=stream.policy, block_size=stream.block_size, chunked=stream.chunked,
                      max_requests=stream.n_requests, preempt=stream.preempt, swap_bytes=stream.swap_bytes)
    n_pre, it = 0, 0
    while it < max_iters:
        for r in stream.arrivals(it):
            a = sch.submit(int(stream.n_prompt[r]), int(stream.n_generate[r]))
            b = ref.submit(int(stream.n_prompt[r]), int(stream.n_generate[r]))
            assert a == b == r
        sch.step()
        got, exp = sch.record(), ref.step()
        for key in KEYS:
            assert got[key] == exp[key], (it, key, got[key], exp[key])
        n_pre += len(exp["preempted"])
        if stats is not None:
            stats["max_running"] = max(stats.get("max_running", 0), exp["n_running"])
        ubs = run_batch(ctx, sch)
        if exp["pos"]:
            st, rubs, _ = eng.split(len(exp["pos"]), exp["pos"], [(q,) for q in exp["seq"]], exp["output"])
            assert st == 0 and len(rubs) == len(ubs)
            for u, ru in zip(ubs, rubs):
                assert u.cells.tolist() == list(ru.cells)
                eng.commit(ru, build_mask=False)
        sch.advance()
        ref.advance()
        compare_tables(ctx, eng, stream.n_stream)
        it += 1
        if ref.idle() and it > int(stream.arrive[-1]):
            break
    assert ref.idle()
    for r in range(stream.n_requests):
        q = sch.request(r)
        assert q["state"] == K.KVATTN_REQ_DONE and q["n_sampled"] == int(stream.n_generate[r])
    return it, n_pre


NATIVE_STREAMS = dict(STREAMS)
NATIVE_STREAMS.update({
    "paged_split_equal": dict(kv_size=64, n_stream=4, rate=2.0, split_mode="equal", n_ubatch=16),
    "paged_split_seq": dict(kv_size=96, rate=1.5, split_mode="seq", n_ubatch=24),
    "paged_wide": dict(n_req=60, kv_size=512, n_seq_max=32, token_budget=128, rate=3.0, burst=20,
                       prompt_range=(1, 90), gen_range=(1, 30)),
    "reserve_unchunked": dict(kv_size=160, policy="reserve", block_size=4, chunked=False, rate=1.5),
    "paged_max_running": dict(kv_size=256, n_seq_max=8, max_running=3, rate=2.0),
})


@pytest.mark.parametrize("name", sorted(NATIVE_STREAMS))
def test_native_loop_matches_oracle(name):
    st = request_stream(seed=2300 + sorted(NATIVE_STREAMS).index(name), **NATIVE_STREAMS[name])
    iters, n_pre = drive_both(st)
    assert iters > 10
    if name.startswith("paged_tight"):
        assert n_pre > 0


def test_native_loop_many_running():
    """More than 64 sequences running at once (sequence ids up to 255): the
    native loop against the oracle loop, every iteration's records, every
    ubatch's cells and the whole cell table bit for bit."""
    st = request_stream(n_req=300, rate=8.0, burst=200, prompt_range=(1, 16), gen_range=(1, 40), kv_size=4096,
                        n_seq_max=256, token_budget=512, n_ubatch=128, seed=2400)
    stats = {}
    iters, _ = drive_both(st, stats=stats)
    assert iters > 10 and stats["max_running"] > 200, stats


def test_native_errors():
    ctx = host_ctx(16, 1, 4, 8)
    with pytest.raises(K.KvattnError):
        K.Scheduler(ctx, token_budget=3)                       # below max_running (4)
    with pytest.raises(K.KvattnError):
        K.Scheduler(ctx, token_budget=9)                       # above the context's n_batch
    with pytest.raises(K.KvattnError):
        K.Scheduler(ctx, max_running=5)
    with pytest.raises(K.KvattnError):
        K.Scheduler(ctx, policy=7)
    with pytest.raises(K.KvattnError):
        K.Scheduler(ctx, policy="reserve", block_size=0)
    sch = K.Scheduler(ctx, chunked=False, max_requests=2)
    assert K.kvattn_get_params(ctx.ctx).n_batch == 8
    for bad in ((9, 1), (4, 6), (0, 1), (1, 0)):
        with pytest.raises(K.KvattnError) as e:
            sch.submit(*bad)
        assert e.value.code == K.KVATTN_EINVAL
        with pytest.raises(SchedError):
            OracleScheduler(16, 1, 4, 8, chunked=False).submit(*bad)
    sch.submit(3, 2)
    sch.submit(2, 2)
    with pytest.raises(K.KvattnError) as e:
        sch.submit(1, 1)
    assert e.value.code == K.KVATTN_ENOMEM
    with pytest.raises(K.KvattnError) as e:
        sch.advance()
    assert e.value.code == K.KVATTN_ESTATE
    sch.step()
    with pytest.raises(K.KvattnError) as e:
        sch.step()
    assert e.value.code == K.KVATTN_ESTATE
    with pytest.raises(K.KvattnError):
        sch.request(2)
    assert sch.request(0)["state"] == K.KVATTN_REQ_RUNNING


def test_get_params_reports_clamps():
    ctx = K.Context(2, 4, 2, 32, kv_size=100, n_stream=2, n_seq_max=6, n_batch=4096, n_ubatch=0,
                    split_mode="auto")
    p = K.kvattn_get_params(ctx.ctx)
    assert (p.n_batch, p.n_ubatch) == (200, 200)
    assert p.split_mode == K.kvattn.KVATTN_SPLIT_EQUAL
    assert abs(p.kq_scale - 32 ** -0.5) < 1e-7
    assert (p.n_layer, p.n_head, p.n_head_kv, p.head_dim, p.kv_size, p.n_stream, p.n_seq_max) == \
        (2, 4, 2, 32, 100, 2, 6)
    assert not p.k_layers and not p.workspace
