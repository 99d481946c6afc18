"""Pins for the oracle's iteration-level batching loop (oracle/scheduler.py).

* hand-worked traces of the loop ("Iteration-Level Batching", "The loop that
  replaces the batch", "The budget that actually binds", "Where it breaks")
  in tests/golden/sched_traces.txt: block reservation, chunked prefill,
  preemption of a prefilling and of a decoding sequence with recomputation,
  first-come-first-served blocking, sequence-id reuse, two streams;
* a closed form: with room for everything, iteration 0 runs every prompt and
  iteration k one token of each sequence that still generates;
* invariants on seeded request streams, with the oracle engine's cell table
  following every retirement and preemption: the budget is never exceeded,
  each request emits exactly n_generate output flags at the right positions,
  the cache never holds more than it has and the cells of each running
  sequence are exactly its cached positions.
"""

import os

import numpy as np
import pytest

from oracle import OracleEngine, seqstate
from oracle.scheduler import OracleScheduler, SchedError, blob_bytes
from synthetic.serving import request_stream

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sched_traces.txt")


def parse_traces():
    cases, cur = {}, None
    for ln in open(GOLDEN):
        ln = ln.strip()
        if not ln or ln.startswith("#"):
            continue
        head, *rest = ln.split(None, 1)
        if head == "case":
            name, *kv = rest[0].split()
            p = dict(x.split("=") for x in kv)
            cur = cases[name] = {"params": p, "reqs": [], "its": []}
        elif head == "req":
            cur["reqs"].append(tuple(int(x) for x in rest[0].split()))
        elif head == "it":
            k, ret, pre, adm, bat = [f.strip() for f in rest[0].split("|")]
            ids = lambda f: [] if f == "-" else [int(x) for x in f.split()]
            admitted = [] if adm == "-" else [tuple(int(y) for y in x.split(":")) for x in adm.split()]
            req, seq, pos, out = [], [], [], []
            if bat != "-":
                for run in bat.split():
                    rs, span = run.split("@")
                    r, s = (int(y) for y in rs.split(":"))
                    star = span.endswith("*")
                    span = span.rstrip("*")
                    a, b = (int(y) for y in span.split("-")) if "-" in span else (int(span), int(span))
                    for p_ in range(a, b + 1):
                        req.append(r)
                        seq.append(s)
                        pos.append(p_)
                        out.append(1 if (star and p_ == b) else 0)
            cur["its"].append(dict(k=int(k), retired=ids(ret), preempted=ids(pre), admitted=admitted,
                                   req=req, seq=seq, pos=pos, output=out))
    return cases


CASES = parse_traces()


def sched_from(p, release=None):
    return OracleScheduler(int(p["kv_size"]), int(p["n_stream"]), int(p["n_seq_max"]), int(p["budget"]),
                           max_running=int(p["max_running"]), policy=p["policy"],
                           block_size=int(p["block_size"]), chunked=p["chunked"] == "1", release=release,
                           preempt=p.get("preempt", "recompute"), swap_bytes=int(p.get("swap_bytes", 0)),
                           n_layer=int(p.get("n_layer", 1)), row_bytes=int(p.get("row_bytes", 0)))


@pytest.mark.parametrize("name", sorted(CASES))
def test_hand_worked_trace(name):
    case = CASES[name]
    s = sched_from(case["params"])
    for pr, g in case["reqs"]:
        s.submit(pr, g)
    for exp in case["its"]:
        got = s.step()
        for key in ("retired", "preempted", "admitted", "req", "seq", "pos", "output"):
            assert list(got[key]) == exp[key], (name, exp["k"], key, got[key], exp[key])
        s.advance()
    assert s.idle()


def test_golden_file_covers_every_mechanism():
    its = [it for c in CASES.values() for it in c["its"]]
    assert any(it["preempted"] for it in its)
    assert {c["params"].get("preempt", "recompute") for c in CASES.values()} == {"recompute", "swap"}
    assert {c["params"]["policy"] for c in CASES.values()} == {"paged", "reserve"}
    assert {c["params"]["chunked"] for c in CASES.values()} == {"0", "1"}
    assert any(int(c["params"]["n_stream"]) > 1 for c in CASES.values())


def test_closed_form_when_everything_fits():
    P, G = [7, 3, 12, 1, 5], [4, 1, 6, 2, 3]
    s = OracleScheduler(kv_size=256, n_stream=1, n_seq_max=8, token_budget=64)
    for p, g in zip(P, G):
        s.submit(p, g)
    it = s.step()
    assert it["admitted"] == [(i, i) for i in range(5)]
    assert it["req"] == [i for i, p in enumerate(P) for _ in range(p)]
    assert it["pos"] == [q for p in P for q in range(p)]
    assert sum(it["output"]) == 5
    s.advance()
    k = 1
    while not s.idle():
        it = s.step()
        assert it["retired"] == [i for i, g in enumerate(G) if g == k]
        live = [i for i, g in enumerate(G) if g > k]
        assert it["req"] == live and it["pos"] == [P[i] + k - 1 for i in live]
        assert it["output"] == [1] * len(live)
        s.advance()
        k += 1
    assert k == max(G) + 1


def test_swap_records_and_arena():
    case = CASES["paged_swap_decoder"]
    s = sched_from(case["params"])
    for pr, g in case["reqs"]:
        s.submit(pr, g)
    outs, ins = {}, {}
    for exp in case["its"]:
        rec = s.step()
        outs[exp["k"]], ins[exp["k"]] = rec["swapped_out"], rec["swapped_in"]
        if exp["k"] == 3:
            assert s.swapped == [(0, 768, 1)] and s.requests[1].n_ctx == 4
        s.advance()
    assert outs[3] == [1] and ins[5] == [1] and s.swapped == []
    assert all(not v for k, v in outs.items() if k != 3) and all(not v for k, v in ins.items() if k != 5)
    fb = sched_from(CASES["paged_swap_fallback"]["params"])
    assert fb._swap_place(768) is None and fb._swap_place(512) == 0


def test_swap_arena_first_fit():
    s = OracleScheduler(kv_size=64, n_stream=1, n_seq_max=4, token_budget=8, preempt="swap", swap_bytes=4096)
    s.swapped = [(0, 512, 0), (1024, 256, 1), (2048, 1024, 2)]
    assert s._swap_place(512) == 512          # the first gap that fits
    assert s._swap_place(768) == 1280
    assert s._swap_place(1024) == 3072        # the tail
    assert s._swap_place(1025) is None


def test_submission_rejections():
    s = OracleScheduler(kv_size=16, n_stream=1, n_seq_max=4, token_budget=8, chunked=False)
    with pytest.raises(SchedError):
        s.submit(9, 1)              # prompt over the budget without chunking
    with pytest.raises(SchedError):
        s.submit(4, 6)              # a paged recomputation of 9 positions could not re-enter
    with pytest.raises(SchedError):
        s.submit(0, 1)
    s2 = OracleScheduler(kv_size=16, n_stream=1, n_seq_max=4, token_budget=8)
    with pytest.raises(SchedError):
        s2.submit(10, 8)            # 17 positions never fit 16 cells
    s2.submit(10, 7)
    s3 = OracleScheduler(kv_size=16, n_stream=1, n_seq_max=4, token_budget=8, policy="reserve", block_size=8)
    with pytest.raises(SchedError):
        s3.submit(10, 7)            # ceil(17 / 8) = 3 blocks > 2
    with pytest.raises(SchedError):
        OracleScheduler(kv_size=16, n_stream=1, n_seq_max=4, token_budget=3)   # budget < max_running


def drive(stream, with_engine=True, max_iters=10000):
    """Run the loop over a request stream; returns the iteration records and
    checks the invariants after every iteration."""
    eng, hooks = None, {}
    if with_engine:
        swap = stream.preempt == "swap"
        eng = OracleEngine(stream.n_layer, stream.n_head, stream.n_head_kv, stream.head_dim, stream.kv_size,
                           stream.n_stream, stream.n_seq_max, stream.token_budget, stream.n_ubatch,
                           layers=None if swap else [], split_mode=stream.split_mode)
        if swap:
            hooks = dict(swap_out=lambda q: seqstate.save(eng, q), swap_in=lambda q, b: seqstate.load(eng, q, b))
    s = OracleScheduler(release=(lambda q: eng.seq_rm(q)) if eng else None, **stream.sched_kwargs(), **hooks)
    outputs = {r: [] for r in range(stream.n_requests)}
    recs, it = [], 0
    while it < max_iters:
        for r in stream.arrivals(it):
            assert s.submit(int(stream.n_prompt[r]), int(stream.n_generate[r])) == r
        rec = s.step()
        n = len(rec["pos"])
        assert n <= stream.token_budget
        if eng is not None and n:
            st, ubs, _ = eng.split(n, rec["pos"], [(q,) for q in rec["seq"]], rec["output"])
            assert st == 0
            for ub in ubs:
                eng.commit(ub, build_mask=False)
        for r, p, o in zip(rec["req"], rec["pos"], rec["output"]):
            if o:
                outputs[r].append(p)
        s.advance()
        recs.append(rec)
        if eng is not None:
            for st_ in range(stream.n_stream):
                pos, member = eng.cells.pos[st_], eng.cells.member[st_]
                used = int((pos >= 0).sum())
                assert used <= stream.kv_size
                held = 0
                for r in s.running:
                    if s.stream_of(r.seq) != st_:
                        continue
                    mine = sorted(int(q) for q in pos[member[:, r.seq] & (pos >= 0)])
                    assert mine == list(range(r.n_ctx)), (it, r.id)
                    held += r.n_ctx
                assert held == used
        it += 1
        if s.idle() and it > int(stream.arrive[-1]):
            break
    assert s.idle()
    for r in range(stream.n_requests):
        P, G = int(stream.n_prompt[r]), int(stream.n_generate[r])
        assert outputs[r][-G:] == list(range(P - 1, P + G - 1)), r
        assert len(outputs[r]) == G, r     # recomputation never re-samples
    return recs


STREAMS = {
    "paged_roomy": dict(kv_size=1024),
    "paged_tight": dict(kv_size=96, rate=1.5),
    "paged_tight_streams": dict(kv_size=64, n_stream=4, rate=2.0),
    "paged_unchunked": dict(kv_size=128, chunked=False, token_budget=64),
    "reserve_blocks": dict(kv_size=128, policy="reserve", block_size=16),
    "reserve_streams": dict(kv_size=96, n_stream=2, policy="reserve", block_size=8, rate=2.0),
    "swap_tight": dict(kv_size=96, rate=1.5, preempt="swap", swap_bytes=1 << 20),
    "swap_small_arena": dict(kv_size=64, n_stream=4, rate=2.0, preempt="swap", swap_bytes=32768),
}


@pytest.mark.parametrize("name", sorted(STREAMS))
def test_invariants_on_request_streams(name):
    st = request_stream(seed=2100 + sorted(STREAMS).index(name), **STREAMS[name])
    recs = drive(st)
    n_pre = sum(len(r["preempted"]) for r in recs)
    if st.policy == "reserve":
        assert n_pre == 0
    if name in ("paged_tight", "paged_tight_streams", "swap_tight", "swap_small_arena"):
        assert n_pre > 0           # the case exists to exercise preemption
    n_swap = sum(len(r["swapped_out"]) for r in recs)
    if name.startswith("swap"):
        assert n_swap > 0 and n_swap == sum(len(r["swapped_in"]) for r in recs)
    if name == "swap_small_arena":
        assert n_swap < n_pre      # some victims did not fit the arena and were recomputed
    # every running sequence with one pending position is served each iteration
    assert all(len(r["pos"]) > 0 or r["n_running"] == 0 for r in recs)
