"""The iteration-level batching loop end to end on the GPU.

The native loop (include/kvsched.h) drives a GPU context: every iteration's
batch is split, each ubatch stores its K/V rows and runs attention for all
of its slots (a forward pass needs every position's attention, not only the
flagged ones).  In lockstep the oracle loop drives the oracle engine on the
same rows.  Checked per iteration: the two loops' records bit for bit, the
cells of every ubatch, and every attention output within |g - r| <= 2e-3 +
5e-3 |r|.  Rows are keyed by (request, position), so a recomputation after
preemption writes what the first pass wrote.  Under preemption by swapping
the oracle loop saves and restores through the oracle's own sequence-state
functions.
"""

import numpy as np
import pytest
import torch

from oracle import OracleEngine, seqstate
from oracle.scheduler import OracleScheduler
from synthetic.serving import request_stream, QWEN3_06B
from synthetic.workloads import KIND_K, KIND_V, KIND_Q

from helpers import assert_parity, model_for

pytestmark = pytest.mark.gpu

KEYS = ("retired", "preempted", "admitted", "swapped_out", "swapped_in", "req", "seq", "pos", "output",
        "n_running", "n_waiting")


def serve_parity(stream, max_iters=400):
    import ubatch_attention_paged_amd as K
    from ubatch_attention_paged_amd.harness import ubatch_rows
    dev = torch.device("cuda:0")
    layers = list(range(stream.n_layer))
    nb = stream.token_budget
    ctx = K.Context(stream.n_layer, stream.n_head, stream.n_head_kv, stream.head_dim, stream.kv_size,
                    stream.n_stream, stream.n_seq_max, nb, stream.n_ubatch, device="cuda:0",
                    attend_layers=len(layers), split_mode=stream.split_mode)
    sch = K.Scheduler(ctx, token_budget=nb, max_running=stream.max_running, policy=stream.policy,
                      block_size=stream.block_size, chunked=stream.chunked, max_requests=stream.n_requests,
                      preempt=stream.preempt, swap_bytes=stream.swap_bytes)
    eng = OracleEngine(stream.n_layer, stream.n_head, stream.n_head_kv, stream.head_dim, stream.kv_size,
                       stream.n_stream, stream.n_seq_max, nb, stream.n_ubatch, layers=layers,
                       split_mode=stream.split_mode)
    hooks = {}
    if stream.preempt == "swap":
        hooks = dict(swap_out=lambda q: seqstate.save(eng, q), swap_in=lambda q, b: seqstate.load(eng, q, b))
    ref = OracleScheduler(release=lambda q: eng.seq_rm(q), **stream.sched_kwargs(), **hooks)
    HD = stream.n_head * stream.head_dim
    stats = dict(iters=0, rows=0, preempted=0, swapped=0, mfma_items=0, valu_items=0, max_abs=0.0)
    it = 0
    while it < max_iters:
        for r in stream.arrivals(it):
            assert sch.submit(int(stream.n_prompt[r]), int(stream.n_generate[r])) == \
                ref.submit(int(stream.n_prompt[r]), int(stream.n_generate[r]))
        sch.step()
        got, exp = sch.record(), ref.step()
        for key in KEYS:
            assert got[key] == exp[key], (it, key)
        stats["preempted"] += len(exp["preempted"])
        stats["swapped"] += len(exp["swapped_out"])
        n = len(exp["pos"])
        if n:
            rows = {(l, k): stream.batch_rows(exp["req"], exp["pos"], l, k)
                    for l in layers for k in (KIND_K, KIND_V, KIND_Q)}
            dK = [torch.from_numpy(rows[(l, KIND_K)]).to(dev) for l in layers]
            dV = [torch.from_numpy(rows[(l, KIND_V)]).to(dev) for l in layers]
            dQ = [torch.from_numpy(rows[(l, KIND_Q)]).to(dev) for l in layers]
            st, ubs, _ = ctx.split_batch(sch.it.batch)
            rst, rubs, _ = eng.split(n, exp["pos"], [(q,) for q in exp["seq"]], exp["output"])
            assert st == 0 and rst == 0 and len(ubs) == len(rubs)
            print(f"iteration {it}: {n} slots in {len(ubs)} ubatches", flush=True)
            for u, ru in zip(ubs, rubs):
                assert u.cells.tolist() == list(ru.cells) and u.src.tolist() == list(ru.src)
                outs = [torch.full((u.n_tokens, HD), float("nan"), device=dev) for _ in layers]
                ctx.store(u, 0, [ubatch_rows(u, t) for t in dK], [ubatch_rows(u, t) for t in dV])
                ctx.attend(u, 0, [ubatch_rows(u, t) for t in dQ], outs)
                ps = ctx.plan_stats()
                stats["mfma_items"] += ps["n_items_mfma"]
                stats["valu_items"] += ps["n_items_valu"]
                eng.commit(ru, build_mask=True)
                for i, l in enumerate(layers):
                    eng.store(ru, l, rows[(l, KIND_K)][ru.src], rows[(l, KIND_V)][ru.src])
                    qr = rows[(l, KIND_Q)][ru.src]
                    want = eng.attend(ru, l, qr)
                    alt, sig = model_for(eng, ru, l, qr)
                    have = outs[i].double().cpu().numpy()
                    e, _ = assert_parity(have, want, tag=f"it {it} ubatch {u.id} layer {l}", alt=alt, sigma=sig)
                    stats["max_abs"] = max(stats["max_abs"], e)
                stats["rows"] += u.n_tokens
        sch.advance()
        ref.advance()
        it += 1
        if ref.idle() and it > int(stream.arrive[-1]):
            break
    assert ref.idle()
    stats["iters"] = it
    torch.cuda.synchronize()
    return stats


def test_serving_small_heads_with_preemption():
    st = request_stream(n_req=24, rate=1.5, kv_size=96, token_budget=64, n_ubatch=32, seed=2501)
    s = serve_parity(st)
    print(s)
    assert s["preempted"] > 0 and s["rows"] > 300


def test_serving_qwen_heads_prefill_chunks_and_decode():
    st = request_stream(n_req=20, rate=0.7, burst=6, prompt_range=(40, 600), gen_range=(4, 24),
                        n_layer=2, kv_size=2048, n_seq_max=16, token_budget=512, n_ubatch=128,
                        seed=2502, **{k: QWEN3_06B[k] for k in ("n_head", "n_head_kv", "head_dim")})
    s = serve_parity(st)
    print(s)
    assert s["mfma_items"] > 0 and s["valu_items"] > 0


def test_serving_streams_split_equal_reserve():
    st = request_stream(n_req=24, rate=2.0, kv_size=128, n_stream=4, n_seq_max=8, token_budget=48,
                        n_ubatch=16, policy="reserve", block_size=8, split_mode="equal", seed=2503)
    s = serve_parity(st)
    print(s)
    assert s["preempted"] == 0 and s["rows"] > 200


def test_serving_swap_preemption():
    """Preempted sequences go to the swap arena and come back: their
    restored rows (other cells, other sequence ids) must attend exactly like
    the oracle's, which restores through the oracle's own save / load."""
    st = request_stream(n_req=28, rate=1.5, kv_size=96, token_budget=64, n_ubatch=32, preempt="swap",
                        swap_bytes=1 << 22, seed=2504)
    s = serve_parity(st)
    print(s)
    assert s["swapped"] > 0 and s["rows"] > 300


def test_serving_swap_arena_too_small_recomputes():
    st = request_stream(n_req=28, rate=2.0, kv_size=64, n_stream=4, n_seq_max=8, token_budget=64, n_ubatch=32,
                        preempt="swap", swap_bytes=32768, seed=2510)
    s = serve_parity(st)
    print(s)
    assert 0 < s["swapped"] < s["preempted"]
