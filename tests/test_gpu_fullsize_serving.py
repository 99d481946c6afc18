"""The iteration-level batching loop at full size, in the launch
configuration the benchmark times.

The Qwen3-0.6B-shaped serving stream (28 layers, one 131072-cell cache, up
to 64 running sequences, a 2048-position budget, n_ubatch 512) runs for 48
iterations: the first ones are prompt chunks filling the budget, the later
ones one decode token per running sequence plus the prompts of newcomers.
Every ubatch stores and attends all 28 layers in one call each, work items
sized for 28 layers.  The oracle loop drives the oracle engine in lockstep,
holding layer 27 only: every iteration's records and every ubatch's cells
are compared bit for bit, and at three iterations sampled rows of every
ubatch of layer 27 are compared with the fp64 oracle, row by row.  Layers
0..26 read a seeded pool (their values do not enter layer 27).
"""

import math

import numpy as np
import pytest
import torch

from oracle import OracleEngine
from oracle.attention import masked_attention
from oracle.scheduler import OracleScheduler
from synthetic.serving import qwen_serving

from helpers import assert_parity, mfma_query, weight_sigma

pytestmark = pytest.mark.gpu

KEYS = ("retired", "preempted", "admitted", "req", "seq", "pos", "output", "n_running", "n_waiting")


def test_serving_loop_full_size_sampled_layer():
    import ubatch_attention_paged_amd as K
    st = qwen_serving()
    L, CHECK, E, HD = st.n_layer, st.n_layer - 1, st.E, st.n_head * st.head_dim
    dev = torch.device("cuda:0")
    ctx = K.Context(L, st.n_head, st.n_head_kv, st.head_dim, st.kv_size, st.n_stream, st.n_seq_max,
                    st.token_budget, st.n_ubatch, device="cuda:0", attend_layers=L)
    sch = K.Scheduler(ctx, token_budget=st.token_budget, policy=st.policy, max_requests=st.n_requests)
    eng = OracleEngine(L, st.n_head, st.n_head_kv, st.head_dim, st.kv_size, st.n_stream, st.n_seq_max,
                       st.token_budget, st.n_ubatch, layers=[CHECK])
    ref = OracleScheduler(release=lambda q: eng.seq_rm(q), **st.sched_kwargs())
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    nb = st.token_budget
    pool_k = torch.randn((L - 1, nb, E), generator=g, device=dev)
    pool_v = torch.randn((L - 1, nb, E), generator=g, device=dev)
    pool_q = torch.randn((L - 1, nb, HD), generator=g, device=dev)
    outs = torch.empty((L, st.n_ubatch, HD), device=dev)
    cur = torch.cuda.current_stream().cuda_stream
    row = lambda t, l, r0, w: t.data_ptr() + 4 * (l * nb * w + r0 * w)
    check_at = {12, 30, 47}
    checked, items = 0, {"n_items_mfma": 0, "n_items_valu": 0}
    for it in range(48):
        for r in st.arrivals(it):
            assert sch.submit(int(st.n_prompt[r]), int(st.n_generate[r])) == \
                ref.submit(int(st.n_prompt[r]), int(st.n_generate[r]))
        sch.step()
        got, exp = sch.record(), ref.step()
        for key in KEYS:
            assert got[key] == exp[key], (it, key)
        n = len(exp["pos"])
        rng = np.random.default_rng(np.random.SeedSequence([st.seed, 5, it]))
        k27 = rng.standard_normal((n, E), dtype=np.float32)
        v27 = rng.standard_normal((n, E), dtype=np.float32)
        q27 = rng.standard_normal((n, HD), dtype=np.float32)
        dk, dv, dq = (torch.from_numpy(x).to(dev) for x in (k27, v27, q27))
        stt, ubs, _ = ctx.split_batch(sch.it.batch)
        rst, rubs, _ = eng.split(n, exp["pos"], [(q,) for q in exp["seq"]], exp["output"])
        assert stt == rst == 0 and len(ubs) == len(rubs)
        print(f"iteration {it}: {n} slots, {len(ubs)} ubatches, {got['n_running']} running", flush=True)
        for u, ru in zip(ubs, rubs):
            assert u.cells.tolist() == list(ru.cells)
            r0 = int(u.src[0])
            assert u.src.tolist() == list(range(r0, r0 + u.n_tokens))      # split_simple: contiguous rows
            kp = [row(pool_k, l, r0, E) for l in range(L - 1)] + [dk.data_ptr() + 4 * r0 * E]
            vp = [row(pool_v, l, r0, E) for l in range(L - 1)] + [dv.data_ptr() + 4 * r0 * E]
            qp = [row(pool_q, l, r0, HD) for l in range(L - 1)] + [dq.data_ptr() + 4 * r0 * HD]
            op = [outs.data_ptr() + 4 * l * st.n_ubatch * HD for l in range(L)]
            K.kvattn_store(ctx.ctx, u, 0, kp, vp, cur)
            K.kvattn_attend(ctx.ctx, u, 0, qp, op, 0, cur)
            check = it in check_at
            eng.commit(ru, build_mask=check)
            eng.store(ru, CHECK, k27[ru.src], v27[ru.src])
            if check:
                ps = ctx.plan_stats()
                for key in items:
                    items[key] += ps[key]
                got27 = outs[CHECK, :u.n_tokens].double().cpu().numpy()
                pick = np.unique(np.random.default_rng(it + u.id).integers(0, u.n_tokens, 24))
                streams = np.asarray(ru.streams)
                qp = q27[np.asarray(ru.src)[pick]]
                args = (eng.K[CHECK], eng.V[CHECK], streams[pick], ru.mask[pick], st.n_head, st.n_head_kv)
                want = masked_attention(qp, *args)
                qt = mfma_query(qp, st.head_dim)
                alt, sig = masked_attention(qt, *args, math.log(2.0)), weight_sigma(qt, *args, math.log(2.0))
                assert_parity(got27[pick], want, tag=f"iteration {it} ubatch {u.id}", alt=alt, sigma=sig)
                checked += len(pick)
        sch.advance()
        ref.advance()
    torch.cuda.synchronize()
    assert checked > 100 and ref.running
    assert items["n_items_mfma"] > 0 and items["n_items_valu"] > 0     # prompt chunks and decode tokens
