#!/usr/bin/env python3
"""Benchmark of the per-ubatch attention step on one MI355X.

Default workload: a 3000-token prompt on the Qwen3-0.6B shape (28 layers, 16
query heads over 8 KV heads of 128, F16 cache of 4096 cells), submitted as
caller calls of 2048 + 952 slots and split into six 512/440-slot ubatches.
One step = the whole path for that prompt: split + placement, then for every
ubatch the F16 K/V store, the visibility-list build and the attention, all
28 layers.  The cache is cleared before each step (the previous request is
retired).  Inputs are seeded synthetic tensors already resident in HBM.

Two decode workloads are measured in the same run and reported under
"decode": 64 continuous-batching sequences with contexts 64..2048 over a
shuffled 65536-cell cache, and 32 sequences sharing a 2048-cell prefix.  A
decode step appends one token per sequence (positions advance each step).

A mixed prefill + decode workload (8 prompts chunked alongside 56 decoders,
split_equal) is reported under "mixed", and the iteration-level batching
loop (the native scheduler admitting, retiring and assembling every
iteration over a stream of requests) under "serving", and save / restore of
a 2048-position sequence's state under "seq_state".

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense F16 matrix peak, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)




def gen_tensors(wl, b, layers, with_q, dev):
    import torch
    from synthetic import workloads as W
    kinds = [W.KIND_K, W.KIND_V] + ([W.KIND_Q] if with_q else [])
    jobs = [(l, k) for l in layers for k in kinds]
    with ThreadPoolExecutor(16) as ex:
        arrs = list(ex.map(lambda lk: wl.tensor(b, lk[0], lk[1]), jobs))
    d = dict(zip(jobs, arrs))
    # one [layers][tokens][width] allocation per tensor kind: a ubatch's rows of
    # every layer are then addressed by pointer arithmetic, no per-layer views
    stack = lambda kind: torch.from_numpy(np.stack([d[(l, kind)] for l in layers])).to(dev)
    K = stack(W.KIND_K)
    V = stack(W.KIND_V)
    Q = stack(W.KIND_Q) if with_q else None
    return K, V, Q


def row_ptrs(t, l0, l1, row0):
    """Addresses of row ``row0`` of layers l0..l1-1 of a [L][n][w] fp32 tensor."""
    L, n, wdt = t.shape
    base = t.data_ptr() + 4 * row0 * wdt
    return [base + 4 * l * n * wdt for l in range(l0, l1)]


def make_ctx(wl, dev, layer_chunk):
    from ubatch_attention_paged_amd import Context
    return Context(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                   wl.n_seq_max, wl.n_batch, wl.n_ubatch, wl.causal, cell_order=wl.cell_order,
                   device=dev, attend_layers=layer_chunk)


class TimingEvents:
    """HIP events for kernel timing, created with hipEventDisableSystemFence
    (timing kept, no system-scope cache writeback and invalidation when the
    kernel they are bound to ends -- with the default flags that fence slows
    the work after every timed kernel) through the HIP runtime torch has
    loaded."""

    _hip = None

    def __init__(self):
        import ctypes
        if TimingEvents._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            TimingEvents._hip = hip
        self.ct = ctypes
        self.pool = []
        self.used = []

    def reserve(self, n):
        """Create event pairs up to n unused ones (before the timed region)."""
        ct, hip = self.ct, TimingEvents._hip
        while len(self.pool) < n:
            pair = []
            for _ in range(2):
                e = ct.c_void_p()
                if hip.hipEventCreateWithFlags(ct.byref(e), 0x20000000) != 0:    # hipEventDisableSystemFence
                    raise RuntimeError("hipEventCreateWithFlags failed")
                pair.append(e.value)
            self.pool.append(tuple(pair))

    def take(self):
        if not self.pool:
            self.reserve(1)
        pair = self.pool.pop()
        self.used.append(pair)
        return pair

    def record(self, event, stream):
        if TimingEvents._hip.hipEventRecord(event, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def recycle(self):
        """Return the taken pairs to the pool (after synchronising): the
        warm-up steps run with timing too, so that the runtime has built
        whatever it keeps per timed launch before the timed region."""
        import torch
        torch.cuda.synchronize()
        self.pool.extend(self.used)
        self.used = []

    def elapsed_ms(self):
        """Elapsed times of the taken pairs, in order (synchronises)."""
        import torch
        torch.cuda.synchronize()
        ct, hip = self.ct, TimingEvents._hip
        out = []
        for a, b in self.used:
            f = ct.c_float()
            if hip.hipEventElapsedTime(ct.byref(f), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(f.value)
        return out

    def close(self):
        for a, b in self.pool + self.used:
            TimingEvents._hip.hipEventDestroy(a)
            TimingEvents._hip.hipEventDestroy(b)
        self.pool, self.used = [], []


class Runner:
    """Drives measured batches through the library and times every timed
    attend call with a pair of HIP events on the stream it runs on: by
    default recorded around the call (its kernels plus the gaps between
    them), or -- with ``kernel`` one of KVATTN_KERNEL_* -- bound by the
    library to that kernel's own start and end (kvattn_time_next_attend,
    hipExtLaunchKernel)."""

    def __init__(self, ctx, layer_chunk, kernel=None, keep_gathered=False):
        self.ctx = ctx
        self.chunk = layer_chunk
        self.kernel = kernel
        self.events = TimingEvents()
        self.calls = 0
        # A ubatch whose slots are not consecutive rows of the batch needs its
        # K/V/Q rows gathered into ubatch order (a forward pass would produce
        # them in that order).  With keep_gathered the gathered copies of the
        # first step are kept and reused by the later steps, which repeat the
        # same split, so the timed steps carry no harness copies.
        self.keep_gathered = keep_gathered
        self.gathered = {}

    def reserve(self, n):
        """n pairs ready for the timed region; the warm-up's are recycled."""
        self.events.recycle()
        self.events.reserve(n)

    def run_batch(self, n, pos, seqs, out_flags, K, V, Q, outs, timed):
        """K, V, Q: [layers][n][width] fp32 device tensors in batch order;
        outs: [layers][>= n_ubatch][n_head*head_dim]."""
        import torch
        from ubatch_attention_paged_amd import kvattn_store, kvattn_attend, kvattn_time_next_attend
        ctx = self.ctx
        st, ubs, _ = ctx.split(n, pos, seqs, out_flags)
        if st != 0:
            raise RuntimeError("cache full")
        L = K.shape[0]
        stream = torch.cuda.current_stream().cuda_stream
        for ub in ubs:
            src = ub.src
            if ub.n_tokens and not (src[-1] - src[0] == ub.n_tokens - 1):
                key = (K.data_ptr(), tuple(src.tolist()))
                hit = self.gathered.get(key)
                if hit is None:
                    idx = torch.as_tensor(src, device=K.device, dtype=torch.long)
                    hit = (K.index_select(1, idx), V.index_select(1, idx), Q.index_select(1, idx))
                    if self.keep_gathered:
                        self.gathered[key] = hit
                Kb, Vb, Qb = hit
                r0 = 0
            else:
                Kb, Vb, Qb, r0 = K, V, Q, int(src[0]) if ub.n_tokens else 0
            for a in range(0, L, self.chunk):
                b = min(L, a + self.chunk)
                kvattn_store(ctx.ctx, ub, a, row_ptrs(Kb, a, b, r0), row_ptrs(Vb, a, b, r0), stream)
                self.calls += 1
                if timed:
                    e0, e1 = self.events.take()
                    if self.kernel is None:
                        self.events.record(e0, stream)
                    else:
                        kvattn_time_next_attend(ctx.ctx, self.kernel, e0, e1)
                kvattn_attend(ctx.ctx, ub, a, row_ptrs(Qb, a, b, r0), row_ptrs(outs, a, b, 0), 0, stream)
                if timed and self.kernel is None:
                    self.events.record(e1, stream)
        return ubs

    def attend_avg_ms(self):
        vals = self.events.elapsed_ms()
        return float(np.mean(vals)) if vals else float("nan"), len(vals)

    def attend_by_position(self, per_step):
        """Mean attend time of the k-th attend call of a step, k < per_step."""
        vals = np.array(self.events.elapsed_ms()).reshape(-1, per_step)
        return vals.mean(axis=0).tolist()


# ---------------------------------------------------------------------------
# prefill (headline)

def prefill_pairs(wl):
    """Visible (query, cell) pairs of one step: every prompt token sees
    itself and every earlier token of its sequence."""
    return sum(int((bt.pos.astype(np.int64) + 1).sum()) for bt in wl.batches)


def bench_prefill(wl, dev, steps, warmup, layer_chunk, kernel=None):
    """kernel: the attend call's kernel to time (KVATTN_KERNEL_*), default
    the whole call.  After the warm-up, a pass of `steps` steps binds the
    events to every launch and gives the per-launch times (attend_*) and its
    own wall time (ms_per_step_timed); then the `steps` timed steps run
    with no per-launch events (wall_s, ms_per_step: the throughput), since
    a launch that carries events costs the step a few microseconds."""
    import torch
    ctx = make_ctx(wl, dev, layer_chunk)
    layers = list(range(wl.n_layer))
    log(f"[bench] prefill: generating inputs ({wl.note})")
    from ubatch_attention_paged_amd import SeqIds
    data = [gen_tensors(wl, b, layers, True, dev) for b in range(len(wl.batches))]
    sids = [SeqIds(bt.seq_ids) for bt in wl.batches]
    HD = wl.n_head * wl.head_dim
    outs = torch.empty((len(layers), wl.n_ubatch, HD), dtype=torch.float32, device=dev)
    runner = Runner(ctx, layer_chunk, kernel)

    def step(timed):
        ctx.seq_rm(-1)                          # retire the previous request
        for b, bt in enumerate(wl.batches):
            K, V, Q = data[b]
            runner.run_batch(bt.n_tokens, bt.pos, sids[b], bt.output, K, V, Q, outs, timed)

    for _ in range(warmup):
        step(True)
    runner.reserve(steps * runner.calls // max(1, warmup))
    # every attend launch timed by its own events
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    wall_timed = time.perf_counter() - t1
    # the timed region: the same steps with no per-launch events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms, n_launch = runner.attend_avg_ms()
    stats = ctx.plan_stats()
    pairs = prefill_pairs(wl)
    flops_step = 4.0 * wl.n_head * wl.head_dim * wl.n_layer * pairs
    n_ub_step = n_launch / steps
    per_ub = runner.attend_by_position(int(round(n_launch / steps)))
    # flops of each ubatch (split_simple over the caller calls, positions in order)
    ub_flops = []
    for bt in wl.batches:
        for a0 in range(0, bt.n_tokens, wl.n_ubatch):
            p = bt.pos[a0:a0 + wl.n_ubatch].astype(np.int64)
            ub_flops.append(4.0 * wl.n_head * wl.head_dim * wl.n_layer * float((p + 1).sum()))
    if len(ub_flops) == len(per_ub) and layer_chunk >= wl.n_layer:
        log("[bench] prefill per ubatch: " + ", ".join(
            f"{ms:.3f} ms {f / (ms * 1e-3) / 1e12:.0f} TF/s" for ms, f in zip(per_ub, ub_flops)))
    res = dict(wall_s=wall, ms_per_step=1e3 * wall / steps, ms_per_step_timed=1e3 * wall_timed / steps,
               tokens=wl.measured_tokens(), flops_step=flops_step, attend_launches_per_step=n_ub_step,
               attend_avg_ms=avg_ms, attend_ms_per_step=avg_ms * n_ub_step, last_plan=stats)
    runner.events.close()
    ctx.close()
    return res


# ---------------------------------------------------------------------------
# decode

def decode_step_cells(wl, t):
    """Unique cells read by decode step t (the context of every sequence
    plus the new token; a cell shared by several sequences counts once)."""
    ctx_cells = set()
    # cells are identified by (first batch, slot) of the setup batches
    for b, bt in enumerate(wl.batches):
        if bt.measured:
            continue
        for i in range(bt.n_tokens):
            ctx_cells.add((b, i))
    n_seq = wl.batches[-1].n_tokens
    return len(ctx_cells) + n_seq * (t + 1)


def bench_decode(wl, dev, steps, warmup, layer_chunk):
    import torch
    from ubatch_attention_paged_amd.harness import decode
    ctx = make_ctx(wl, dev, layer_chunk)
    layers = list(range(wl.n_layer))
    log(f"[bench] decode {wl.name}: filling the context ({wl.note})")
    t0 = time.perf_counter()
    for b, bt in enumerate(wl.batches):
        if bt.measured:
            continue
        K, V, _ = gen_tensors(wl, b, layers, False, dev)
        st, _, _ = decode(ctx, bt.n_tokens, bt.pos, bt.seq_ids, bt.output, list(K), list(V))
        assert st == 0
        del K, V
    torch.cuda.synchronize()
    log(f"[bench] decode {wl.name}: context filled in {time.perf_counter() - t0:.1f}s")
    mb = len(wl.batches) - 1
    bt = wl.batches[mb]
    K, V, Q = gen_tensors(wl, mb, layers, True, dev)
    from ubatch_attention_paged_amd import SeqIds
    sid = SeqIds(bt.seq_ids)
    HD = wl.n_head * wl.head_dim
    outs = torch.empty((len(layers), bt.n_tokens, HD), dtype=torch.float32, device=dev)
    runner = Runner(ctx, layer_chunk)
    t = 0
    for _ in range(warmup):
        runner.run_batch(bt.n_tokens, bt.pos + t, sid, bt.output, K, V, Q, outs, True)
        t += 1
    runner.reserve(steps * runner.calls // max(1, warmup))
    # a pass with events around every attend call (the attend times), then
    # the timed steps without them (the throughput): each event in the
    # stream holds the next kernel back a few microseconds
    torch.cuda.synchronize()
    t_first = t
    for _ in range(steps):
        runner.run_batch(bt.n_tokens, bt.pos + t, sid, bt.output, K, V, Q, outs, True)
        t += 1
    torch.cuda.synchronize()
    cells = np.mean([decode_step_cells(wl, s) for s in range(t_first, t)])
    t0 = time.perf_counter()
    for _ in range(steps):
        runner.run_batch(bt.n_tokens, bt.pos + t, sid, bt.output, K, V, Q, outs, False)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms, n_launch = runner.attend_avg_ms()
    row = 2 * wl.n_head_kv * wl.head_dim * 2                       # K + V bytes per cell per layer
    kv_bytes = cells * row * wl.n_layer
    qo_bytes = 2 * bt.n_tokens * HD * 4 * wl.n_layer
    launches = n_launch / steps
    # the decode metric counts the unique K/V bytes a step must read; the
    # fp32 query and output rows are reported beside it, not in it
    gbs = kv_bytes / launches / (avg_ms * 1e-3) / 1e9
    res = dict(wall_s=wall, ms_per_step=1e3 * wall / steps, tokens_per_step=bt.n_tokens,
               tokens_per_s=bt.n_tokens * steps / wall, unique_cells=float(cells),
               kv_bytes_step=kv_bytes, qo_bytes_step=qo_bytes, attend_avg_ms=avg_ms,
               attend_launches_per_step=launches, kv_read_gbs=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
               kv_qo_gbs=(kv_bytes + qo_bytes) / launches / (avg_ms * 1e-3) / 1e9, plan=ctx.plan_stats())
    runner.events.close()
    ctx.close()
    return res


# ---------------------------------------------------------------------------
# mixed prefill + decode (non-unified cache, split_equal)

def bench_mixed(wl, dev, steps, warmup, layer_chunk):
    """Every measured call of the mixed workload (one decode token per decoder
    plus prompt chunks, split_equal into ubatches) per step; the prompts and
    the decoders' new tokens are retired between steps.  Ubatches whose
    sequences each contribute one slot run on the vector-ALU decode kernel
    (HBM-bound); prompt-chunk ubatches on the matrix cores.  The K/V/Q rows
    of each ubatch are gathered into ubatch order once, in the first
    warm-up step, as a forward pass would produce them."""
    import torch
    from ubatch_attention_paged_amd.harness import decode
    from ubatch_attention_paged_amd import SeqIds
    ctx = make_ctx(wl, dev, layer_chunk)
    layers = list(range(wl.n_layer))
    log(f"[bench] mixed: filling the decoders' contexts ({wl.note})")
    t0 = time.perf_counter()
    ctx_len = {}
    for b, bt in enumerate(wl.batches):
        if bt.measured:
            continue
        K, V, _ = gen_tensors(wl, b, layers, False, dev)
        st, _, _ = decode(ctx, bt.n_tokens, bt.pos, bt.seq_ids, bt.output, list(K), list(V))
        assert st == 0
        del K, V
        for p, s in zip(bt.pos, bt.seq_ids):
            ctx_len[s[0]] = max(ctx_len.get(s[0], 0), int(p) + 1)
    meas = [b for b, bt in enumerate(wl.batches) if bt.measured]
    data = {b: gen_tensors(wl, b, layers, True, dev) for b in meas}
    sids = {b: SeqIds(wl.batches[b].seq_ids) for b in meas}
    torch.cuda.synchronize()
    log(f"[bench] mixed: ready in {time.perf_counter() - t0:.1f}s, {len(meas)} measured calls")
    prompts = sorted({s[0] for b in meas for s in wl.batches[b].seq_ids} - set(ctx_len))
    HD = wl.n_head * wl.head_dim
    outs = torch.empty((len(layers), wl.n_ubatch, HD), dtype=torch.float32, device=dev)
    runner = Runner(ctx, layer_chunk, keep_gathered=True)

    def step(timed):
        for k in prompts:
            ctx.seq_rm(k)
        for d, n in ctx_len.items():
            ctx.seq_rm(d, n, -1)
        shapes = []
        for b in meas:
            bt = wl.batches[b]
            K, V, Q = data[b]
            for ub in runner.run_batch(bt.n_tokens, bt.pos, sids[b], bt.output, K, V, Q, outs, timed):
                shapes.append((ub.n_seq_tokens, np.asarray(ub.pos, np.int64).copy()))
        return shapes

    for _ in range(warmup):
        shapes = step(True)
    runner.reserve(steps * runner.calls // max(1, warmup))
    # a pass with events around every attend call (the per-ubatch attend
    # times), then the timed steps without them (the throughput)
    torch.cuda.synchronize()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    chunk_calls = (wl.n_layer + layer_chunk - 1) // layer_chunk
    per_call = runner.attend_by_position(len(shapes) * chunk_calls)
    per_ub = [sum(per_call[u * chunk_calls:(u + 1) * chunk_calls]) for u in range(len(shapes))]
    single = [u for u, (nst, _) in enumerate(shapes) if nst == 1]
    chunks = [u for u in range(len(shapes)) if u not in single]
    row = 2 * wl.n_head_kv * wl.head_dim * 2
    # one sequence id per slot, contiguous positions from 0: a slot at
    # position p sees p + 1 cells, none shared with another slot
    cells = lambda u: float((shapes[u][1] + 1).sum())
    ms_single = sum(per_ub[u] for u in single)
    ms_chunks = sum(per_ub[u] for u in chunks)
    kv_bytes = sum(cells(u) for u in single) * row * wl.n_layer
    flops = sum(cells(u) for u in chunks) * 4.0 * HD * wl.n_layer
    tokens = sum(wl.batches[b].n_tokens for b in meas)
    res = dict(workload=wl.note, tokens_per_s=round(tokens * steps / wall, 1), ms_per_step=round(1e3 * wall / steps, 4),
               tokens_per_step=tokens, ubatches_per_step=len(shapes))
    if single:
        gbs = kv_bytes / (ms_single * 1e-3) / 1e9
        res["single_token_ubatches"] = dict(count=len(single), attend_ms=round(ms_single, 4),
                                            kv_read_gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
    if chunks:
        tf = flops / (ms_chunks * 1e-3) / 1e12
        # a chunk's fp32 q rows are read and its fp32 outputs written once,
        # and each sequence's visible cells (its positions 0..max) once per
        # layer: short chunks over short histories carry ~80 flop per byte,
        # far below the ~310 at which the matrix cores would bind
        qo = sum(shapes[u][1].size for u in chunks) * HD * 4 * 2
        kv = sum(float((shapes[u][1].reshape(-1, shapes[u][0]).max(axis=1) + 1).sum()) for u in chunks) * row
        chunk_bytes = (qo + kv) * wl.n_layer
        hbm_ms = chunk_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
        mfma_ms = flops / (MFMA_F16_PEAK_TFLOPS * 1e12) * 1e3
        res["prompt_chunk_ubatches"] = dict(count=len(chunks), attend_ms=round(ms_chunks, 4),
                                            tflops=round(tf, 1), mfma_frac=round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                            bytes=round(chunk_bytes), flop_per_byte=round(flops / chunk_bytes, 1),
                                            gbs=round(chunk_bytes / (ms_chunks * 1e-3) / 1e9, 1),
                                            bound="hbm" if hbm_ms >= mfma_ms else "mfma",
                                            roofline_frac=round(max(hbm_ms, mfma_ms) / ms_chunks, 4))
    runner.events.close()
    ctx.close()
    return res


# ---------------------------------------------------------------------------
# iteration-level batching loop (native scheduler) over a request stream

def bench_serving(stream, dev, warm_iters, timed_iters, layer_chunk, swap_bytes=0):
    """The native loop (retire, admit, assemble) drives the context for
    warm_iters untimed iterations, then timed_iters timed ones.  Every
    iteration splits the assembled batch and, for each ubatch, stores K/V and
    runs attention for all slots over all layers.  K/V/Q rows come from a
    seeded pool resident in HBM (the values do not steer the loop)."""
    import torch
    from ubatch_attention_paged_amd import Context, Scheduler, kvattn_store, kvattn_attend
    L = stream.n_layer
    ctx = Context(L, stream.n_head, stream.n_head_kv, stream.head_dim, stream.kv_size, stream.n_stream,
                  stream.n_seq_max, stream.token_budget, stream.n_ubatch, device=dev, attend_layers=layer_chunk,
                  split_mode=stream.split_mode)
    sch = Scheduler(ctx, token_budget=stream.token_budget, policy=stream.policy, block_size=stream.block_size,
                    chunked=stream.chunked, max_requests=stream.n_requests, preempt=stream.preempt,
                    swap_bytes=swap_bytes)
    g = torch.Generator(device=dev)
    g.manual_seed(stream.seed)
    nb, HD = stream.token_budget, stream.n_head * stream.head_dim
    K = torch.randn((L, nb, stream.E), generator=g, device=dev)
    V = torch.randn((L, nb, stream.E), generator=g, device=dev)
    Q = torch.randn((L, nb, HD), generator=g, device=dev)
    outs = torch.empty((L, stream.n_ubatch, HD), dtype=torch.float32, device=dev)
    cur = torch.cuda.current_stream().cuda_stream
    # event pairs recorded around each timed attend call, created before timing
    events = TimingEvents()

    def iteration(k, timed):
        for r in stream.arrivals(k):
            sch.submit(int(stream.n_prompt[r]), int(stream.n_generate[r]))
        t0 = time.perf_counter()
        it = sch.step()
        t_sched = time.perf_counter() - t0
        n = it.batch.n_tokens
        info = (n, it.n_decode, 0, it.n_running, it.n_waiting, it.n_preempted, 0, 0, it.n_swapped_out)
        if n:
            pos = np.ctypeslib.as_array(it.batch.pos, shape=(n,)).astype(np.int64)
            req = np.ctypeslib.as_array(it.req, shape=(n,))
            out = np.ctypeslib.as_array(it.batch.output, shape=(n,))
            # one sequence id per slot, each sequence's slots contiguous and
            # ascending: the last slot of a run at position p reads p + 1
            # cells once for its whole visibility class
            last = np.nonzero(np.append(req[1:] != req[:-1], True))[0]
            info = (n, it.n_decode, int(out.sum()), it.n_running, it.n_waiting, it.n_preempted,
                    int((pos[last] + 1).sum()), int((pos + 1).sum()), it.n_swapped_out)
        if n:
            st, ubs, _ = ctx.split_batch(it.batch)
            if st != 0:
                raise RuntimeError("the loop assembled a batch the cache cannot hold")
            for ub in ubs:
                r0 = int(ub.src[0])
                assert ub.src[-1] - r0 == ub.n_tokens - 1
                for a in range(0, L, layer_chunk):
                    b = min(L, a + layer_chunk)
                    kvattn_store(ctx.ctx, ub, a, row_ptrs(K, a, b, r0), row_ptrs(V, a, b, r0), cur)
                    if timed:
                        e0, e1 = events.take()
                        events.record(e0, cur)
                    kvattn_attend(ctx.ctx, ub, a, row_ptrs(Q, a, b, r0), row_ptrs(outs, a, b, 0), 0, cur)
                    if timed:
                        events.record(e1, cur)
        sch.advance()
        return t_sched, info

    log(f"[bench] serving: {warm_iters} warm-up iterations")
    for k in range(warm_iters):
        iteration(k, True)
    events.recycle()
    # at most token_budget / n_ubatch + n_stream ubatches per iteration
    events.reserve(timed_iters * ((nb + stream.n_ubatch - 1) // stream.n_ubatch + stream.n_stream)
                   * ((L + layer_chunk - 1) // layer_chunk))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = [iteration(warm_iters + k, True) for k in range(timed_iters)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attend_ms = sum(events.elapsed_ms())
    events.close()
    sched_us = np.array([r[0] for r in recs]) * 1e6
    info = np.array([r[1] for r in recs], dtype=np.int64)
    slots, dec, gen = int(info[:, 0].sum()), int(info[:, 1].sum()), int(info[:, 2].sum())
    row = 2 * stream.n_head_kv * stream.head_dim * 2
    kv_bytes = float(info[:, 6].sum()) * row * L         # visible cells, each read once per class
    flops = float(info[:, 7].sum()) * 4.0 * HD * L        # QK^T and PV over visible (query, cell) pairs
    bound_ms = max(kv_bytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_F16_PEAK_TFLOPS * 1e12)) * 1e3
    res = dict(workload=f"{stream.name}: {stream.note()}", iterations=timed_iters,
               generated_tokens_per_s=round(gen / wall, 1), positions_per_s=round(slots / wall, 1),
               ms_per_iteration=round(1e3 * wall / timed_iters, 4),
               attend_ms_per_iteration=round(attend_ms / timed_iters, 4),
               sched_step_us=dict(mean=round(float(sched_us.mean()), 2),
                                  p99=round(float(np.percentile(sched_us, 99)), 2)),
               mean_running=round(float(info[:, 3].mean()), 2), mean_waiting=round(float(info[:, 4].mean()), 1),
               decode_slot_frac=round(dec / max(1, slots), 4), preemptions=int(info[:, 5].sum()),
               swapped_out=int(info[:, 8].sum()), positions_per_generated=round(slots / max(1, gen), 3),
               attend_kv_read_gbs=round(kv_bytes / (attend_ms * 1e-3) / 1e9, 1),
               attend_tflops=round(flops / (attend_ms * 1e-3) / 1e12, 1),
               attend_roofline_frac=round(bound_ms / attend_ms, 4))
    sch.close()
    ctx.close()
    return res


# ---------------------------------------------------------------------------
# sequence-state save / restore

def bench_seq_state(dev, n_pos=2048, reps=10):
    """Save and restore of one n_pos-position sequence of the Qwen3-0.6B
    shape (28 layers, F16 rows of 2 KiB): each save gathers 2 * 28 * n_pos
    scattered cache rows into the blob, each restore scatters them back into
    freshly placed cells (after reading the blob's metadata back)."""
    import torch
    from ubatch_attention_paged_amd import Context
    L, E = 28, 1024
    order = np.random.default_rng(9).permutation(4096).astype(np.int32)[None, :]
    ctx = Context(L, 16, 8, 128, 4096, 1, 4, 2048, 512, device=dev, attend_layers=L, cell_order=order)
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    st, ubs, _ = ctx.split(n_pos, list(range(n_pos)), [(0,)] * n_pos, None)
    assert st == 0
    for u in ubs:
        ctx.store(u, 0, [torch.randn((u.n_tokens, E), generator=g, device=dev) for _ in range(L)],
                  [torch.randn((u.n_tokens, E), generator=g, device=dev) for _ in range(L)])
    blob = torch.empty(ctx.state_size(0), dtype=torch.uint8, device=dev)
    for _ in range(2):
        ctx.state_save(0, blob)
        ctx.state_load(1, blob)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        ctx.state_save(0, blob)
        e1.record()
    torch.cuda.synchronize()
    save_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    t0 = time.perf_counter()
    for _ in range(reps):
        ctx.state_load(1, blob)
    torch.cuda.synchronize()
    load_ms = 1e3 * (time.perf_counter() - t0) / reps
    payload = 2 * L * n_pos * E * 2
    moved = 2 * payload                       # each row read once and written once
    res = dict(workload=f"one {n_pos}-position sequence, 28 layers, 8 KV heads x 128, shuffled cells",
               blob_bytes=int(blob.numel()), save_ms=round(save_ms, 4),
               save_gbs=round(moved / (save_ms * 1e-3) / 1e9, 1),
               save_hbm_frac=round(moved / (save_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               load_ms_wall=round(load_ms, 4), load_gbs_wall=round(moved / (load_ms * 1e-3) / 1e9, 1))
    ctx.close()
    return res


# ---------------------------------------------------------------------------
# oracle on the host cores

def host_description():
    """Host cores, the BLAS threads numpy's matrix products use (the threads
    the oracle actually runs on) and the CPU model."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(host_cpus=os.cpu_count(), blas_threads=int(blas), cpu_model=model)


def cpu_baseline_prefill(wl, budget_s=25.0):
    """The fp64 oracle over the same prompt for as many layers as fit in
    about budget_s, scaled to the full step."""
    from oracle import OracleEngine
    from synthetic import workloads as W
    done_layers, t_all = 0, 0.0
    for layer in range(wl.n_layer):
        eng = OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                           wl.n_seq_max, wl.n_batch, wl.n_ubatch, wl.causal, cell_order=wl.cell_order,
                           layers=[layer])
        tens = [(wl.tensor(b, layer, W.KIND_K), wl.tensor(b, layer, W.KIND_V), wl.tensor(b, layer, W.KIND_Q))
                for b in range(len(wl.batches))]
        t0 = time.perf_counter()
        for b, bt in enumerate(wl.batches):
            st, ubs, _ = eng.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
            k, v, q = tens[b]
            for ub in ubs:
                eng.commit(ub)
                eng.store(ub, layer, k[ub.src], v[ub.src])
                eng.attend(ub, layer, q[ub.src])
        t_all += time.perf_counter() - t0
        done_layers += 1
        if t_all >= budget_s:
            break
    per_step = t_all / done_layers * wl.n_layer
    return dict(value=round(wl.measured_tokens() / per_step, 2), unit="tokens/s",
                sample=f"{done_layers} of {wl.n_layer} layers of the full {wl.measured_tokens()}-token prompt "
                       f"(all {len(wl.batches)} calls, every ubatch: split, placement, mask, store, attention), "
                       f"{t_all:.1f}s, scaled x{wl.n_layer / done_layers:.2f}")


def cpu_baseline_decode(wl, layers):
    """The fp64 oracle on one decode step of ``wl`` for the sampled layers:
    the context is stored first (untimed, as on the GPU), then the step's
    split + placement + mask (once) and store + attention (per layer) are
    timed and scaled to every layer."""
    from oracle import OracleEngine
    from synthetic import workloads as W
    eng = OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                       wl.n_seq_max, wl.n_batch, wl.n_ubatch, wl.causal, cell_order=wl.cell_order, layers=layers)
    t_setup = time.perf_counter()
    for b, bt in enumerate(wl.batches):
        if bt.measured:
            continue
        st, ubs, _ = eng.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0
        tens = {l: (wl.tensor(b, l, W.KIND_K), wl.tensor(b, l, W.KIND_V)) for l in layers}
        for ub in ubs:
            eng.commit(ub, build_mask=False)
            for l in layers:
                eng.store(ub, l, tens[l][0][ub.src], tens[l][1][ub.src])
    t_setup = time.perf_counter() - t_setup
    mb = len(wl.batches) - 1
    bt = wl.batches[mb]
    tens = {l: [wl.tensor(mb, l, k) for k in (W.KIND_K, W.KIND_V, W.KIND_Q)] for l in layers}
    t0 = time.perf_counter()
    st, ubs, _ = eng.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
    for ub in ubs:
        eng.commit(ub)
    t_once = time.perf_counter() - t0
    t_layers = 0.0
    for l in layers:
        k, v, q = tens[l]
        t0 = time.perf_counter()
        for ub in ubs:
            eng.store(ub, l, k[ub.src], v[ub.src])
            eng.attend(ub, l, q[ub.src])
        t_layers += time.perf_counter() - t0
    per_step = t_once + t_layers / len(layers) * wl.n_layer
    return dict(value=round(bt.n_tokens / per_step, 2), unit="tokens/s",
                sample=f"one decode step of {bt.n_tokens} sequences ({wl.note}): split, placement and mask "
                       f"{t_once:.2f}s once, store + attention of {len(layers)} of {wl.n_layer} layers "
                       f"{t_layers:.1f}s, scaled x{wl.n_layer / len(layers):.2f}; the context "
                       f"({t_setup:.0f}s to store) is not timed, as on the GPU")


def cpu_baseline(wl_prefill):
    """The oracle as it stands, on this host's cores, for the prefill (the
    headline) and the two decode workloads."""
    from synthetic import workloads as W
    pre = cpu_baseline_prefill(wl_prefill)
    cfg = {"qwen_prefill": pre,
           "cb_decode": cpu_baseline_decode(W.cb_decode(), [0, 27]),
           "prefix_decode": cpu_baseline_decode(W.prefix_decode(), [0, 9, 18, 27])}
    host = host_description()
    return dict(value=pre["value"], unit="tokens/s", cores=host["blas_threads"], kind="oracle",
                sample=pre["sample"], **host, configs=cfg)


def kernel_source_digest(source):
    """sha256 over a kernel source file and, recursively, the local headers
    it includes (csrc/ or include/), in name order: a change to any of them
    changes the compiled kernel."""
    import hashlib
    import re
    dirs = [os.path.join(ROOT, "ubatch_attention_paged_amd", "csrc"), os.path.join(ROOT, "include")]

    def find(name):
        for d in dirs:
            f = os.path.join(d, name)
            if os.path.exists(f):
                return f
        return None

    seen, todo = {}, [source]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        f = find(name)
        if f is None:
            continue
        seen[name] = open(f, "rb").read()
        todo.extend(re.findall(r'#include "([^"]+)"', seen[name].decode("utf-8", "replace")))
    h = hashlib.sha256()
    for name in sorted(seen):
        h.update(name.encode())
        h.update(seen[name])
    return h.hexdigest()


def committed_trace_ms(kernel, source, leg):
    """Mean duration (ms) of ``kernel`` over the timed dispatches of ``leg``
    from the committed rocprofv3 kernel-trace summary (profiles/
    <kernel>_trace.json: the dispatches of exactly the loop the HIP events
    time, picked out of the whole run's trace by --trace-stats --skip /
    --take); None when absent or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_trace.json")
    try:
        rec = json.load(open(path))
        digest = kernel_source_digest(source)
    except (OSError, ValueError):
        return None
    legs = rec.get("legs", {})
    if rec.get("source_digest") != digest or leg not in legs:
        return None
    return legs[leg]["avg_ns"] * 1e-6


def _trace_rows(csv_path):
    """(dispatch id, bare kernel name, full name, duration ns) of every
    dispatch in a rocprofv3 kernel_trace.csv, in dispatch order."""
    import csv
    out = []
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            bare = (name[5:] if name.startswith("void ") else name).split("(")[0].split("<")[0].split("::")[-1]
            out.append((int(row["Dispatch_Id"]), bare, name, int(row["End_Timestamp"]) - int(row["Start_Timestamp"])))
    out.sort()
    return out


def trace_stats(csv_path, kernel, skip, take):
    """Duration statistics of the dispatches of ``kernel`` (name prefix, after
    an optional "void " and namespace) in a rocprofv3 kernel_trace.csv, in
    dispatch order: the first ``skip`` are dropped (warm-up), the next
    ``take`` kept (0 = all the rest)."""
    durs = [d for _, bare, _, d in _trace_rows(csv_path) if bare == kernel]
    sel = durs[skip:skip + take if take else None]
    if not sel:
        raise SystemExit(f"no dispatches of {kernel} left after skipping {skip} of {len(durs)}")
    a = np.asarray(sel, dtype=np.float64)
    return dict(kernel=kernel, dispatches_total=len(durs), skipped=skip, n=len(sel), avg_ns=round(float(a.mean()), 1),
                min_ns=int(a.min()), max_ns=int(a.max()), median_ns=float(np.median(a)))


def trace_table(csv_path, kernel, skip, take, step_start):
    """Per-kernel calls / mean / total of every dispatch in the steps that
    hold the selected dispatches of ``kernel``: a step begins at a dispatch
    of ``step_start`` (the first kernel each step launches; several names
    joined by commas) and the window ends before the next step's first
    dispatch, the next dispatch of ``kernel`` or the first kernel of another
    library (the next bench leg)."""
    rows = _trace_rows(csv_path)
    starts = set(step_start.split(","))
    idx = [i for i, r in enumerate(rows) if r[1] == kernel]
    sel = idx[skip:skip + take if take else None]
    if not sel:
        raise SystemExit(f"no dispatches of {kernel} left after skipping {skip} of {len(idx)}")
    a = sel[0]
    while a > 0 and rows[a][1] not in starts:
        a -= 1
    b = sel[-1] + 1
    while b < len(rows) and "kvattn::" in rows[b][2] and rows[b][1] not in starts and rows[b][1] != kernel:
        b += 1
    stats = {}
    for _, _, name, d in rows[a:b]:
        s = stats.setdefault(name, [0, 0])
        s[0] += 1
        s[1] += d
    total = sum(v[1] for v in stats.values())
    lines = [f"{'kernel':<64}{'calls':>7}{'avg_us':>10}{'total_ms':>10}{'pct':>7}"]
    for name, (c, d) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"{name[:62]:<64}{c:>7}{d / c / 1e3:>10.2f}{d / 1e6:>10.3f}{100 * d / total:>7.2f}")
    return "\n".join(lines)


def counter_stats(csv_path, kernel, skip, take):
    """Mean per dispatch of every counter in a rocprofv3 --pmc
    counter_collection.csv, over the dispatches of ``kernel`` (same
    selection as trace_stats)."""
    import csv
    per = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            name = name[5:] if name.startswith("void ") else name
            if name.split("(")[0].split("<")[0].split("::")[-1] != kernel:
                continue
            d = per.setdefault(int(row["Dispatch_Id"]), {})
            d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    ids = sorted(per)[skip:skip + take if take else None]
    if not ids:
        raise SystemExit(f"no dispatches of {kernel} left after skipping {skip} of {len(per)}")
    names = sorted({k for i in ids for k in per[i]})
    return dict(kernel=kernel, dispatches_total=len(per), skipped=skip, n=len(ids),
                mean=dict((k, float(np.mean([per[i].get(k, 0.0) for i in ids]))) for k in names))


PROFILE_COMMAND = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out> "
                   "-o run -- python -u <repo>/bench.py --gpus 1 --steps 20 --warmup 5 --no-cpu-baseline")

KERNEL_SOURCES = {"k_attn_mfma": "attn_mfma.hip", "k_attn_valu": "attn_valu.hip", "k_attn_reduce": "attn_valu.hip",
                  "k_attn_both": "attn_both.hip",
                  "k_store_commit": "kernels_commit.hip", "k_store": "kernels_commit.hip"}


def write_trace_record(path, kernel, leg, rec, argv, profile_command):
    """Merge one leg's statistics into the per-kernel summary JSON, with the
    digest of the kernel's sources as they are now (run it in the tree that
    was profiled) and the rocprofv3 command whose trace it summarises."""
    try:
        out = json.load(open(path))
    except (OSError, ValueError):
        out = {}
    out["kernel"] = kernel
    out["source_digest"] = kernel_source_digest(KERNEL_SOURCES[kernel])
    out.pop("profile_command", None)
    out.setdefault("legs", {})[leg] = dict(rec, profile_command=profile_command,
                                           summary_command=f"python bench.py {argv}".replace(ROOT + "/", ""))
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


def hbm_copy_gbs(dev, nbytes=2 << 30, reps=10):
    """Device-to-device copy of nbytes with torch (read + write both
    counted), timed with HIP events: what the memory system delivers to a
    plain streaming kernel, for context beside the 8 TB/s spec."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def ceilings(dev, reps=10):
    """What this GPU delivers to the two instruction forms the attention
    kernels are built on, measured through the library's probes and timed
    with fence-free HIP events: whole 2 KiB rows read in a shuffled order
    (every row of a 2 GiB buffer once per launch: the decode kernel's access,
    read-only) and back-to-back independent 32x32x16 F16 matrix-core
    products (the prefill kernel's instruction)."""
    import torch
    from ubatch_attention_paged_amd import kvattn_probe_gather, kvattn_probe_mfma
    stream = torch.cuda.current_stream().cuda_stream
    n_rows = 1 << 20
    rows = torch.full((n_rows, 1024), 0.5, dtype=torch.float16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    index = torch.randperm(n_rows, generator=g, device=dev).to(torch.int32)
    n_wg = 1024                      # 4 wavefronts per SIMD: the best of 512 .. 16384 measured
    out = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    ev = TimingEvents()
    ev.reserve(2 * reps)

    def timed(launch):
        for _ in range(2):
            launch()
        ev.recycle()
        for _ in range(reps):
            e0, e1 = ev.take()
            ev.record(e0, stream)
            launch()
            ev.record(e1, stream)
        ms = float(np.mean(ev.elapsed_ms()))
        ev.recycle()
        return ms

    g_ms = timed(lambda: kvattn_probe_gather(rows.data_ptr(), n_rows, index.data_ptr(), n_rows, out.data_ptr(),
                                             n_wg, stream))
    index.copy_(torch.arange(n_rows, device=dev, dtype=torch.int32))
    s_ms = timed(lambda: kvattn_probe_gather(rows.data_ptr(), n_rows, index.data_ptr(), n_rows, out.data_ptr(),
                                             n_wg, stream))
    gbs, sgbs = (n_rows * 2048 / (t * 1e-3) / 1e9 for t in (g_ms, s_ms))
    del rows, index
    ab = torch.ones(16, dtype=torch.float16, device=dev)
    m_wg, iters = 4096, 4096
    out = torch.empty(m_wg * 256, dtype=torch.float32, device=dev)
    m_ms = timed(lambda: kvattn_probe_mfma(ab.data_ptr(), out.data_ptr(), m_wg, iters, stream))
    tf = m_wg * 4 * iters * 4 * 32768 / (m_ms * 1e-3) / 1e12
    ev.close()
    return {"gather_read_gbs": round(gbs, 1), "gather_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "sequential_read_gbs": round(sgbs, 1),
            "mfma_f16_tflops": round(tf, 1), "mfma_frac_of_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "how": "library probes: every row of a 2 GiB buffer of 2 KiB rows read once per launch, in a "
                   "shuffled order and in order, 1024 workgroups of 4 wavefronts; 4096 workgroups x 4 "
                   "wavefronts x 4096 rounds of four independent 32x32x16 F16 products"}


def committed_traffic(kernel, source):
    """HBM bytes per launch of ``kernel`` from the committed FETCH_SIZE /
    WRITE_SIZE summary, scaled by the copy-kernel calibration recorded there;
    None when no summary exists or the kernel's sources changed since it was
    taken (the summary stores kernel_source_digest of them)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    try:
        rec = json.load(open(path))
        digest = kernel_source_digest(source)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != digest:
        return None
    return round(rec["bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layer-chunk", type=int, default=28,
                    help="layers per store/attend call (28 = one call per ubatch, 1 = per layer)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-layer", action="store_true",
                    help="skip the one-call-per-layer runs of the prefill and 64-sequence decode")
    ap.add_argument("--trace-stats", metavar="CSV",
                    help="no GPU: statistics of one kernel's dispatches in a rocprofv3 kernel_trace.csv, "
                         "skipping the first --skip (warm-up) and taking the next --take (the timed loop)")
    ap.add_argument("--counter-stats", metavar="CSV",
                    help="no GPU: per-dispatch means of the counters in a rocprofv3 --pmc counter_collection.csv "
                         "for --kernel, with the same --skip / --take selection")
    ap.add_argument("--kernel", help="with --trace-stats / --counter-stats: kernel name (e.g. k_attn_mfma)")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--take", type=int, default=0)
    ap.add_argument("--leg", help="with --trace-stats: record the result under this leg in --trace-out")
    ap.add_argument("--trace-out", metavar="JSON", help="with --trace-stats: merge the result into this file")
    ap.add_argument("--event-ms", type=float,
                    help="with --trace-out: the event average (ms) the profiled run itself printed for this leg, "
                         "recorded beside the trace average")
    ap.add_argument("--profile-command", default=PROFILE_COMMAND,
                    help="with --trace-out: the rocprofv3 command that wrote the trace, recorded beside the leg")
    ap.add_argument("--table", metavar="STEP_START",
                    help="with --trace-stats: print every kernel of the steps that hold the selected dispatches, "
                         "a step beginning at a dispatch of the kernel STEP_START (comma-separated names)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode workloads (for profiling their kernels alone)")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed prefill + decode workload")
    ap.add_argument("--no-serving", action="store_true", help="skip the iteration-level batching loop")
    ap.add_argument("--no-seq-state", action="store_true", help="skip sequence-state save / restore")
    ap.add_argument("--only", choices=["serving", "seq_state"],
                    help="run just this leg and print its result (for profiling its kernels alone)")
    ap.add_argument("--serving-iters", type=int, default=200, help="timed iterations of the serving loop")
    ap.add_argument("--decode-workload", choices=["cb_decode", "prefix_decode"], action="append",
                    help="restrict the decode runs to this workload (repeatable)")
    args = ap.parse_args()
    if args.counter_stats:
        print(json.dumps(counter_stats(args.counter_stats, args.kernel, args.skip, args.take)), flush=True)
        return
    if args.trace_stats and args.table:
        print(trace_table(args.trace_stats, args.kernel, args.skip, args.take, args.table), flush=True)
        return
    if args.trace_stats:
        rec = trace_stats(args.trace_stats, args.kernel, args.skip, args.take)
        if args.event_ms:
            rec["event_avg_ms_same_run"] = args.event_ms
            rec["trace_over_event"] = round(rec["avg_ns"] * 1e-6 / args.event_ms, 4)
        print(json.dumps(rec), flush=True)
        if args.trace_out:
            argv = [a for a in sys.argv[1:]]
            for opt in ("--profile-command",):
                if opt in argv:
                    k = argv.index(opt)
                    del argv[k:k + 2]
            # the trace's own location is the profiling run's output folder
            argv = [f"<out>/{os.path.basename(a)}" if a == args.trace_stats else a for a in argv]
            write_trace_record(args.trace_out, args.kernel, args.leg, rec, " ".join(argv), args.profile_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the attention path is not "
              f"sharded across GPUs; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from synthetic import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "serving":
        from synthetic.serving import qwen_serving
        print(json.dumps({"serving": bench_serving(qwen_serving(), dev, 300, args.serving_iters, args.layer_chunk)}),
              flush=True)
        return
    if args.only == "seq_state":
        print(json.dumps({"seq_state": bench_seq_state(dev)}), flush=True)
        return
    decode_names = args.decode_workload or ["cb_decode", "prefix_decode"]
    decode_wls = [(name, W.by_name(name)) for name in decode_names]
    if args.decode_only:
        dec = {name: bench_decode(w, dev, args.steps, args.warmup, args.layer_chunk) for name, w in decode_wls}
        print(json.dumps({"decode_only": {k: {"tokens_per_s": v["tokens_per_s"], "kv_read_gbs": v["kv_read_gbs"],
                                              "hbm_frac": v["hbm_frac"], "attend_avg_ms": v["attend_avg_ms"]}
                                          for k, v in dec.items()}}), flush=True)
        return
    wl = W.qwen_prefill()
    from ubatch_attention_paged_amd import KVATTN_KERNEL_MFMA
    pre = bench_prefill(wl, dev, args.steps, args.warmup, args.layer_chunk, KVATTN_KERNEL_MFMA)
    tok_s = pre["tokens"] * args.steps / pre["wall_s"]
    per_launch_flop = pre["flops_step"] / pre["attend_launches_per_step"]
    # the matrix-core kernel's own execution time, every timed launch
    kern_ms = pre["attend_avg_ms"]
    mfma_tf = per_launch_flop / (kern_ms * 1e-3) / 1e12
    log(f"[bench] prefill: {tok_s:,.0f} tok/s, {pre['ms_per_step']:.3f} ms/step, "
        f"k_attn_mfma {kern_ms:.4f} ms/launch x {pre['attend_launches_per_step']:.0f}, {mfma_tf:.1f} TFLOP/s")
    line = {
        "metric": "ubatch attention tokens/s + decode KV-read GB/s (% HBM peak), 1xMI355X",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-0.6B-shape single-sequence prefill: 3000-token prompt, caller calls "
                               "2048+952, split_simple n_ubatch=512 (6 ubatches), 28 layers, 16 q-heads / "
                               "8 kv-heads x 128, F16 cache kv_size=4096",
                   "n_layer": 28, "n_tokens": 3000, "n_batch": 2048, "n_ubatch": 512, "kv_size": 4096,
                   "layers_per_call": args.layer_chunk, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "k_attn_mfma",
                     "achieved": round(mfma_tf, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(mfma_tf / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": committed_traffic("k_attn_mfma", "attn_mfma.hip"),
                     "per_launch": f"{per_launch_flop / 1e9:.2f} GFLOP "
                                   f"(4*H*d per visible (query, cell) pair x 28 layers of one ubatch)",
                     "event_avg_ms": round(kern_ms, 4),
                     "event_kind": "k_attn_mfma execution, HIP events bound to every launch of a pass of "
                                   "the same steps run just before the timed ones (hipExtLaunchKernel start/stop)",
                     "ms_per_step_with_events": round(pre["ms_per_step_timed"], 4)},
    }
    # the committed kernel trace of the same command: its average over the
    # timed dispatches and the event average that profiled run printed
    # (boxes differ by a few per cent, so the pair, not this run, is the
    # trace-against-events comparison)
    trace_ms = committed_trace_ms("k_attn_mfma", "attn_mfma.hip", "prefill")
    if trace_ms is not None:
        rec = json.load(open(os.path.join(ROOT, "profiles", "k_attn_mfma_trace.json")))["legs"]["prefill"]
        line["roofline"]["profile"] = {"file": "profiles/k_attn_mfma_trace.json", "trace_avg_ms": round(trace_ms, 4),
                                       "event_avg_ms_same_run": rec.get("event_avg_ms_same_run"),
                                       "frac_trace": round(per_launch_flop / (trace_ms * 1e-3) / 1e12
                                                           / MFMA_F16_PEAK_TFLOPS, 4)}
    line["hbm_copy_gbs"] = hbm_copy_gbs(dev)
    log(f"[bench] device-to-device copy: {line['hbm_copy_gbs']:.0f} GB/s")
    line["ceilings"] = ceilings(dev)
    log(f"[bench] ceilings: {line['ceilings']}")
    if not args.no_per_layer:
        # a forward pass calls attend once per layer (layer l+1's q depends on
        # layer l): the same prompt with one store and one attend per layer
        ps = max(2, args.steps // 2)
        pl = bench_prefill(wl, dev, ps, 1, 1)
        line["per_layer_calls"] = {"prefill": {
            "tokens_per_s": round(pl["tokens"] * ps / pl["wall_s"], 1), "ms_per_step": round(pl["ms_per_step"], 4),
            "attend_launches_per_step": round(pl["attend_launches_per_step"], 1),
            "attend_us_per_launch": round(1e3 * pl["attend_avg_ms"], 2),
            "attend_ms_per_step": round(pl["attend_ms_per_step"], 4),
            "tflops_attend": round(pre["flops_step"] / (pl["attend_ms_per_step"] * 1e-3) / 1e12, 1)}}
        log(f"[bench] prefill, one call per layer: {line['per_layer_calls']['prefill']}")
    if not args.no_decode:
        dec = {}
        for name, w in decode_wls:
            r = bench_decode(w, dev, args.steps, args.warmup, args.layer_chunk)
            log(f"[bench] {name}: {r['tokens_per_s']:,.0f} tok/s, attend {r['attend_avg_ms']:.3f} ms, "
                f"{r['kv_read_gbs']:.0f} GB/s ({100 * r['hbm_frac']:.1f}% of HBM)")
            dec[name] = {"workload": w.note, "tokens_per_s": round(r["tokens_per_s"], 1),
                         "ms_per_step": round(r["ms_per_step"], 4),
                         "kv_read_gbs": round(r["kv_read_gbs"], 1), "hbm_frac": round(r["hbm_frac"], 4),
                         "kv_bytes_per_step": round(r["kv_bytes_step"]), "qo_bytes_per_step": round(r["qo_bytes_step"]),
                         "kv_qo_gbs": round(r["kv_qo_gbs"], 1),
                         "attend_avg_ms": round(r["attend_avg_ms"], 4),
                         "unique_cells_per_step": r["unique_cells"], "plan": r["plan"]}
            if name == "cb_decode" and not args.no_per_layer:
                rp = bench_decode(w, dev, args.steps, args.warmup, 1)
                line.setdefault("per_layer_calls", {})["cb_decode"] = {
                    "tokens_per_s": round(rp["tokens_per_s"], 1), "ms_per_step": round(rp["ms_per_step"], 4),
                    "attend_launches_per_step": round(rp["attend_launches_per_step"], 1),
                    "attend_us_per_launch": round(1e3 * rp["attend_avg_ms"], 2),
                    "kv_read_gbs": round(rp["kv_read_gbs"], 1), "hbm_frac": round(rp["hbm_frac"], 4)}
                log(f"[bench] cb_decode, one call per layer: {line['per_layer_calls']['cb_decode']}")
            if name == "cb_decode":
                # the vector-ALU kernel's HBM bytes per launch from the committed
                # FETCH_SIZE / WRITE_SIZE summary of this workload (None if stale)
                dec[name]["traffic_k_attn_valu"] = committed_traffic("k_attn_valu", "attn_valu.hip")
        line["decode"] = dec
    if not args.no_mixed:
        m = bench_mixed(W.mixed(), dev, max(2, args.steps // 2), 1, args.layer_chunk)
        log(f"[bench] mixed: {m['tokens_per_s']:,.0f} tok/s; " + "; ".join(
            f"{k}: {v}" for k, v in m.items() if k.endswith("_ubatches")))
        line["mixed"] = m
    if not args.no_serving:
        from synthetic.serving import qwen_serving
        sv = bench_serving(qwen_serving(), dev, 300, args.serving_iters, args.layer_chunk)
        log(f"[bench] serving: {sv['generated_tokens_per_s']:,.0f} generated tok/s, "
            f"{sv['positions_per_s']:,.0f} positions/s, {sv['ms_per_iteration']:.3f} ms/iteration, "
            f"scheduler {sv['sched_step_us']['mean']:.1f} us/iteration")
        line["serving"] = sv
        # the same stream over a cache too small for it: preemption by
        # recomputation against preemption by swapping ("Where it breaks")
        pr = {}
        for mode in ("recompute", "swap"):
            r = bench_serving(qwen_serving(kv_size=40960, preempt=mode), dev, 300, args.serving_iters,
                              args.layer_chunk, swap_bytes=2 << 30)
            pr[mode] = {k: r[k] for k in ("generated_tokens_per_s", "positions_per_s", "ms_per_iteration",
                                          "preemptions", "swapped_out", "positions_per_generated",
                                          "mean_running", "sched_step_us")}
        log(f"[bench] serving under cache pressure (40960 cells): recompute "
            f"{pr['recompute']['generated_tokens_per_s']:,.0f} tok/s, swap {pr['swap']['generated_tokens_per_s']:,.0f} tok/s")
        line["serving_pressure"] = dict(workload="qwen_serving over a 40960-cell cache, 2 GiB swap arena", **pr)
    if not args.no_seq_state:
        ss = bench_seq_state(dev)
        log(f"[bench] seq state: save {ss['save_ms']:.3f} ms ({ss['save_gbs']:.0f} GB/s), "
            f"load {ss['load_ms_wall']:.3f} ms wall")
        line["seq_state"] = ss
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(wl)
        log(f"[bench] oracle: " + ", ".join(f"{k} {v['value']:.1f} tok/s"
                                            for k, v in line["cpu_baseline"]["configs"].items()))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
