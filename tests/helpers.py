"""Shared drivers for the parity tests: run a synthetic workload through the
oracle (CPU, fp64) and through the HIP library (GPU), same seeded inputs."""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import OracleEngine
from synthetic import workloads as W

ATOL, RTOL = 2e-3, 5e-3        # |g - r| <= ATOL + RTOL * |r| elementwise, and max |g - r| <= ATOL
# Internal bounds, tighter than the tolerance, to catch mistakes that stay
# inside it.  The fp32 vector-ALU path differs from the fp64 oracle only by
# fp32 rounding.  The matrix-core path rounds the scaled q and the softmax
# weights to F16; the first-order effect on an output is bounded by the
# weights' relative error times the spread of the visible values.
VALU_BOUND = 2e-5
MFMA_BOUND = 1.6e-3


def batch_tensors(wl, b, layers, with_q):
    kinds = [W.KIND_K, W.KIND_V] + ([W.KIND_Q] if with_q else [])
    jobs = [(l, k) for l in layers for k in kinds]
    with ThreadPoolExecutor(8) as ex:
        arrs = list(ex.map(lambda lk: wl.tensor(b, lk[0], lk[1]), jobs))
    out = {}
    for (l, k), a in zip(jobs, arrs):
        out[(l, k)] = a
    return out


def oracle_run(wl, layers, measured_only=True, keep_masks=False, n_ubatch=None):
    """Returns (engine, results) where results[(b, l)] = fp64 outputs in batch
    order for measured batches; masks[(b, u)] when keep_masks."""
    eng = OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                       wl.n_seq_max, wl.n_batch, wl.n_ubatch if n_ubatch is None else n_ubatch, wl.causal,
                       cell_order=wl.cell_order, layers=layers, split_mode=wl.split_mode, swa=wl.swa)
    res, masks, ubmeta = {}, {}, {}
    for b, bt in enumerate(wl.batches):
        st, ubs, _ = eng.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0
        t = batch_tensors(wl, b, layers, bt.measured)
        outs = {l: np.zeros((bt.n_tokens, wl.n_head * wl.head_dim)) for l in layers}
        for u, ub in enumerate(ubs):
            eng.commit(ub, build_mask=bt.measured or keep_masks)
            if keep_masks:
                masks[(b, u)] = ub.mask.copy()
            for l in layers:
                eng.store(ub, l, t[(l, W.KIND_K)][ub.src], t[(l, W.KIND_V)][ub.src])
                if bt.measured:
                    outs[l][ub.src] = eng.attend(ub, l, t[(l, W.KIND_Q)][ub.src])
            ubmeta[(b, u)] = ub
        if bt.measured:
            for l in layers:
                res[(b, l)] = outs[l]
    return eng, res, masks, ubmeta


def make_ctx(wl, device="cuda:0", n_ubatch=None, attend_layers=0):
    from ubatch_attention_paged_amd import Context
    # every layer of the workload gets a cache; tests may run a subset
    return Context(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream, wl.n_seq_max,
                   wl.n_batch, wl.n_ubatch if n_ubatch is None else n_ubatch, wl.causal,
                   cell_order=wl.cell_order, device=device, attend_layers=attend_layers,
                   split_mode=wl.split_mode, swa_window=wl.swa)


def gpu_run(wl, layers, layer_chunk=None, only_outputs=False, on_ubatch=None, ctx=None, n_ubatch=None,
            keep_layers=None):
    """Returns (ctx, results) with results[(b, l)] float64 numpy in batch
    order (only for keep_layers when given).  on_ubatch(ctx, b, ub) runs
    after each ubatch is stored."""
    import torch
    from ubatch_attention_paged_amd.harness import ubatch_rows
    dev = torch.device("cuda:0")
    chunk = len(layers) if layer_chunk is None else layer_chunk
    ctx = ctx or make_ctx(wl, n_ubatch=n_ubatch, attend_layers=chunk)
    res = {}
    keep = set(layers if keep_layers is None else keep_layers)
    assert layers == list(range(layers[0], layers[0] + len(layers)))
    HD = wl.n_head * wl.head_dim
    for b, bt in enumerate(wl.batches):
        t = batch_tensors(wl, b, layers, bt.measured)
        K = [torch.from_numpy(t[(l, W.KIND_K)]).to(dev) for l in layers]
        V = [torch.from_numpy(t[(l, W.KIND_V)]).to(dev) for l in layers]
        Q = [torch.from_numpy(t[(l, W.KIND_Q)]).to(dev) for l in layers] if bt.measured else None
        st, ubs, _ = ctx.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0
        outs = [torch.zeros((bt.n_tokens, HD), dtype=torch.float32, device=dev) for _ in layers]
        for ub in ubs:
            kr = [ubatch_rows(ub, x) for x in K]
            vr = [ubatch_rows(ub, x) for x in V]
            qr = [ubatch_rows(ub, x) for x in Q] if Q is not None else None
            nrow = ub.n_outputs if only_outputs else ub.n_tokens
            uo = [torch.full((nrow, HD), float("nan"), device=dev) for _ in layers]
            for a in range(0, len(layers), chunk):
                idx = list(range(a, min(len(layers), a + chunk)))
                ctx.store(ub, layers[idx[0]], [kr[i] for i in idx], [vr[i] for i in idx])
                if on_ubatch is not None and a == 0:
                    on_ubatch(ctx, b, ub)
                if Q is not None:
                    ctx.attend(ub, layers[idx[0]], [qr[i] for i in idx], [uo[i] for i in idx], only_outputs)
            if Q is not None:
                rows = ub.src if not only_outputs else ub.src[ub.output.astype(bool)]
                ridx = torch.as_tensor(rows, device=dev, dtype=torch.long)
                for i in range(len(layers)):
                    outs[i].index_copy_(0, ridx, uo[i])
        if bt.measured:
            torch.cuda.synchronize()
            for i, l in enumerate(layers):
                if l in keep:
                    res[(b, l)] = outs[i].double().cpu().numpy()
        del K, V, Q, outs
    torch.cuda.synchronize()
    return ctx, res


def assert_parity(got, ref, rows=None, tag="", strict_abs=True):
    """Elementwise |g - r| <= ATOL + RTOL |r| and, with strict_abs, also
    max |g - r| <= ATOL; returns (max abs, max rel over |r| >= 1e-2)."""
    g, r = got, ref
    if rows is not None:
        g, r = g[rows], r[rows]
    assert np.isfinite(g).all(), f"{tag}: non-finite output"
    err = np.abs(g - r)
    bad = err > ATOL + RTOL * np.abs(r)
    big = np.abs(r) >= 1e-2
    rel = (err[big] / np.abs(r[big])).max() if big.any() else 0.0
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{tag}: {bad.sum()} elements out of tolerance; first at {tuple(i)}: "
                             f"got {g[tuple(i)]!r} ref {r[tuple(i)]!r}; max abs {err.max():.3e}")
    assert not strict_abs or err.max() <= ATOL, f"{tag}: max abs error {err.max():.3e} above {ATOL}"
    return float(err.max()), float(rel)
