"""Shared drivers for the parity tests: run a synthetic workload through the
oracle (CPU, fp64) and through the HIP library (GPU), same seeded inputs."""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import OracleEngine
from oracle.attention import masked_attention
from synthetic import workloads as W

ATOL, RTOL = 2e-3, 5e-3        # |g - r| <= ATOL + RTOL * |r| elementwise, and max |g - r| <= ATOL
# Internal bounds, tighter than the tolerance, to catch mistakes that stay
# inside it.  The fp32 vector-ALU path differs from the fp64 oracle only by
# fp32 rounding.  The matrix-core path rounds the scaled q and the softmax
# weights to F16; the first-order effect on an output is bounded by the
# weights' relative error times the spread of the visible values.
VALU_BOUND = 2e-5
MFMA_BOUND = 1.6e-3     # flat bound, kept only where the per-element model below is not computed

# Per-element error model of the matrix-core path.  That path holds the
# query as fp32 q * fp32(kq_scale * log2 e) rounded to F16 (mfma_query), and
# rounds every softmax weight to F16 before the PV product, with the row sum
# taken over the same F16 weights; K and V are F16 on both sides and the rest
# is fp32.  So its output is the oracle's attention evaluated at that F16
# query (alt), plus the weight roundings: a relative error eta_j on weight j
# moves the output by sum_j w_j eta_j (v_j[d] - o[d]) to first order.  With
# independent eta_j of RMS at most ROUND_RMS (an error uniform in [-u, u],
# u = 2^-11; values spread over their binade give ~0.73 of it), that has
# standard deviation ROUND_RMS * sqrt(sum_j w_j^2 (v_j[d] - o[d])^2); weights
# below the F16 normal range (2^-14 of a maximum weight of at least 1) carry
# an absolute error of at most 2^-25 instead.  An output must lie within
# SIGMA_Z standard deviations plus SIGMA_FLOOR (fp32 arithmetic) of alt --
# or of the oracle itself, for rows the fp32 vector-ALU path computes.  A
# dropped cell moves its row by ~w_j |a_j|, for n visible cells
# ~1 / (ROUND_RMS sqrt(n)) standard deviations: 39 at n = 4096.
F16_U = 2.0 ** -11
ROUND_RMS = F16_U / 3.0 ** 0.5
SUB_RMS = 2.0 ** -25 / 3.0 ** 0.5
SIGMA_Z = 6.0
SIGMA_FLOOR = 2e-5


def mfma_query(q, d, kq_scale=None):
    """q as the matrix-core path holds it, in log2 units: fp32 q times
    fp32(kq_scale) * fp32(log2 e), rounded to F16 (nearest even); kq_scale
    defaults to 1 / sqrt(d) in fp32.  Attention over it uses scale ln 2."""
    sc = np.float32(kq_scale) if kq_scale else np.float32(1.0) / np.sqrt(np.float32(d))
    sl = np.float32(sc * np.float32(1.4426950408889634))
    return (np.asarray(q, dtype=np.float32) * sl).astype(np.float16).astype(np.float64)


def weight_sigma(q, k_cache, v_cache, streams, mask, n_head, n_head_kv, scale):
    """Standard deviation of each output element from the F16 weight
    roundings, under the model above; same arguments and layout as the
    oracle's dense masked attention.  Rows without a visible cell get 0."""
    q = np.asarray(q, dtype=np.float64)
    T = q.shape[0]
    d = q.shape[1] // n_head
    grp = n_head // n_head_kv
    m = np.asarray(mask, dtype=np.float64)
    nkv = m.shape[1]
    streams = np.asarray(streams)
    var = np.zeros((T, n_head * d))
    for s in np.unique(streams):
        rs = np.nonzero(streams == s)[0]
        Kc = np.asarray(k_cache[s, :nkv], dtype=np.float64)
        Vc = np.asarray(v_cache[s, :nkv], dtype=np.float64)
        ms = m[rs]
        vis = np.isfinite(ms).any(axis=1)
        for h in range(n_head):
            g = h // grp
            Vh = Vc[:, g * d:(g + 1) * d]
            sc = scale * (q[rs, h * d:(h + 1) * d] @ Kc[:, g * d:(g + 1) * d].T) + ms
            top = np.where(vis, sc.max(axis=1), 0.0)
            p = np.exp(sc - top[:, None])                  # 1 at each row's largest weight
            w = p / np.where(vis, p.sum(axis=1), 1.0)[:, None]
            o = w @ Vh
            def spread(c):                                  # sum_j c_j (v_j - o)^2, per row and d
                return c @ (Vh * Vh) - 2.0 * o * (c @ Vh) + o * o * c.sum(axis=1)[:, None]
            sub = ((p > 0) & (p < 2.0 ** -14)).astype(np.float64)
            var[rs, h * d:(h + 1) * d] = (ROUND_RMS ** 2 * np.maximum(spread(w * w), 0.0) +
                                          SUB_RMS ** 2 * np.maximum(spread(sub), 0.0))
    return np.sqrt(var)


def model_for(eng, ub, layer, q_rows):
    """(alt, sigma) of the rounding model for one oracle attend call."""
    qt = mfma_query(q_rows, eng.head_dim, eng.kq_scale)
    args = (eng.K[layer], eng.V[layer], ub.streams, ub.mask, eng.n_head, eng.n_head_kv, math.log(2.0))
    return masked_attention(qt, *args), weight_sigma(qt, *args)


class Results(dict):
    """results[(b, l)] -> fp64 outputs; when computed, .alt[(b, l)] -> the
    same attention at the matrix-core path's F16 query and .sigma[(b, l)] ->
    the weight-rounding model's standard deviations."""

    def __init__(self):
        super().__init__()
        self.alt = {}
        self.sigma = {}

    def model(self, key):
        """keyword arguments of assert_parity for the rounding model (none
        when it was not computed)"""
        return {"alt": self.alt[key], "sigma": self.sigma[key]} if key in self.sigma else {}


def batch_tensors(wl, b, layers, with_q):
    kinds = [W.KIND_K, W.KIND_V] + ([W.KIND_Q] if with_q else [])
    jobs = [(l, k) for l in layers for k in kinds]
    with ThreadPoolExecutor(8) as ex:
        arrs = list(ex.map(lambda lk: wl.tensor(b, lk[0], lk[1]), jobs))
    out = {}
    for (l, k), a in zip(jobs, arrs):
        out[(l, k)] = a
    return out


def oracle_run(wl, layers, measured_only=True, keep_masks=False, n_ubatch=None, sigma=True):
    """Returns (engine, results, masks, ubatches) where results[(b, l)] =
    fp64 outputs in batch order for measured batches (and, with sigma, the
    rounding model's results.alt and results.sigma);
    masks[(b, u)] when keep_masks."""
    eng = OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, wl.n_stream,
                       wl.n_seq_max, wl.n_batch, wl.n_ubatch if n_ubatch is None else n_ubatch, wl.causal,
                       cell_order=wl.cell_order, layers=layers, split_mode=wl.split_mode, swa=wl.swa)
    res, masks, ubmeta = Results(), {}, {}
    for b, bt in enumerate(wl.batches):
        st, ubs, _ = eng.split(bt.n_tokens, bt.pos, bt.seq_ids, bt.output)
        assert st == 0
        t = batch_tensors(wl, b, layers, bt.measured)
        outs = {l: np.zeros((bt.n_tokens, wl.n_head * wl.head_dim)) for l in layers}
        alts = {l: np.zeros((bt.n_tokens, wl.n_head * wl.head_dim)) for l in layers} if sigma else None
        sigs = {l: np.zeros((bt.n_tokens, wl.n_head * wl.head_dim)) for l in layers} if sigma else None
        for u, ub in enumerate(ubs):
            eng.commit(ub, build_mask=bt.measured or keep_masks)
            if keep_masks:
                masks[(b, u)] = ub.mask.copy()
            for l in layers:
                eng.store(ub, l, t[(l, W.KIND_K)][ub.src], t[(l, W.KIND_V)][ub.src])
                if bt.measured:
                    qr = t[(l, W.KIND_Q)][ub.src]
                    outs[l][ub.src] = eng.attend(ub, l, qr)
                    if sigma:
                        alts[l][ub.src], sigs[l][ub.src] = model_for(eng, ub, l, qr)
            ubmeta[(b, u)] = ub
        if bt.measured:
            for l in layers:
                res[(b, l)] = outs[l]
                if sigma:
                    res.alt[(b, l)] = alts[l]
                    res.sigma[(b, l)] = sigs[l]
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


def assert_parity(got, ref, rows=None, tag="", strict_abs=True, sigma=None, alt=None):
    """Elementwise |g - r| <= ATOL + RTOL |r| and, with strict_abs, also
    max |g - r| <= ATOL; with the rounding model (alt, sigma) also
    min(|g - r|, |g - alt|) <= SIGMA_Z sigma + SIGMA_FLOOR elementwise.
    Returns (max abs, max rel over |r| >= 1e-2)."""
    g, r = got, ref
    if rows is not None:
        g, r = g[rows], r[rows]
        sigma = None if sigma is None else sigma[rows]
        alt = None if alt is None else alt[rows]
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
    zmax = 0.0
    if sigma is not None:
        em = np.minimum(err, np.abs(g - alt))
        over = em > SIGMA_Z * sigma + SIGMA_FLOOR
        if over.any():
            i = tuple(np.argwhere(over)[0])
            raise AssertionError(f"{tag}: {over.sum()} elements beyond the rounding model; first at {i}: "
                                 f"got {g[i]!r} ref {r[i]!r} F16-query ref {alt[i]!r} sigma {sigma[i]:.3e}")
        zmax = float(((em - SIGMA_FLOOR).clip(min=0) / np.maximum(sigma, 1e-30)).max())
    log = os.environ.get("KVATTN_PARITY_LOG")
    if log:     # per-comparison worst errors, for setting the internal bounds
        with open(log, "a") as f:
            f.write(f"{os.environ.get('PYTEST_CURRENT_TEST', '-').split(' ')[0]}\t{tag}\t{err.max():.4e}\t{rel:.4e}"
                    f"\t{zmax:.3f}\n")
    return float(err.max()), float(rel)
