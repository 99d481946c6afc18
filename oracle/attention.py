"""Masked-softmax grouped-query attention in fp64.

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ("llama.cpp and the ubatch", "Where the memory actually sits": a query is compared
with the key of every earlier token and the values are mixed by those
weights; "llama.cpp and the ubatch", "The mask is doing the work": masked keys become -inf before the
softmax and contribute nothing; "llama.cpp and the ubatch", "The output projection": each head's
output is a weighted sum of value vectors):

    O[i, h] = sum_j softmax_j(scale * q[i, h] . K[j, g] + M[i, j]) V[j, g]

with g = h // (n_head / n_head_kv).  Readings (the pages give neither): the
query heads that share a KV head are contiguous ("Iteration-Level Batching", "The budget that actually
binds" gives only the ratio), and scale = 1 / sqrt(head_dim).  A row with no
visible key produces zeros.
"""

from __future__ import annotations

import math

import numpy as np


def masked_attention(q, k_cache, v_cache, streams, mask, n_head, n_head_kv, scale=None):
    """Dense definition over the first n_kv cells of each query's stream.

    q        fp32 [T][n_head * head_dim] (exact in fp64)
    k_cache  F16 [n_stream][>= n_kv][n_head_kv * head_dim]  (one layer)
    v_cache  same shape as k_cache
    streams  stream of each query
    mask     F16 [T][n_kv], 0 (visible) or -inf
    returns  fp64 [T][n_head * head_dim]
    """
    q = np.asarray(q, dtype=np.float64)
    T = q.shape[0]
    d = q.shape[1] // n_head
    group = n_head // n_head_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m = np.asarray(mask, dtype=np.float64)
    nkv = m.shape[1]
    streams = np.asarray(streams)
    out = np.zeros((T, n_head * d), dtype=np.float64)
    for s in np.unique(streams):
        rows = np.nonzero(streams == s)[0]
        K = np.asarray(k_cache[s, :nkv], dtype=np.float64)
        V = np.asarray(v_cache[s, :nkv], dtype=np.float64)
        ms = m[rows]
        any_visible = np.isfinite(ms).any(axis=1)
        for h in range(n_head):
            g = h // group
            scores = scale * (q[rows, h * d:(h + 1) * d] @ K[:, g * d:(g + 1) * d].T) + ms
            top = np.where(any_visible, scores.max(axis=1), 0.0)
            p = np.exp(scores - top[:, None])          # exp(-inf) = 0 for masked cells
            tot = p.sum(axis=1)
            o = (p @ V[:, g * d:(g + 1) * d]) / np.where(tot > 0, tot, 1.0)[:, None]
            out[rows, h * d:(h + 1) * d] = np.where(any_visible[:, None], o, 0.0)
    return out


def brute_force_attention(queries, history, n_head, n_head_kv, head_dim, causal=True, scale=None, swa=0):
    """Per-sequence attention by explicit loops over the token history.

    Independent of cells, placement, n_kv and the mask: a query (pos, first
    seq id s, q) sees every stored token whose sequence set contains s and,
    when causal, whose position is not later than its own; with a sliding
    window of swa > 0 positions, only tokens fewer than swa positions back.

    queries  list of (pos, seq0, q[n_head*head_dim])
    history  list of (pos, seq_set, k_f16[n_head_kv*head_dim], v_f16[...])
    returns  list of fp64 rows
    """
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    group = n_head // n_head_kv
    rows = []
    for (qp, s0, q) in queries:
        seen = [(float_row(k), float_row(v)) for (p, ss, k, v) in history
                if s0 in ss and (not causal or p <= qp) and (swa <= 0 or qp - p < swa)]
        o = [0.0] * (n_head * head_dim)
        for h in range(n_head):
            g = h // group
            scores = []
            for (k, _) in seen:
                acc = 0.0
                for e in range(head_dim):
                    acc += float(q[h * head_dim + e]) * k[g * head_dim + e]
                scores.append(acc * scale)
            if not scores:
                continue
            top = max(scores)
            w = [math.exp(x - top) for x in scores]
            tot = sum(w)
            for e in range(head_dim):
                acc = 0.0
                for wj, (_, v) in zip(w, seen):
                    acc += wj * v[g * head_dim + e]
                o[h * head_dim + e] = acc / tot
        rows.append(o)
    return rows


def float_row(x):
    return [float(v) for v in np.asarray(x, dtype=np.float64)]
