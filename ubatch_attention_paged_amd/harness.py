"""Caller-side plumbing around the C ABI: one decode call, the way a model
forward pass would issue it.

``decode`` mirrors the loop of "Batch、Ubatch 与解码主循环", Part F: split the
batch (reserving cells for every ubatch), then for each ubatch write its K/V
rows and run attention, layer by layer or over a layer range per call.  The
arithmetic all happens in the library; this only slices torch tensors and
passes addresses.
"""

from __future__ import annotations

import numpy as np

from .kvattn import KvattnError, KVATTN_NO_SLOT


def ubatch_rows(ub, t):
    """Rows of a batch-order tensor that belong to ubatch ``ub``, in ubatch
    order: a view when they are contiguous, else a gathered copy."""
    import torch
    n = ub.n_tokens
    src = ub.src
    if n == 0:
        return t[:0]
    if src[-1] - src[0] == n - 1 and np.all(np.diff(src) == 1):
        return t[int(src[0]):int(src[0]) + n]
    return t.index_select(0, torch.as_tensor(src, device=t.device, dtype=torch.long)).contiguous()


def decode(ctx, n_tokens, pos, seq_ids, output, K, V, Q=None, layers=None, layer_chunk=None,
           only_outputs=False, collect=True):
    """Run one decode call.

    K, V  per-layer fp32 device tensors [n_tokens][E] in batch order
    Q     per-layer fp32 device tensors [n_tokens][n_head*head_dim] or None
          (store only: e.g. filling a context)
    layers       layer indices (default all); K/V/Q are indexed like it
    layer_chunk  layers per store/attend call (default: all in one call)

    Returns (status, ubatches, outs): outs[i] is the attention output of
    layers[i] in batch order (rows of unflagged slots stay zero with
    only_outputs), or None when Q is None or collect is False.
    """
    import torch
    layers = list(range(ctx.n_layer)) if layers is None else list(layers)
    chunk = len(layers) if layer_chunk is None else layer_chunk
    st, ubs, _ = ctx.split(n_tokens, pos, seq_ids, output)
    if st == KVATTN_NO_SLOT:
        return st, [], None
    HD = ctx.n_head * ctx.head_dim
    outs = None
    if Q is not None and collect:
        outs = [torch.zeros((n_tokens, HD), dtype=torch.float32, device=K[0].device) for _ in layers]
    for ub in ubs:
        krows = [ubatch_rows(ub, k) for k in K]
        vrows = [ubatch_rows(ub, v) for v in V]
        qrows = [ubatch_rows(ub, q) for q in Q] if Q is not None else None
        nrow = ub.n_outputs if only_outputs else ub.n_tokens
        ubo = [torch.empty((nrow, HD), dtype=torch.float32, device=K[0].device) for _ in layers] if Q is not None else None
        for a in range(0, len(layers), chunk):
            idx = list(range(a, min(len(layers), a + chunk)))
            il0 = layers[idx[0]]
            if layers[idx[-1]] - il0 != len(idx) - 1:
                raise ValueError("layer chunks must be contiguous")
            ctx.store(ub, il0, [krows[i] for i in idx], [vrows[i] for i in idx])
            if Q is not None:
                ctx.attend(ub, il0, [qrows[i] for i in idx], [ubo[i] for i in idx], only_outputs)
        if outs is not None:
            rows = ub.src if not only_outputs else ub.src[ub.output.astype(bool)]
            ridx = torch.as_tensor(rows, device=K[0].device, dtype=torch.long)
            for i in range(len(layers)):
                outs[i].index_copy_(0, ridx, ubo[i])
    return st, ubs, outs
