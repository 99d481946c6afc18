"""The KV cache as the pages describe it: cells, placement, n_kv, the KQ mask.

Test infrastructure only (see ``oracle/__init__.py``).

Layout ("What does llama.cpp's KV cache actually look like in memory?", "28 layers, 56 tensors", "The tensor's three dimensions"): every
layer owns one K and one V tensor of shape [n_stream][kv_size][n_head_kv *
head_dim] in F16; a cell is a row index shared by all layers; stream s is the
slab at offset s * kv_size * row_bytes ("What does llama.cpp's KV cache actually look like in memory?", "Unified versus non-unified").
Each cell records whether it is empty, its position and the set of sequences
that may read it ("llama.cpp and the ubatch", "The mask is doing the work").
"""

from __future__ import annotations

import numpy as np

from .batching import SplitError

F16_BYTES = 2                 # "What does llama.cpp's KV cache actually look like in memory?", "One row, one token's keys": two bytes per number
N_PAD_FLOOR = 256             # "llama.cpp and the ubatch", "Prefill and decode are not the same shape"
MASK_VISIBLE = np.float16(0.0)
MASK_HIDDEN = np.float16(-np.inf)


def f16_round(x) -> np.ndarray:
    """fp32 -> IEEE binary16 with round-to-nearest-even (numpy's cast).
    The pages store K/V as 2-byte F16 ("What does llama.cpp's KV cache actually look like in memory?", "One row, one token's keys");
    the rounding mode is a reading."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16)


def row_bytes(n_head_kv: int, head_dim: int) -> int:
    """Bytes of one cell's K (or V) row in one layer: n_head_kv * head_dim F16
    numbers ("What does llama.cpp's KV cache actually look like in memory?", "One row, one token's keys": 8 x 128 -> 2048 bytes)."""
    return n_head_kv * head_dim * F16_BYTES


def cache_bytes(n_layer, n_head_kv, head_dim, kv_size, n_stream=1) -> int:
    """Total K+V allocation: every cell of every stream, in K and V, in every
    layer ("What does llama.cpp's KV cache actually look like in memory?", "One row, one token's keys" and "The measured allocation":
    4096 cells of Qwen3-0.6B -> 448 MiB)."""
    return 2 * n_layer * n_stream * kv_size * row_bytes(n_head_kv, head_dim)


def k_elem_offset(cell, head, elem, n_head_kv, head_dim, stream=0, kv_size=0) -> int:
    """Byte offset of one F16 element inside a layer's K tensor, from the
    strides nb = (2, row_bytes, kv_size * row_bytes) ("What does llama.cpp's KV cache actually look like in memory?", "The tensor's three
    dimensions": cell 37, head 3, element 10 -> 76,564 bytes)."""
    nb1 = row_bytes(n_head_kv, head_dim)
    nb2 = kv_size * nb1
    return stream * nb2 + cell * nb1 + (head * head_dim + elem) * F16_BYTES


class CellTable:
    """Per-stream cell metadata plus a free list.

    ``pos[s, j]``        position held by cell j of stream s, -1 when empty;
    ``member[s, j, q]``  True when sequence q may read that cell.

    Placement is not described on the pages beyond two facts: every ubatch
    of a batch gets its cells reserved before any of them runs ("Batch、Ubatch 与解码主循环", Part C,
    strategy choice), and a token takes one cell however many sequences it
    belongs to ("Batch、Ubatch 与解码主循环", Part E).  Reading: each
    stream hands out its free cells lowest rank first, where rank is the
    cell's index in ``order[s]`` (ascending cell index when no order is
    given); a freed cell returns with its original rank.
    """

    def __init__(self, kv_size: int, n_stream: int = 1, n_seq_max: int = 1, order=None):
        self.kv_size = int(kv_size)
        self.n_stream = int(n_stream)
        self.n_seq_max = int(n_seq_max)
        self.pos = np.full((n_stream, kv_size), -1, dtype=np.int64)
        self.member = np.zeros((n_stream, kv_size, n_seq_max), dtype=bool)
        if order is None:
            order = np.tile(np.arange(kv_size), (n_stream, 1))
        order = np.asarray(order).reshape(n_stream, kv_size)
        self.rank = np.empty((n_stream, kv_size), dtype=np.int64)
        for s in range(n_stream):
            if not np.array_equal(np.sort(order[s]), np.arange(kv_size)):
                raise SplitError("cell order is not a permutation")
            self.rank[s, order[s]] = np.arange(kv_size)
        # cells handed out by reserve() but not yet committed
        self.reserved = np.zeros((n_stream, kv_size), dtype=bool)

    # -- placement -------------------------------------------------------
    def free_cells_by_rank(self, s) -> np.ndarray:
        free = np.nonzero((self.pos[s] < 0) & ~self.reserved[s])[0]
        return free[np.argsort(self.rank[s, free], kind="stable")]

    def reserve(self, streams: list):
        """All-or-nothing placement for a whole batch ("Batch、Ubatch 与解码主循环", Part C: prepare
        reserves slots for every ubatch before any is processed; "Batch、Ubatch 与解码主循环", Part F:
        a full cache makes llama_decode return 1).  ``streams`` lists the
        stream of every slot in ubatch order.  Returns the cell of each slot,
        or None (nothing reserved) when a stream runs out."""
        need = {}
        for s in streams:
            need[s] = need.get(s, 0) + 1
        pools = {}
        for s, n in need.items():
            pool = self.free_cells_by_rank(s)
            if len(pool) < n:
                return None
            pools[s] = pool
        cells, taken = [], {s: 0 for s in need}
        for s in streams:
            j = int(pools[s][taken[s]])
            taken[s] += 1
            cells.append(j)
            self.reserved[s, j] = True
        return cells

    def release(self, streams, cells):
        for s, j in zip(streams, cells):
            self.reserved[s, j] = False

    def commit(self, streams, cells, pos, seq_sets):
        """A ubatch's cells become occupied: position and sequence set.  Once
        written an entry is final ("llama.cpp and the ubatch", "Where the memory actually sits")."""
        for s, j, p, ss in zip(streams, cells, pos, seq_sets):
            self.reserved[s, j] = False
            self.pos[s, j] = int(p)
            self.member[s, j, :] = False
            self.member[s, j, list(ss)] = True

    def seq_rm(self, seq_id: int, p0: int, p1: int):
        """Drop sequence ``seq_id`` (every sequence when negative) from cells
        whose position lies in [p0, p1) (open ends when negative); a cell
        left with no sequence becomes empty."""
        lo = 0 if p0 < 0 else p0
        hit = (self.pos >= 0) & (self.pos >= lo)
        if p1 >= 0:
            hit &= self.pos < p1
        if seq_id < 0:
            self.member[hit] = False
        else:
            self.member[hit, seq_id] = False
        self.pos[~self.member.any(axis=2)] = -1

    def seq_pos_max(self, seq_id: int) -> int:
        sel = (self.pos >= 0) & self.member[:, :, seq_id]
        return int(self.pos[sel].max()) if sel.any() else -1

    # -- n_kv ----------------------------------------------------------
    def used_max_p1(self, s) -> int:
        occ = np.nonzero(self.pos[s] >= 0)[0]
        return int(occ.max()) + 1 if occ.size else 0

    def n_kv(self) -> int:
        """get_n_kv ("llama.cpp and the ubatch", "Prefill and decode are not the same shape"): per
        stream, the occupied extent padded up to a multiple of 256 (and never
        below 256), capped at the stream size; the reported value is the
        largest over streams (reading of the elided running ``result``)."""
        result = 0
        for s in range(self.n_stream):
            u = self.used_max_p1(s)
            padded = -(-u // N_PAD_FLOOR) * N_PAD_FLOOR
            result = max(min(self.kv_size, max(N_PAD_FLOOR, padded)), result)
        return result

    # -- the KQ mask -----------------------------------------------------
    def visible_row(self, s, q_pos, q_seq0, nkv, causal=True, swa=0) -> np.ndarray:
        """"llama.cpp and the ubatch", "The mask is doing the work": skip empty cells, cells of other
        sequences, under causal attention cells from the future, and for
        models with sliding-window attention cells outside the window.  The
        query's sequence is its FIRST listed id.  Cells j < nkv of stream s.

        The window rule is elided on the page (``is_masked_swa(...)``).
        Reading: with a window of ``swa`` > 0 positions a cell is outside it
        when ``q_pos - pos >= swa``, i.e. a query sees the last ``swa``
        positions up to its own; ``swa == 0`` means no window."""
        pos = self.pos[s, :nkv]
        vis = (pos >= 0) & self.member[s, :nkv, q_seq0]
        if causal:
            vis &= pos <= q_pos
        if swa > 0:
            vis &= q_pos - pos < swa
        return vis

    def mask(self, streams, q_pos, q_seq0, causal=True, swa=0) -> np.ndarray:
        """F16 KQ mask [n_tokens][n_kv]: 0 where visible, -inf elsewhere,
        row-major without padding (encoding is a reading)."""
        nkv = self.n_kv()
        m = np.full((len(q_pos), nkv), MASK_HIDDEN, dtype=np.float16)
        for i in range(len(q_pos)):
            m[i, self.visible_row(streams[i], q_pos[i], q_seq0[i], nkv, causal, swa)] = MASK_VISIBLE
        return m
