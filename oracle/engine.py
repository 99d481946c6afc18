"""The decode loop of the pages, strung together from the oracle's parts.

Test infrastructure only (see ``oracle/__init__.py``).

"Batch、Ubatch 与解码主循环", Part F (the llama_decode main loop): validate and auto-fill the batch,
split it into ubatches and reserve cache cells for all of them, then process
the ubatches in order -- each one writes its K/V rows into its cells and runs
attention over the cells it may see.  Later ubatches of the same batch see
the cells of earlier ones ("Batch、Ubatch 与解码主循环", Part D: a later ubatch's attention reads what an
earlier ubatch wrote; "llama.cpp and the ubatch", "Chunked prefill is the same mechanism").
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .batching import clamp_params, fill_batch, split_batch, output_ids, SplitError
from .kvcache import CellTable, f16_round
from .attention import masked_attention


@dataclass
class OracleUbatch:
    src: list            # batch row of each slot, ubatch order
    pos: list
    seq_ids: list        # tuples, first id first
    output: list
    n_seq_tokens: int
    n_seqs: int
    streams: list
    cells: list
    copies: list = field(default_factory=list)   # (slot index, stream, cell): separate copies
    committed: bool = False
    n_kv: int = 0
    mask: np.ndarray = field(default=None, repr=False)

    @property
    def n_tokens(self):
        return len(self.src)


class OracleEngine:
    """Cell table + per-layer F16 caches (only the layers in ``layers``)."""

    def __init__(self, n_layer, n_head, n_head_kv, head_dim, kv_size, n_stream=1,
                 n_seq_max=1, n_batch=0, n_ubatch=512, causal=True, kq_scale=None, swa=0,
                 cell_order=None, layers=None, split_mode="auto"):
        self.n_layer, self.n_head, self.n_head_kv, self.head_dim = n_layer, n_head, n_head_kv, head_dim
        self.kv_size, self.n_stream, self.n_seq_max = kv_size, n_stream, n_seq_max
        self.causal = bool(causal)
        self.swa = int(swa)                   # sliding window in positions, 0 = none
        self.kq_scale = kq_scale
        self.split_mode = split_mode          # "auto", "simple", "equal" or "seq"
        self.n_batch, self.n_ubatch = clamp_params(kv_size * n_stream, n_batch, n_ubatch, causal)
        self.cells = CellTable(kv_size, n_stream, n_seq_max, cell_order)
        self.E = n_head_kv * head_dim
        self.layers = list(range(n_layer)) if layers is None else list(layers)
        self.K = {l: np.zeros((n_stream, kv_size, self.E), np.float16) for l in self.layers}
        self.V = {l: np.zeros((n_stream, kv_size, self.E), np.float16) for l in self.layers}
        self._pending = []

    # -- batch intake, split and placement ("Batch、Ubatch 与解码主循环", Part C and Part F) ---------
    def split(self, n_tokens, pos=None, seq_id=None, output=None):
        """Returns (status, ubatches, output_ids); status 1 = no room (nothing
        reserved).  Invalid input raises SplitError.  Cells reserved by a
        previous split and never committed are returned to the free list."""
        for ub in self._pending:
            if not ub.committed:
                self.cells.release(ub.streams, ub.cells)
                self.cells.release([c[1] for c in ub.copies], [c[2] for c in ub.copies])
        self._pending = []
        if n_tokens > self.n_batch:
            raise SplitError("n_tokens > n_batch")       # "llama.cpp and the ubatch": an assertion on n_batch
        next_pos = {}
        if pos is None:
            for s in range(self.n_seq_max):
                next_pos[s] = self.cells.seq_pos_max(s) + 1
        p, sids, out = fill_batch(n_tokens, pos, seq_id, output, next_pos,
                                  self.n_seq_max, self.n_stream)
        parts = split_batch([set(x) for x in sids], self.n_ubatch, self.n_stream, self.split_mode)
        # a slot's cell is in the stream of its first id (seq % n_stream);
        # "What does llama.cpp's KV cache actually look like in memory?", "Unified versus non-unified": with several streams a common
        # prefix needs separate copies -- a slot whose ids span streams also
        # gets a cell in each other stream it touches (ascending), holding
        # the ids that live there.  Cells are taken per stream in slot order.
        want = []                               # (stream, slot, primary?) in placement order
        for (slots, _, _) in parts:
            for i in slots:
                s0 = sids[i][0] % self.n_stream
                want.append((s0, i, True))
                for s2 in sorted({q % self.n_stream for q in sids[i]} - {s0}):
                    want.append((s2, i, False))
        cells = self.cells.reserve([w[0] for w in want])
        if cells is None:
            return 1, [], None
        placed = {}
        for (st, i, prim), c in zip(want, cells):
            placed.setdefault(i, []).append((st, c, prim))
        ubs = []
        for (slots, nst, ns) in parts:
            prim = [next((st, c) for st, c, pr in placed[i] if pr) for i in slots]
            copies = [(k, st, c) for k, i in enumerate(slots) for st, c, pr in placed[i] if not pr]
            ubs.append(OracleUbatch(src=list(slots), pos=[p[i] for i in slots],
                                    seq_ids=[sids[i] for i in slots],
                                    output=[out[i] for i in slots], n_seq_tokens=nst,
                                    n_seqs=ns, streams=[x[0] for x in prim], cells=[x[1] for x in prim],
                                    copies=copies))
        self._pending = ubs
        return 0, ubs, output_ids(out, self.n_batch)

    # -- per ubatch ------------------------------------------------------
    def commit(self, ub: OracleUbatch, build_mask=True):
        """The ubatch's cells become visible, then its mask is built over
        the table as it now stands (later ubatches are not yet committed).
        ``build_mask=False`` only records placement (for placement checks)."""
        here = lambda ids, st: tuple(q for q in ids if q % self.n_stream == st)   # the ids a cell of st holds
        self.cells.commit(ub.streams, ub.cells, ub.pos,
                          [here(ids, st) for ids, st in zip(ub.seq_ids, ub.streams)])
        self.cells.commit([c[1] for c in ub.copies], [c[2] for c in ub.copies], [ub.pos[c[0]] for c in ub.copies],
                          [here(ub.seq_ids[c[0]], c[1]) for c in ub.copies])
        ub.committed = True
        ub.n_kv = self.cells.n_kv()
        if build_mask:
            ub.mask = self.cells.mask(ub.streams, ub.pos, [s[0] for s in ub.seq_ids], self.causal, self.swa)
        return ub.mask

    def store(self, ub: OracleUbatch, layer: int, k_rows, v_rows):
        """Write the ubatch's K/V rows (fp32, ubatch order) into its cells,
        rounded to F16."""
        k16, v16 = f16_round(k_rows), f16_round(v_rows)
        for r, (s, j) in enumerate(zip(ub.streams, ub.cells)):
            self.K[layer][s, j] = k16[r]
            self.V[layer][s, j] = v16[r]
        for r, s, j in ub.copies:
            self.K[layer][s, j] = k16[r]
            self.V[layer][s, j] = v16[r]

    def attend(self, ub: OracleUbatch, layer: int, q_rows):
        """fp64 attention for every slot of the ubatch (ubatch order)."""
        if not ub.committed:
            raise SplitError("attend before commit")
        return masked_attention(q_rows, self.K[layer], self.V[layer], ub.streams, ub.mask,
                                self.n_head, self.n_head_kv, self.kq_scale)

    def seq_rm(self, seq_id, p0=-1, p1=-1):
        self.cells.seq_rm(seq_id, p0, p1)
