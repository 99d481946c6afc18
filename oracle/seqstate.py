"""Save / restore of one sequence's cached K/V, in the record layout of
"What does llama.cpp's KV cache actually look like in memory?".

Test infrastructure only (see ``oracle/__init__.py``).

"What does llama.cpp's KV cache actually look like in memory?", "Opening the .bin dump" saves one sequence's occupied cells across all
layers and describes the file: metadata first, then one record per layer
for K (layers 0..L-1), then one per layer for V; each record is a small
header followed by the sequence's rows.  Its numbers fix the sizes: seven
cells of the Qwen3-0.6B shape make 802,816 payload bytes and 780 bytes of
metadata (803,596 in all), the first K record starts at byte 108 and its
12-byte header puts the first K value at byte 120.  That is 108 bytes of
leading metadata plus 56 record headers of 12 bytes.

The page does not say what the headers hold.  Reading (stated once, also
for the library): all fields little-endian,

* leading metadata = 80 fixed bytes plus one int32 position per cell
  (80 + 4 * 7 = 108):
  magic "KVSS", u32 version 1, u32 n_layer, u32 n_head_kv, u32 head_dim,
  u32 n_cells, u32 K type, u32 V type (1 = F16), u64 row bytes, u64 offset
  of the first record, u64 total bytes, 24 zero bytes; then the cells'
  positions, ascending;
* record header = u32 type (1 = F16) + u64 row bytes (4 + 8 = 12);
* rows in the order of the positions, each the cell's full row of that
  layer's tensor (all KV heads, "What does llama.cpp's KV cache actually look like in memory?", "One row, one token's keys").

The sequence's cells are every committed cell whose sequence set holds it
(shared prefix cells included), ordered by position (then cell index).
Restoring replaces the destination sequence's cells: it is removed, then
one cell per saved position is placed in its stream, lowest free-cell rank
first (the placement reading of the batch path), all-or-nothing.
"""

from __future__ import annotations

import struct

import numpy as np

MAGIC = b"KVSS"
VERSION = 1
TYPE_F16 = 1
FIXED = 80
RECORD_HEADER = 12


class StateError(ValueError):
    """A blob that does not fit the context, or no room to restore it."""


def state_bytes(n_layer, n_head_kv, head_dim, n_cells):
    """Leading metadata + 2 * n_layer records of header + n_cells rows."""
    row = n_head_kv * head_dim * 2
    return FIXED + 4 * n_cells + 2 * n_layer * (RECORD_HEADER + n_cells * row)


def record_offset(n_layer, n_head_kv, head_dim, n_cells, kind, layer):
    """Byte offset of the record of (kind 0 = K / 1 = V, layer)."""
    row = n_head_kv * head_dim * 2
    r = kind * n_layer + layer
    return FIXED + 4 * n_cells + r * (RECORD_HEADER + n_cells * row)


def sequence_cells(eng, seq):
    """(stream, cells, positions) of a sequence: its stream's committed cells
    holding ``seq``, ordered by (position, cell)."""
    s = seq % eng.n_stream
    pos = eng.cells.pos[s]
    mine = np.nonzero((pos >= 0) & eng.cells.member[s, :, seq])[0]
    order = sorted(mine.tolist(), key=lambda c: (int(pos[c]), c))
    return s, order, [int(pos[c]) for c in order]


def save(eng, seq) -> bytes:
    """Serialize sequence ``seq`` of an oracle engine holding every layer."""
    assert eng.layers == list(range(eng.n_layer)), "the engine must hold every layer"
    s, cells, positions = sequence_cells(eng, seq)
    n, L = len(cells), eng.n_layer
    row = eng.E * 2
    total = state_bytes(L, eng.n_head_kv, eng.head_dim, n)
    out = bytearray()
    out += MAGIC
    out += struct.pack("<7I", VERSION, L, eng.n_head_kv, eng.head_dim, n, TYPE_F16, TYPE_F16)
    out += struct.pack("<3Q", row, FIXED + 4 * n, total)
    out += bytes(FIXED - len(out))
    out += struct.pack(f"<{n}i", *positions)
    for cache in (eng.K, eng.V):
        for layer in range(L):
            out += struct.pack("<IQ", TYPE_F16, row)
            for c in cells:
                out += cache[layer][s, c].astype("<f2").tobytes()
    assert len(out) == total
    return bytes(out)


def parse_header(blob, n_layer, n_head_kv, head_dim):
    """Validate the leading metadata against a context's geometry; returns
    (n_cells, positions)."""
    if len(blob) < FIXED or blob[:4] != MAGIC:
        raise StateError("not a sequence-state blob")
    version, L, hk, hd, n, kt, vt = struct.unpack_from("<7I", blob, 4)
    row, first, total = struct.unpack_from("<3Q", blob, 32)
    if version != VERSION or (L, hk, hd) != (n_layer, n_head_kv, head_dim) or kt != TYPE_F16 or vt != TYPE_F16:
        raise StateError("geometry or type does not match the context")
    if row != n_head_kv * head_dim * 2 or first != FIXED + 4 * n or \
            total != state_bytes(L, hk, hd, n) or len(blob) < total:
        raise StateError("sizes in the metadata are inconsistent")
    positions = list(struct.unpack_from(f"<{n}i", blob, FIXED))
    if any(p < 0 for p in positions):
        raise StateError("negative position")
    for r in range(2 * L):
        off = record_offset(L, hk, hd, n, r // L, r % L)
        if struct.unpack_from("<IQ", blob, off) != (TYPE_F16, row):
            raise StateError("record header does not match")
    return n, positions


def load(eng, seq, blob):
    """Replace sequence ``seq``'s cells with the saved ones."""
    assert eng.layers == list(range(eng.n_layer)), "the engine must hold every layer"
    L = eng.n_layer
    n, positions = parse_header(blob, L, eng.n_head_kv, eng.head_dim)
    s = seq % eng.n_stream
    t = eng.cells
    only_mine = (t.pos[s] >= 0) & t.member[s, :, seq] & (t.member[s].sum(axis=1) == 1)
    if len(t.free_cells_by_rank(s)) + int(only_mine.sum()) < n:
        raise StateError("no room for the saved cells")
    t.seq_rm(seq, -1, -1)
    cells = t.free_cells_by_rank(s)[:n].tolist()
    t.commit([s] * n, cells, positions, [(seq,)] * n)
    row = eng.E * 2
    for kind, cache in enumerate((eng.K, eng.V)):
        for layer in range(L):
            off = record_offset(L, eng.n_head_kv, eng.head_dim, n, kind, layer) + RECORD_HEADER
            rows = np.frombuffer(blob, dtype="<f2", count=n * eng.E, offset=off).reshape(n, eng.E)
            for i, c in enumerate(cells):
                cache[layer][s, c] = rows[i]
    return cells
