"""ctypes binding of libkvattn.so (include/kvattn.h, include/kvsched.h), same
names as the C ABI.

Argument marshalling only: every step of the path runs in the library.  The
``Context`` class adds torch plumbing -- it allocates the F16 K/V caches and
the workspace on the GPU and passes their addresses down.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# KVATTN_LIB selects another build of the same library (the host-sanitizer
# build for CPU test runs); the default is the in-tree libkvattn.so
LIB_PATH = os.environ.get("KVATTN_LIB") or os.path.join(HERE, "libkvattn.so")

KVATTN_OK, KVATTN_NO_SLOT = 0, 1
KVATTN_SPLIT_AUTO, KVATTN_SPLIT_SIMPLE, KVATTN_SPLIT_EQUAL, KVATTN_SPLIT_SEQ = 0, 1, 2, 3
SPLIT_MODES = {"auto": KVATTN_SPLIT_AUTO, "simple": KVATTN_SPLIT_SIMPLE, "equal": KVATTN_SPLIT_EQUAL,
               "seq": KVATTN_SPLIT_SEQ}
KVATTN_EINVAL, KVATTN_ESTATE, KVATTN_ENOMEM, KVATTN_EHIP, KVATTN_ENODEV = -1, -2, -3, -4, -5
KVATTN_ADMIT_RESERVE, KVATTN_ADMIT_PAGED = 0, 1
ADMIT_POLICIES = {"reserve": KVATTN_ADMIT_RESERVE, "paged": KVATTN_ADMIT_PAGED}
KVATTN_REQ_WAITING, KVATTN_REQ_RUNNING, KVATTN_REQ_DONE = 0, 1, 2
KVATTN_PREEMPT_RECOMPUTE, KVATTN_PREEMPT_SWAP = 0, 1
KVATTN_KERNEL_MFMA, KVATTN_KERNEL_VALU, KVATTN_KERNEL_MERGE = 0, 1, 2
PREEMPT_MODES = {"recompute": KVATTN_PREEMPT_RECOMPUTE, "swap": KVATTN_PREEMPT_SWAP}
MAX_SEQ = 256
SEQ_WORDS = 4          # a sequence set is 4 uint64 words: id q is bit q % 64 of word q // 64

_i32p = ctypes.POINTER(ctypes.c_int32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_vpp = ctypes.POINTER(ctypes.c_void_p)


class kvattn_params(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("n_head", ctypes.c_int32),
                ("n_head_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_size", ctypes.c_int32), ("n_stream", ctypes.c_int32),
                ("n_seq_max", ctypes.c_int32), ("n_batch", ctypes.c_int32),
                ("n_ubatch", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("kq_scale", ctypes.c_float), ("cell_order", _i32p),
                ("k_layers", _vpp), ("v_layers", _vpp),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("device", ctypes.c_int32), ("attend_layers", ctypes.c_int32),
                ("split_mode", ctypes.c_int32), ("swa_window", ctypes.c_int32)]


class kvattn_batch(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("pos", _i32p), ("n_seq_id", _i32p),
                ("seq_id", ctypes.POINTER(_i32p)), ("output", ctypes.POINTER(ctypes.c_int8))]


class kvattn_ubatch(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("n_seq_tokens", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("n_seqs_unq", ctypes.c_int32), ("n_outputs", ctypes.c_int32),
                ("pos", _i32p), ("n_seq_id", _i32p), ("seq_id", ctypes.POINTER(_i32p)),
                ("seq_id_unq", _i32p), ("output", ctypes.POINTER(ctypes.c_int8)),
                ("src_idx", _i32p), ("stream", _i32p), ("cells", _i32p),
                ("n_copies", ctypes.c_int32), ("copy_src", _i32p), ("copy_stream", _i32p),
                ("copy_cell", _i32p)]


class kvattn_sched_params(ctypes.Structure):
    _fields_ = [("token_budget", ctypes.c_int32), ("max_running", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("chunked", ctypes.c_int32), ("max_requests", ctypes.c_int32),
                ("preempt", ctypes.c_int32), ("swap_space", ctypes.c_void_p),
                ("swap_bytes", ctypes.c_size_t), ("hip_stream", ctypes.c_void_p)]


class kvattn_sched_iter(ctypes.Structure):
    _fields_ = [("batch", kvattn_batch), ("req", _i32p),
                ("n_retired", ctypes.c_int32), ("retired", _i32p),
                ("n_preempted", ctypes.c_int32), ("preempted", _i32p),
                ("n_admitted", ctypes.c_int32), ("admitted", _i32p), ("admitted_seq", _i32p),
                ("n_swapped_out", ctypes.c_int32), ("swapped_out", _i32p),
                ("n_swapped_in", ctypes.c_int32), ("swapped_in", _i32p),
                ("n_running", ctypes.c_int32), ("n_waiting", ctypes.c_int32),
                ("n_decode", ctypes.c_int32)]


class KvattnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"kvattn error {code}: {msg}")
        self.code = code


_lib = None

SIGNATURES = {
    "kvattn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(kvattn_params)]),
    "kvattn_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(kvattn_params)]),
    "kvattn_create": (ctypes.c_int, [ctypes.POINTER(kvattn_params), ctypes.POINTER(ctypes.c_void_p)]),
    "kvattn_destroy": (None, [ctypes.c_void_p]),
    "kvattn_split": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_batch),
                                    ctypes.POINTER(kvattn_ubatch), ctypes.c_int32, _i32p, _i32p]),
    "kvattn_store": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_ubatch), ctypes.c_int32,
                                    ctypes.c_int32, _vpp, _vpp, ctypes.c_void_p]),
    "kvattn_attend": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_ubatch), ctypes.c_int32,
                                     ctypes.c_int32, _vpp, _vpp, ctypes.c_int32, ctypes.c_void_p]),
    "kvattn_attend_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_ubatch), ctypes.c_int32,
                                             ctypes.c_int32, _vpp, _vpp, ctypes.c_int32, ctypes.c_void_p]),
    "kvattn_time_next_attend": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "kvattn_n_kv": (ctypes.c_int32, [ctypes.c_void_p]),
    "kvattn_probe_gather": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "kvattn_probe_mfma": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p]),
    "kvattn_get_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_ubatch), ctypes.c_void_p,
                                       ctypes.c_size_t, _i32p, ctypes.c_void_p]),
    "kvattn_get_classes": (ctypes.c_int, [ctypes.c_void_p, _i32p, _i32p, _u64p, _i32p, ctypes.c_int32,
                                          _i32p, _i32p, ctypes.c_int32, ctypes.c_void_p]),
    "kvattn_get_cells": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, _i32p, _u64p]),
    "kvattn_seq_rm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "kvattn_seq_pos_max": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32]),
    "kvattn_plan_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, _i32p]),
    "kvattn_get_params": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_params)]),
    "kvattn_seq_state_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "kvattn_seq_state_save": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p]),
    "kvattn_seq_state_load": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p]),
    "kvattn_last_error": (ctypes.c_char_p, [ctypes.c_void_p]),
    "kvattn_sched_create": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_sched_params),
                                           ctypes.POINTER(ctypes.c_void_p)]),
    "kvattn_sched_destroy": (None, [ctypes.c_void_p]),
    "kvattn_sched_submit": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _i32p]),
    "kvattn_sched_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(kvattn_sched_iter)]),
    "kvattn_sched_advance": (ctypes.c_int, [ctypes.c_void_p]),
    "kvattn_sched_request": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, _i32p, _i32p, _i32p, _i32p]),
    "kvattn_sched_last_error": (ctypes.c_char_p, [ctypes.c_void_p]),
}


def load(path: str = LIB_PATH):
    """Load the HIP library; raises when it has not been built (there is no
    fallback implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m ubatch_attention_paged_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _arr(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.POINTER(np.ctypeslib.as_ctypes_type(dtype)))


# --- thin wrappers with the C names ---------------------------------------

def kvattn_workspace_bytes(p: kvattn_params) -> int:
    return load().kvattn_workspace_bytes(ctypes.byref(p))


def kvattn_cache_bytes(p: kvattn_params) -> int:
    return load().kvattn_cache_bytes(ctypes.byref(p))


def kvattn_create(p: kvattn_params) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    rc = load().kvattn_create(ctypes.byref(p), ctypes.byref(ctx))
    if rc != 0:
        raise KvattnError(rc, "kvattn_create rejected the parameters")
    return ctx


def kvattn_destroy(ctx):
    load().kvattn_destroy(ctx)


def kvattn_last_error(ctx) -> str:
    r = load().kvattn_last_error(ctx)
    return r.decode() if r else ""


def _take(p, k, dt):
    return np.ctypeslib.as_array(p, shape=(k,)).astype(dt) if k else np.zeros(0, dt)


class Ubatch:
    """Host-side copy of a kvattn_ubatch plus the raw struct for later calls."""

    def __init__(self, raw: kvattn_ubatch):
        self.raw = raw
        n = raw.n_tokens
        self.id = raw.id
        self.n_tokens = n
        self.n_seq_tokens, self.n_seqs = raw.n_seq_tokens, raw.n_seqs
        self.n_outputs = raw.n_outputs
        self.pos = _take(raw.pos, n, np.int32)
        self.src = _take(raw.src_idx, n, np.int32)
        self.stream = _take(raw.stream, n, np.int32)
        self.cells = _take(raw.cells, n, np.int32)
        self.output = _take(raw.output, n, np.int8)
        self.seq_id_unq = _take(raw.seq_id_unq, raw.n_seqs_unq, np.int32)
        self.copies = list(zip(_take(raw.copy_src, raw.n_copies, np.int32).tolist(),
                               _take(raw.copy_stream, raw.n_copies, np.int32).tolist(),
                               _take(raw.copy_cell, raw.n_copies, np.int32).tolist()))
        self._seq_ids = None

    @property
    def seq_ids(self):
        """Sequence ids of every slot (first id first), read on demand."""
        if self._seq_ids is None:
            raw, n = self.raw, self.n_tokens
            nsid = _take(raw.n_seq_id, n, np.int32)
            self._seq_ids = [tuple(raw.seq_id[i][t] for t in range(nsid[i])) for i in range(n)]
        return self._seq_ids


class SeqIds:
    """Sequence-id lists marshalled once: a flat int32 array, the count per
    slot and a matching array of row addresses (what llama_batch.seq_id
    points at)."""

    def __init__(self, seq_ids):
        if isinstance(seq_ids, np.ndarray) and seq_ids.ndim == 2:
            self.flat = np.ascontiguousarray(seq_ids, np.int32).reshape(-1)
            self.counts = np.full(seq_ids.shape[0], seq_ids.shape[1], np.int32)
        else:
            self.counts = np.fromiter((len(s) for s in seq_ids), np.int32, len(seq_ids))
            self.flat = np.fromiter((x for s in seq_ids for x in s), np.int32, int(self.counts.sum()))
        offs = np.zeros(len(self.counts), np.int64)
        if len(self.counts) > 1:
            offs[1:] = np.cumsum(self.counts[:-1])
        self.rows = (self.flat.ctypes.data + 4 * offs).astype(np.uint64)

    def __len__(self):
        return len(self.counts)


def kvattn_split(ctx, n_tokens, pos=None, seq_ids=None, output=None, cap=None, with_ids=False):
    """Returns (status, [Ubatch], output_ids or None).  status is 0 or 1
    (no room); invalid input raises KvattnError.  With ``with_ids`` the
    output_ids buffer holds the library's clamped n_batch entries
    (kvattn_get_params), as kvattn_split fills."""
    lib = load()
    keep = []
    b = kvattn_batch()
    b.n_tokens = n_tokens
    if pos is not None:
        a, p = _arr(pos, np.int32)
        keep.append(a)
        b.pos = p
    if seq_ids is not None:
        sid = seq_ids if isinstance(seq_ids, SeqIds) else SeqIds(seq_ids)
        if len(sid) < n_tokens:
            raise KvattnError(KVATTN_EINVAL, "fewer sequence-id lists than tokens")
        keep.append(sid)
        b.seq_id = ctypes.cast(ctypes.c_void_p(sid.rows.ctypes.data), ctypes.POINTER(_i32p))
        b.n_seq_id = sid.counts.ctypes.data_as(_i32p)
    if output is not None:
        a, p = _arr(output, np.int8)
        keep.append(a)
        b.output = p
    return _split(lib, ctx, b, keep, cap, kvattn_get_params(ctx).n_batch if with_ids else 0)


def kvattn_split_batch(ctx, b: kvattn_batch, cap=None):
    """kvattn_split of an already marshalled batch (e.g. a scheduler's)."""
    return _split(load(), ctx, b, None, cap, 0)


def _split(lib, ctx, b, keep, cap, n_batch_ids):
    n_tokens = b.n_tokens
    if cap is None:
        cap = max(1, n_tokens)
    ubs = (kvattn_ubatch * cap)()
    n_ubs = ctypes.c_int32(0)
    ids = np.zeros(max(1, n_batch_ids), np.int32)
    rc = lib.kvattn_split(ctx, ctypes.byref(b), ubs, cap, ctypes.byref(n_ubs),
                          ids.ctypes.data_as(_i32p) if n_batch_ids else None)
    if rc < 0:
        raise KvattnError(rc, kvattn_last_error(ctx))
    if rc == KVATTN_NO_SLOT:
        return rc, [], None
    return rc, [Ubatch(ubs[k]) for k in range(n_ubs.value)], (ids if n_batch_ids else None)


def _ptrs(vals):
    arr = (ctypes.c_void_p * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


def kvattn_store(ctx, ub: Ubatch, il0, k_ptrs: Sequence[int], v_ptrs: Sequence[int], stream=0):
    rc = load().kvattn_store(ctx, ctypes.byref(ub.raw), il0, len(k_ptrs),
                             ctypes.cast(_ptrs(k_ptrs), _vpp), ctypes.cast(_ptrs(v_ptrs), _vpp),
                             ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))


def kvattn_attend(ctx, ub: Ubatch, il0, q_ptrs: Sequence[int], out_ptrs: Sequence[int], only_outputs=0, stream=0):
    rc = load().kvattn_attend(ctx, ctypes.byref(ub.raw), il0, len(q_ptrs),
                              ctypes.cast(_ptrs(q_ptrs), _vpp), ctypes.cast(_ptrs(out_ptrs), _vpp),
                              int(only_outputs), ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))


def kvattn_attend_noalloc(ctx, ub: Ubatch, il0, q_ptrs: Sequence[int], out_ptrs: Sequence[int], only_outputs=0,
                          stream=0):
    rc = load().kvattn_attend_noalloc(ctx, ctypes.byref(ub.raw), il0, len(q_ptrs),
                                      ctypes.cast(_ptrs(q_ptrs), _vpp), ctypes.cast(_ptrs(out_ptrs), _vpp),
                                      int(only_outputs), ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))


def kvattn_time_next_attend(ctx, kind, start_event, stop_event):
    """Bind two HIP events (hipEvent_t handles) to the start and end of
    kernel ``kind`` (KVATTN_KERNEL_*) in the next attend call."""
    rc = load().kvattn_time_next_attend(ctx, int(kind), ctypes.c_void_p(start_event), ctypes.c_void_p(stop_event))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))


def kvattn_probe_gather(rows, n_rows, index, n_index, out, n_wg, stream=0):
    """Device addresses: rows [n_rows][1024] F16, index int32[n_index],
    out float[n_wg * 256]."""
    rc = load().kvattn_probe_gather(ctypes.c_void_p(rows), n_rows, ctypes.c_void_p(index), n_index,
                                    ctypes.c_void_p(out), n_wg, ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, "kvattn_probe_gather")


def kvattn_probe_mfma(ab, out, n_wg, iters, stream=0):
    """Device addresses: ab 16 F16, out float[n_wg * 256]."""
    rc = load().kvattn_probe_mfma(ctypes.c_void_p(ab), ctypes.c_void_p(out), n_wg, iters, ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, "kvattn_probe_mfma")


def kvattn_n_kv(ctx) -> int:
    return load().kvattn_n_kv(ctx)


def kvattn_get_mask(ctx, ub: Ubatch, d_mask_ptr: int, cap_elems: int, stream=0) -> int:
    nkv = ctypes.c_int32(0)
    rc = load().kvattn_get_mask(ctx, ctypes.byref(ub.raw), ctypes.c_void_p(d_mask_ptr), cap_elems,
                                ctypes.byref(nkv), ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))
    return nkv.value


def kvattn_get_classes(ctx, stream=0):
    """Returns list of (stream, mask, cells ndarray) in class order."""
    lib = load()
    ncls, ncells = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = lib.kvattn_get_classes(ctx, ctypes.byref(ncls), None, None, None, 0, ctypes.byref(ncells), None, 0,
                                ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))
    k, n = ncls.value, ncells.value
    st = np.zeros(max(1, k), np.int32)
    mk = np.zeros((max(1, k), SEQ_WORDS), np.uint64)
    ct = np.zeros(max(1, k), np.int32)
    cells = np.zeros(max(1, n), np.int32)
    rc = lib.kvattn_get_classes(ctx, ctypes.byref(ncls), st.ctypes.data_as(_i32p), mk.ctypes.data_as(_u64p),
                                ct.ctypes.data_as(_i32p), k, ctypes.byref(ncells), cells.ctypes.data_as(_i32p), n,
                                ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))
    out, off = [], 0
    for i in range(k):
        out.append((int(st[i]), seqset_int(mk[i]), cells[off:off + ct[i]].copy()))
        off += ct[i]
    return out


def seqset_int(words):
    """A sequence set (SEQ_WORDS uint64 words) as one Python integer: bit q
    set when sequence q is a member."""
    return sum(int(w) << (64 * j) for j, w in enumerate(words))


def seqset_members(mask, n_seq):
    """Membership table [n, n_seq] (bool) of n sequence sets given as an
    [n, SEQ_WORDS] uint64 array."""
    q = np.arange(n_seq)
    return ((mask[:, q // 64] >> (q % 64).astype(np.uint64)) & np.uint64(1)).astype(bool)


def kvattn_get_cells(ctx, stream: int, kv_size: int):
    """(pos [kv_size] int32, mask [kv_size, SEQ_WORDS] uint64) of one stream."""
    pos = np.zeros(kv_size, np.int32)
    mask = np.zeros((kv_size, SEQ_WORDS), np.uint64)
    rc = load().kvattn_get_cells(ctx, stream, pos.ctypes.data_as(_i32p), mask.ctypes.data_as(_u64p))
    if rc != 0:
        raise KvattnError(rc, "kvattn_get_cells")
    return pos, mask


def kvattn_seq_rm(ctx, seq_id, p0=-1, p1=-1):
    rc = load().kvattn_seq_rm(ctx, seq_id, p0, p1)
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))


def kvattn_seq_pos_max(ctx, seq_id) -> int:
    return load().kvattn_seq_pos_max(ctx, seq_id)


def kvattn_seq_state_size(ctx, seq_id) -> int:
    n = ctypes.c_size_t(0)
    rc = load().kvattn_seq_state_size(ctx, seq_id, ctypes.byref(n))
    if rc != 0:
        raise KvattnError(rc, "kvattn_seq_state_size: sequence id out of range")
    return n.value


def kvattn_seq_state_save(ctx, seq_id, dst_ptr, cap, stream=0) -> int:
    n = ctypes.c_size_t(0)
    rc = load().kvattn_seq_state_save(ctx, seq_id, ctypes.c_void_p(dst_ptr), cap, ctypes.byref(n),
                                      ctypes.c_void_p(stream))
    if rc != 0:
        raise KvattnError(rc, kvattn_last_error(ctx))
    return n.value


def kvattn_seq_state_load(ctx, seq_id, src_ptr, nbytes, stream=0) -> int:
    """Returns 0, or KVATTN_NO_SLOT when the cells do not fit (nothing
    changed); invalid blobs raise."""
    rc = load().kvattn_seq_state_load(ctx, seq_id, ctypes.c_void_p(src_ptr), nbytes, ctypes.c_void_p(stream))
    if rc < 0:
        raise KvattnError(rc, kvattn_last_error(ctx))
    return rc


def kvattn_get_params(ctx) -> kvattn_params:
    p = kvattn_params()
    rc = load().kvattn_get_params(ctx, ctypes.byref(p))
    if rc != 0:
        raise KvattnError(rc, "kvattn_get_params")
    return p


def kvattn_plan_stats(ctx, only_outputs=0):
    vals = [ctypes.c_int32(0) for _ in range(5)]
    load().kvattn_plan_stats(ctx, int(only_outputs), *[ctypes.byref(v) for v in vals])
    keys = ("n_classes", "n_items_valu", "n_items_mfma", "n_partial_rows", "n_reduced")
    return dict(zip(keys, [v.value for v in vals]))


# --- torch plumbing ----------------------------------------------------------

class Context:
    """One library context plus its device memory.

    The caches live in one torch allocation holding K0, V0, K1, V1, ... in
    layer order ("What does llama.cpp's KV cache actually look like in
    memory?", "28 layers, 56 tensors"); each tensor is [n_stream][kv_size][E]
    F16.  ``device=None`` makes a host-only context (split / placement only).
    """

    def __init__(self, n_layer, n_head, n_head_kv, head_dim, kv_size, n_stream=1, n_seq_max=1,
                 n_batch=0, n_ubatch=512, causal=True, kq_scale=0.0, cell_order=None, device=None,
                 attend_layers=0, split_mode=0, swa_window=0):
        self.n_layer, self.n_head, self.n_head_kv, self.head_dim = n_layer, n_head, n_head_kv, head_dim
        self.kv_size, self.n_stream, self.n_seq_max = kv_size, n_stream, n_seq_max
        self.E = n_head_kv * head_dim
        p = kvattn_params()
        p.n_layer, p.n_head, p.n_head_kv, p.head_dim = n_layer, n_head, n_head_kv, head_dim
        p.kv_size, p.n_stream, p.n_seq_max = kv_size, n_stream, n_seq_max
        p.n_batch, p.n_ubatch, p.causal, p.kq_scale = n_batch, n_ubatch, int(bool(causal)), kq_scale
        p.attend_layers = attend_layers
        p.split_mode = SPLIT_MODES[split_mode] if isinstance(split_mode, str) else int(split_mode)
        p.swa_window = swa_window
        self._order = None
        if cell_order is not None:
            self._order, p.cell_order = _arr(np.asarray(cell_order).reshape(-1), np.int32)
        self.device = device
        self.cache = None
        if device is not None:
            import torch
            dev = torch.device(device)
            p.device = dev.index or 0
            per = n_stream * kv_size * self.E
            self.cache = torch.zeros(2 * n_layer * per, dtype=torch.float16, device=dev)
            self.K = [self.cache[(2 * l) * per:(2 * l + 1) * per].view(n_stream, kv_size, self.E) for l in range(n_layer)]
            self.V = [self.cache[(2 * l + 1) * per:(2 * l + 2) * per].view(n_stream, kv_size, self.E) for l in range(n_layer)]
            ws = kvattn_workspace_bytes(p)
            if ws == 0:
                raise KvattnError(KVATTN_EINVAL, "invalid parameters")
            self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
            self._kp = _ptrs([t.data_ptr() for t in self.K])
            self._vp = _ptrs([t.data_ptr() for t in self.V])
            p.k_layers = ctypes.cast(self._kp, _vpp)
            p.v_layers = ctypes.cast(self._vp, _vpp)
            p.workspace = self.workspace.data_ptr()
            p.workspace_bytes = ws
        self.params = p
        self.ctx = kvattn_create(p)

    def close(self):
        if self.ctx:
            kvattn_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self, stream):
        if stream is not None:
            return stream
        if self.device is None:
            return 0
        import torch
        return torch.cuda.current_stream(torch.device(self.device)).cuda_stream

    def split(self, n_tokens, pos=None, seq_ids=None, output=None, with_ids=False):
        return kvattn_split(self.ctx, n_tokens, pos, seq_ids, output, with_ids=with_ids)

    def split_batch(self, b: kvattn_batch):
        return kvattn_split_batch(self.ctx, b)

    def n_batch(self):
        """The context's n_batch as the library clamped it (sizes output_ids)."""
        return kvattn_get_params(self.ctx).n_batch

    def store(self, ub, il0, k_list, v_list, stream=None):
        kvattn_store(self.ctx, ub, il0, [t.data_ptr() for t in k_list], [t.data_ptr() for t in v_list],
                     self._stream(stream))

    def attend(self, ub, il0, q_list, out_list, only_outputs=False, stream=None):
        kvattn_attend(self.ctx, ub, il0, [t.data_ptr() for t in q_list], [t.data_ptr() for t in out_list],
                      only_outputs, self._stream(stream))

    def attend_noalloc(self, ub, il0, q_list, out_list, only_outputs=False, stream=None):
        kvattn_attend_noalloc(self.ctx, ub, il0, [t.data_ptr() for t in q_list], [t.data_ptr() for t in out_list],
                              only_outputs, self._stream(stream))

    def mask(self, ub, stream=None):
        import torch
        nkv = kvattn_n_kv(self.ctx)
        buf = torch.empty(ub.n_tokens * nkv, dtype=torch.int16, device=self.device)
        got = kvattn_get_mask(self.ctx, ub, buf.data_ptr(), buf.numel(), self._stream(stream))
        return buf[:ub.n_tokens * got].view(ub.n_tokens, got)

    def classes(self, stream=None):
        return kvattn_get_classes(self.ctx, self._stream(stream))

    def cells(self, stream=0):
        return kvattn_get_cells(self.ctx, stream, self.kv_size)

    def seq_rm(self, seq_id, p0=-1, p1=-1):
        kvattn_seq_rm(self.ctx, seq_id, p0, p1)

    def state_size(self, seq_id):
        return kvattn_seq_state_size(self.ctx, seq_id)

    def state_save(self, seq_id, out=None, stream=None):
        """Serialized state of a sequence as a uint8 device tensor (``out``
        when given, else a new one of exactly the size)."""
        import torch
        n = self.state_size(seq_id)
        if out is None:
            out = torch.empty(n, dtype=torch.uint8, device=self.device)
        kvattn_seq_state_save(self.ctx, seq_id, out.data_ptr(), out.numel(), self._stream(stream))
        return out[:n]

    def state_load(self, seq_id, blob, stream=None):
        """Restore a uint8 device tensor as sequence seq_id; returns 0 or
        KVATTN_NO_SLOT."""
        return kvattn_seq_state_load(self.ctx, seq_id, blob.data_ptr(), blob.numel(), self._stream(stream))

    def n_kv(self):
        return kvattn_n_kv(self.ctx)

    def plan_stats(self, only_outputs=False):
        return kvattn_plan_stats(self.ctx, only_outputs)


# --- the iteration-level batching loop (include/kvsched.h) ------------------

def kvattn_sched_create(ctx, token_budget=0, max_running=0, policy="paged", block_size=1, chunked=True,
                        max_requests=4096, preempt="recompute", swap_space=0, swap_bytes=0, stream=0):
    p = kvattn_sched_params()
    p.token_budget, p.max_running = token_budget, max_running
    p.policy = ADMIT_POLICIES[policy] if isinstance(policy, str) else int(policy)
    p.block_size, p.chunked, p.max_requests = block_size, int(bool(chunked)), max_requests
    p.preempt = PREEMPT_MODES[preempt] if isinstance(preempt, str) else int(preempt)
    p.swap_space, p.swap_bytes, p.hip_stream = swap_space or None, swap_bytes, stream or None
    out = ctypes.c_void_p()
    rc = load().kvattn_sched_create(ctx, ctypes.byref(p), ctypes.byref(out))
    if rc != 0:
        raise KvattnError(rc, "kvattn_sched_create: invalid scheduler parameters")
    return out


def kvattn_sched_destroy(s):
    load().kvattn_sched_destroy(s)


def kvattn_sched_last_error(s) -> str:
    r = load().kvattn_sched_last_error(s)
    return r.decode() if r else ""


def kvattn_sched_submit(s, n_prompt, n_generate) -> int:
    rid = ctypes.c_int32(-1)
    rc = load().kvattn_sched_submit(s, n_prompt, n_generate, ctypes.byref(rid))
    if rc != 0:
        raise KvattnError(rc, kvattn_sched_last_error(s))
    return rid.value


def kvattn_sched_step(s, it: kvattn_sched_iter):
    rc = load().kvattn_sched_step(s, ctypes.byref(it))
    if rc != 0:
        raise KvattnError(rc, kvattn_sched_last_error(s))


def kvattn_sched_advance(s):
    rc = load().kvattn_sched_advance(s)
    if rc != 0:
        raise KvattnError(rc, kvattn_sched_last_error(s))


def kvattn_sched_request(s, req_id):
    vals = [ctypes.c_int32(0) for _ in range(4)]
    rc = load().kvattn_sched_request(s, req_id, *[ctypes.byref(v) for v in vals])
    if rc != 0:
        raise KvattnError(rc, "unknown request id")
    return dict(zip(("state", "seq", "n_cached", "n_sampled"), [v.value for v in vals]))


class Scheduler:
    """The native loop over a ``Context``.  ``step()`` returns the raw
    iteration (``.batch`` feeds ``Context.split_batch``) and ``record()``
    its host copy as plain lists."""

    def __init__(self, ctx: "Context", token_budget=0, max_running=0, policy="paged", block_size=1,
                 chunked=True, max_requests=4096, preempt="recompute", swap_bytes=0, stream=None):
        """With preempt="swap" on a device context the swap arena is a uint8
        device tensor of swap_bytes allocated here; saves and restores run
        on ``stream`` (torch's current stream by default)."""
        self.context = ctx
        self.swap = None
        ptr = 0
        if preempt == "swap" and swap_bytes and ctx.device is not None:
            import torch
            self.swap = torch.empty(swap_bytes, dtype=torch.uint8, device=ctx.device)
            ptr = self.swap.data_ptr()
        self.s = kvattn_sched_create(ctx.ctx, token_budget, max_running, policy, block_size, chunked,
                                     max_requests, preempt, ptr, swap_bytes, ctx._stream(stream))
        self.it = kvattn_sched_iter()

    def close(self):
        if self.s:
            kvattn_sched_destroy(self.s)
            self.s = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, n_prompt, n_generate):
        return kvattn_sched_submit(self.s, n_prompt, n_generate)

    def step(self) -> kvattn_sched_iter:
        kvattn_sched_step(self.s, self.it)
        return self.it

    def advance(self):
        kvattn_sched_advance(self.s)

    def request(self, req_id):
        return kvattn_sched_request(self.s, req_id)

    def record(self):
        it = self.it
        n = it.batch.n_tokens
        seq = [it.batch.seq_id[i][0] for i in range(n)]
        return {"retired": _take(it.retired, it.n_retired, np.int32).tolist(),
                "preempted": _take(it.preempted, it.n_preempted, np.int32).tolist(),
                "admitted": list(zip(_take(it.admitted, it.n_admitted, np.int32).tolist(),
                                     _take(it.admitted_seq, it.n_admitted, np.int32).tolist())),
                "swapped_out": _take(it.swapped_out, it.n_swapped_out, np.int32).tolist(),
                "swapped_in": _take(it.swapped_in, it.n_swapped_in, np.int32).tolist(),
                "req": _take(it.req, n, np.int32).tolist(), "seq": seq,
                "pos": _take(it.batch.pos, n, np.int32).tolist(),
                "output": _take(it.batch.output, n, np.int8).tolist(),
                "n_running": it.n_running, "n_waiting": it.n_waiting, "n_decode": it.n_decode}
