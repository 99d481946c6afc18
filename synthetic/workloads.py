"""Seeded workload descriptions: which decode calls a caller makes, in order.

A workload is a list of batches (one per decode call), each a list of token
slots with a position, sequence ids and an output flag, plus the model shape
and cache geometry.  Tensors are drawn on demand, independently per
(batch, layer, tensor) from ``SeedSequence([seed, 2, batch, layer, kind])``
as fp32 standard normals, so any layer of any batch can be regenerated
without drawing the others.  The free-cell order, when a workload asks for a
shuffled one, is ``default_rng(SeedSequence([seed, 1])).permutation``.

Shapes follow Qwen3-0.6B as the pages describe it (28 layers, 8 KV heads of
128 numbers; "What does llama.cpp's KV cache actually look like in memory?",
"28 layers, 56 tensors" and "One row, one token's keys"); its 16 query heads
are the model's published geometry.  Batch sizes default to n_batch=2048 and
n_ubatch=512 ("llama.cpp and the ubatch", "Back to the VRAM question").
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

QWEN3_06B = dict(n_layer=28, n_head=16, n_head_kv=8, head_dim=128)

KIND_K, KIND_V, KIND_Q = 0, 1, 2
PURPOSE_STRUCTURE, PURPOSE_CELL_ORDER, PURPOSE_TENSORS = 0, 1, 2


@dataclass
class Batch:
    pos: np.ndarray                 # int32 [n]
    seq_ids: list                   # list of tuples (first id first)
    output: np.ndarray              # int8 [n]
    measured: bool = True           # attention runs on its ubatches

    @property
    def n_tokens(self):
        return int(len(self.pos))


@dataclass
class Workload:
    name: str
    n_layer: int
    n_head: int
    n_head_kv: int
    head_dim: int
    kv_size: int
    n_stream: int
    n_seq_max: int
    seed: int
    batches: list
    n_batch: int = 2048
    n_ubatch: int = 512
    causal: bool = True
    cell_order: Optional[np.ndarray] = field(default=None, repr=False)
    split_mode: str = "auto"          # "auto", "simple", "equal" or "seq"
    swa: int = 0                      # sliding window in positions, 0 = none
    note: str = ""

    @property
    def E(self):
        return self.n_head_kv * self.head_dim

    def width(self, kind):
        return self.n_head * self.head_dim if kind == KIND_Q else self.E

    def tensor(self, b: int, layer: int, kind: int) -> np.ndarray:
        """fp32 [n_tokens of batch b][width] standard normals."""
        n = self.batches[b].n_tokens
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, PURPOSE_TENSORS, b, layer, kind]))
        return rng.standard_normal((n, self.width(kind)), dtype=np.float32)

    def params(self):
        return dict(n_layer=self.n_layer, n_head=self.n_head, n_head_kv=self.n_head_kv,
                    head_dim=self.head_dim, kv_size=self.kv_size, n_stream=self.n_stream,
                    n_seq_max=self.n_seq_max, n_batch=self.n_batch, n_ubatch=self.n_ubatch,
                    causal=self.causal)

    def measured_tokens(self):
        return sum(b.n_tokens for b in self.batches if b.measured)


def _chunks(n, size):
    return [(a, min(n, a + size)) for a in range(0, n, size)]


def _batch(pos, seqs, out, measured=True):
    return Batch(np.asarray(pos, np.int32), [tuple(s) for s in seqs],
                 np.asarray(out, np.int8), measured)


def _prompt_batches(seq_set, start, length, n_batch, measured, out_last=True):
    """A prompt of ``length`` tokens at positions start.. for ``seq_set``,
    cut into caller-side calls of at most n_batch slots ("llama.cpp and the
    ubatch", "Three things called batch": 5000 tokens -> 2048, 2048, 904)."""
    res = []
    for a, b in _chunks(length, n_batch):
        out = np.zeros(b - a, np.int8)
        if out_last and b == length:
            out[-1] = 1
        res.append(_batch(np.arange(start + a, start + b), [seq_set] * (b - a), out, measured))
    return res


def tiny(seed=1001):
    """1 layer, 2 query heads over 1 KV head of 16, 64 cells, one sequence: a
    7-token prompt in one ubatch, then 8 single-token decode ubatches."""
    batches = [_batch(np.arange(7), [(0,)] * 7, [0] * 6 + [1])]
    for p in range(7, 15):
        batches.append(_batch([p], [(0,)], [1]))
    return Workload("tiny", 1, 2, 1, 16, kv_size=64, n_stream=1, n_seq_max=1,
                    seed=seed, batches=batches)


def qwen_prefill(n_prompt=3000, n_layer=28, kv_size=4096, n_batch=2048, n_ubatch=512, seed=1002):
    """Single-sequence prefill of an n_prompt-token prompt on the Qwen3-0.6B
    shape; output flag only on the prompt's last token."""
    batches = _prompt_batches((0,), 0, n_prompt, n_batch, measured=True)
    return Workload("qwen_prefill", n_layer, 16, 8, 128, kv_size=kv_size, n_stream=1,
                    n_seq_max=1, seed=seed, batches=batches, n_batch=n_batch, n_ubatch=n_ubatch,
                    note=f"{n_prompt}-token prompt, n_batch={n_batch}, n_ubatch={n_ubatch}")


CB_LENGTHS = (64, 128, 256, 512, 512, 1024, 1024, 2048)


def cb_decode(n_seq=64, lengths=CB_LENGTHS, n_layer=28, kv_size=65536, shuffled=True, seed=1003):
    """Continuous-batching decode step: sequence i holds lengths[i % 8] cached
    tokens (positions 0..L-1, stored by setup calls), then one measured call
    with one token per sequence at position L.  The context lengths are the
    spread "Iteration-Level Batching" uses ("Two resources idled by a fixed
    batch").  Cells come from a seeded shuffled free list."""
    batches = []
    ctx = [lengths[i % len(lengths)] for i in range(n_seq)]
    for i in range(n_seq):
        batches += _prompt_batches((i,), 0, ctx[i], 2048, measured=False, out_last=False)
    batches.append(_batch(ctx, [(i,) for i in range(n_seq)], [1] * n_seq, True))
    order = None
    if shuffled:
        rng = np.random.default_rng(np.random.SeedSequence([seed, PURPOSE_CELL_ORDER]))
        order = rng.permutation(kv_size).astype(np.int32)[None, :]
    return Workload("cb_decode", n_layer, 16, 8, 128, kv_size=kv_size, n_stream=1,
                    n_seq_max=n_seq, seed=seed, batches=batches, cell_order=order,
                    note=f"{n_seq} sequences, contexts {sorted(set(ctx))}")


def mixed(n_prompt_seq=8, n_decoders=56, prompt_range=(128, 1024), ctx_range=(256, 4096),
          n_layer=28, n_stream=8, kv_size=32768, n_batch=2048, n_ubatch=512, seed=1004):
    """Mixed prefill + decode over a non-unified cache (stream = seq % n_stream).

    Prompts are sequences 0..n_prompt_seq-1, decoders the next n_decoders ids.
    Setup stores every decoder's context.  Then each measured call carries one
    decode token per decoder plus the next prompt chunks, in sequence order,
    up to n_batch slots ("Iteration-Level Batching", "The loop that replaces
    the batch"); the output flag sits on each sequence's last slot."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, PURPOSE_STRUCTURE]))
    plen = rng.integers(prompt_range[0], prompt_range[1], size=n_prompt_seq, endpoint=True)
    ctx = rng.integers(ctx_range[0], ctx_range[1], size=n_decoders, endpoint=True)
    dec_ids = list(range(n_prompt_seq, n_prompt_seq + n_decoders))
    batches = []
    for d, L in zip(dec_ids, ctx):
        batches += _prompt_batches((d,), 0, int(L), n_batch, measured=False, out_last=False)
    done = [0] * n_prompt_seq
    t = 0
    while any(done[k] < plen[k] for k in range(n_prompt_seq)):
        pos, seqs, out = [], [], []
        for d, L in zip(dec_ids, ctx):
            pos.append(int(L) + t)
            seqs.append((d,))
            out.append(1)
        room = n_batch - len(pos)
        for k in range(n_prompt_seq):
            if room == 0:
                break
            take = min(room, int(plen[k]) - done[k])
            if take <= 0:
                continue
            pos += list(range(done[k], done[k] + take))
            seqs += [(k,)] * take
            out += [0] * (take - 1) + [1]
            done[k] += take
            room -= take
        batches.append(_batch(pos, seqs, out, True))
        t += 1
    n_seq = n_prompt_seq + n_decoders
    return Workload("mixed", n_layer, 16, 8, 128, kv_size=kv_size, n_stream=n_stream,
                    n_seq_max=n_seq, seed=seed, batches=batches, n_batch=n_batch,
                    n_ubatch=n_ubatch,
                    note=f"prompts {plen.tolist()}, {n_decoders} decoders")


def prefix_decode(n_seq=32, prefix=2048, private=256, n_layer=28, kv_size=16384, n_stream=1, seed=1005):
    """Prefix sharing: one prefix of ``prefix`` tokens stored once for all
    n_seq sequences (slots with n_seq ids; "Batch、Ubatch 与解码主循环" Part E),
    then ``private`` tokens per sequence, then one measured decode token per
    sequence.  With several streams (kv_size cells each) the prefix slots'
    ids span the streams, so the prefix is stored once per stream."""
    everyone = tuple(range(n_seq))
    batches = _prompt_batches(everyone, 0, prefix, 2048, measured=False, out_last=False)
    pos, seqs = [], []
    for i in range(n_seq):
        pos += list(range(prefix, prefix + private))
        seqs += [(i,)] * private
    for a, b in _chunks(len(pos), 2048):
        batches.append(_batch(pos[a:b], seqs[a:b], [0] * (b - a), False))
    batches.append(_batch([prefix + private] * n_seq, [(i,) for i in range(n_seq)],
                          [1] * n_seq, True))
    return Workload("prefix_decode", n_layer, 16, 8, 128, kv_size=kv_size, n_stream=n_stream,
                    n_seq_max=n_seq, seed=seed, batches=batches,
                    note=f"{n_seq} sequences share {prefix} cells, {private} private each")


def many_sequences(n_seq=256, group=8, prefix=24, private=(3, 40), n_shared=0, shared_size=8, n_layer=1,
                   kv_size=16384, seed=1007):
    """Many live sequences at once: groups of ``group`` sequences share a
    prefix stored once (cells holding ``group`` ids), every sequence then
    gets a private prompt of random length, and ``n_shared`` further slots
    each hold ``shared_size`` random sequences (so one decode ubatch sees up
    to n_shared more distinct sequence sets, each read by several queries).
    Then two measured steps of one decode token per sequence."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, PURPOSE_STRUCTURE]))
    next_pos = [0] * n_seq
    batches = []
    pos, seqs = [], []
    for g0 in range(0, n_seq, group):
        ids = tuple(range(g0, min(n_seq, g0 + group)))
        pos += list(range(prefix))
        seqs += [ids] * prefix
        for i in ids:
            next_pos[i] = prefix
    lens = rng.integers(private[0], private[1], size=n_seq, endpoint=True)
    for i in range(n_seq):
        pos += list(range(next_pos[i], next_pos[i] + int(lens[i])))
        seqs += [(i,)] * int(lens[i])
        next_pos[i] += int(lens[i])
    for _ in range(n_shared):
        ids = tuple(int(x) for x in rng.choice(n_seq, size=shared_size, replace=False))
        p = max(next_pos[i] for i in ids)
        pos.append(p)
        seqs.append(ids)
        for i in ids:
            next_pos[i] = p + 1
    for a, b in _chunks(len(pos), 2048):
        batches.append(_batch(pos[a:b], seqs[a:b], [0] * (b - a), False))
    for _ in range(2):
        batches.append(_batch([next_pos[i] for i in range(n_seq)], [(i,) for i in range(n_seq)], [1] * n_seq, True))
        next_pos = [p + 1 for p in next_pos]
    return Workload("many_sequences", n_layer, 16, 8, 128, kv_size=kv_size, n_stream=1, n_seq_max=n_seq,
                    seed=seed, batches=batches, n_batch=2048, n_ubatch=512,
                    note=f"{n_seq} sequences in groups of {group} sharing {prefix} cells, {private[0]}..{private[1]} "
                         f"private each, {n_shared} slots of {shared_size} random sequences, two decode steps")


def random_mix(seed, n_batches=6):
    """A randomized small workload for differential tests: random head shape
    (head_dim 64 or 128, group 1, 2 or 4, 2 to 8 KV heads), one to four
    streams, shuffled or ordered free lists, any split strategy, causal or
    not, sometimes a sliding window; batches mix prompt runs of one sequence
    (consecutive positions), decode tokens, slots shared by several
    sequences (which may span streams) and positions drawn at random, with
    random output flags.  Every batch is measured and the cache never fills.
    Half of the seeds spread the sequences over a wide id space (n_seq_max
    drawn in [65, 256], ids placed at random in it), so that sets span
    several 64-bit words; that draw comes from a stream of its own, so the
    rest of a seed's workload does not depend on it."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, PURPOSE_STRUCTURE, 9]))
    irng = np.random.default_rng(np.random.SeedSequence([seed, PURPOSE_STRUCTURE, 10]))
    head_dim = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4]))
    hk = int(rng.choice([2, 4, 8]))
    n_stream = int(rng.choice([1, 1, 2, 4]))
    n_seq = int(rng.integers(2, 9))
    n_batch = int(rng.choice([16, 48, 96]))
    n_ubatch = int(rng.choice([7, 16, 32, 96]))
    causal = bool(rng.random() < 0.8)
    swa = int(rng.choice([0, 0, 0, 5, 40]))
    split = str(rng.choice(["auto", "simple", "equal", "seq"]))
    next_pos = [0] * n_seq
    batches, total = [], 0
    for _ in range(n_batches):
        n = int(rng.integers(1, n_batch + 1))
        pos, seqs = [], []
        while len(pos) < n:
            kind = rng.random()
            s = int(rng.integers(0, n_seq))
            if kind < 0.4:                       # a prompt run of one sequence
                run = int(min(n - len(pos), rng.integers(1, 24)))
                pos += list(range(next_pos[s], next_pos[s] + run))
                seqs += [(s,)] * run
                next_pos[s] += run
            elif kind < 0.75:                    # one decode token
                pos.append(next_pos[s])
                seqs.append((s,))
                next_pos[s] += 1
            elif kind < 0.9:                     # a slot shared by several sequences
                ids = [s] + [int(x) for x in rng.choice(n_seq, size=int(rng.integers(1, n_seq)), replace=False)
                             if int(x) != s]
                p = max(next_pos[i] for i in ids)
                pos.append(p)
                seqs.append(tuple(ids))
                for i in ids:
                    next_pos[i] = p + 1
            else:                                # a position drawn at random
                pos.append(int(rng.integers(0, 64)))
                seqs.append((s,))
        out = (rng.random(n) < 0.4).astype(np.int8)
        batches.append((pos, seqs, out))
        total += n
    n_seq_max = n_seq
    ids = list(range(n_seq))
    if irng.random() < 0.5:                  # a wide id space
        n_seq_max = int(irng.integers(65, 257))
        ids = [int(x) for x in irng.choice(n_seq_max, size=n_seq, replace=False)]
    batches = [_batch(pos, [tuple(ids[i] for i in t) for t in seqs], out, True) for pos, seqs, out in batches]
    kv_size = int(2 * total + 64)            # every slot and its copies fit, in any stream
    wl = Workload(f"random_mix_{seed}", 1, hk * g, hk, head_dim, kv_size=kv_size, n_stream=n_stream,
                  n_seq_max=n_seq_max, seed=seed, batches=batches, n_batch=n_batch, n_ubatch=n_ubatch,
                  causal=causal, split_mode=split, swa=swa,
                  note=f"random mix {seed}: d={head_dim} g={g} kv heads {hk}, {n_stream} streams, {split}, "
                       f"causal={causal}, window {swa}, ids {ids} of {n_seq_max}")
    if rng.random() < 0.5:
        orng = np.random.default_rng(np.random.SeedSequence([seed, PURPOSE_CELL_ORDER]))
        wl.cell_order = np.stack([orng.permutation(kv_size) for _ in range(n_stream)]).astype(np.int32)
    return wl


WORKLOADS = {"tiny": tiny, "qwen_prefill": qwen_prefill, "cb_decode": cb_decode,
             "mixed": mixed, "prefix_decode": prefix_decode}


def by_name(name, **kw):
    return WORKLOADS[name](**kw)
