"""Batch intake and the batch -> ubatch split, restated from the pages.

Test infrastructure only (see ``oracle/__init__.py``).

A batch is a list of token slots; slot i carries a position, a set of
sequence ids and an output flag ("llama.cpp and the ubatch", "Three things called batch"; "Batch、Ubatch 与解码主循环", Part A,
the llama_batch statement).  A ubatch is what one forward pass processes
("llama.cpp and the ubatch", "Three things called batch"; "Batch、Ubatch 与解码主循环", Part B, the llama_ubatch statement).
"""

from __future__ import annotations

import numpy as np

DEFAULT_N_BATCH = 2048   # "llama.cpp and the ubatch", "Back to the VRAM question"; "Batch、Ubatch 与解码主循环" two-level batch parameters
DEFAULT_N_UBATCH = 512


class SplitError(ValueError):
    """An invalid batch (the library reports these as negative status codes)."""


def clamp_params(n_ctx: int, n_batch: int, n_ubatch: int, causal: bool = True):
    """Context-creation clamps ("llama.cpp and the ubatch", "Three things called batch").

    Under causal attention n_batch is limited to the cache capacity n_ctx;
    n_ubatch falls back to n_batch when zero and is then limited to n_batch.
    A zero n_batch takes the common default of 2048 ("llama.cpp and the ubatch", "Back to the VRAM
    question" -- reading: zero means "use the default").
    """
    if n_batch < 0 or n_ubatch < 0 or n_ctx <= 0:
        raise SplitError("negative size")
    if n_batch == 0:
        n_batch = DEFAULT_N_BATCH
    nb = min(n_ctx, n_batch) if causal else n_batch
    nub = min(nb, n_batch if n_ubatch == 0 else n_ubatch)
    return nb, nub


def fill_batch(n_tokens, pos, seq_id, output, next_pos, n_seq_max, n_stream):
    """Validate a batch and fill the fields the caller left out.

    "Batch、Ubatch 与解码主循环", Part A says pos may be NULL (auto-increment) and that the sampler only
    needs the last token's output; "Batch、Ubatch 与解码主循环", Part F says llama_decode first validates
    and auto-fills pos, seq_id and logits.  Readings (the pages do not say how):

    * ``seq_id is None``  -> every slot belongs to sequence {0};
    * ``pos is None``     -> per first sequence id, continue from
      ``next_pos[s]`` (1 + the largest committed position of s, 0 if none),
      incrementing in slot order;
    * ``output is None``  -> only the last slot is flagged.

    A slot's sequence ids form a set (duplicates collapse).  Rejected: an id
    outside [0, n_seq_max), an empty id list, a negative position.  (With
    several streams a slot whose ids live in different streams is stored once
    per stream: see ``OracleEngine.split``.)

    Returns (pos list, list of sorted seq-id tuples, output list).
    """
    if n_tokens < 0:
        raise SplitError("n_tokens < 0")
    if seq_id is None:
        sids = [(0,) for _ in range(n_tokens)]
    else:
        sids = []
        for i in range(n_tokens):
            ids = sorted(set(int(s) for s in seq_id[i]))
            if len(ids) == 0:
                raise SplitError(f"slot {i}: empty seq id list")
            for s in ids:
                if s < 0 or s >= n_seq_max:
                    raise SplitError(f"slot {i}: seq id {s} out of range")
            sids.append(tuple(ids))
    if pos is None:
        counter = dict(next_pos)
        p = []
        for i in range(n_tokens):
            s0 = seq_id[i][0] if seq_id is not None else 0
            s0 = int(s0)
            cur = counter.get(s0, 0)
            p.append(cur)
            counter[s0] = cur + 1
    else:
        p = [int(x) for x in pos[:n_tokens]]
    for i, x in enumerate(p):
        if x < 0:
            raise SplitError(f"slot {i}: negative position")
    if output is None:
        out = [0] * n_tokens
        if n_tokens:
            out[-1] = 1
    else:
        out = [1 if int(o) else 0 for o in output[:n_tokens]]
    # the query masks against the FIRST listed id ("llama.cpp and the ubatch", "The mask is doing the
    # work"); keep it first, then the rest of the set in ascending order.
    if seq_id is not None:
        sids = [tuple([int(seq_id[i][0])] + [s for s in sids[i] if s != int(seq_id[i][0])])
                for i in range(n_tokens)]
    return p, sids, out


def split_simple(unused: list, n_ubatch: int):
    """One split_simple step: the next <= n_ubatch unused slots in submission
    order, ignoring sequence ids ("llama.cpp and the ubatch", "Part 1: putting different conversations
    in the same ubatch"; "Batch、Ubatch 与解码主循环", Part C item 1: 1000 tokens -> 512 + 488)."""
    take = [i for i, u in enumerate(unused) if u][:n_ubatch]
    for i in take:
        unused[i] = False
    return take


def split_equal(unused: list, seq_sets: list, n_ubatch: int):
    """One split_equal(n_ubatch, sequential=true) step.

    "Batch、Ubatch 与解码主循环", Part C item 2: pick non-overlapping sequence sets, then take the same
    number of tokens from each set until the ubatch nears n_ubatch or a set
    runs out; "llama.cpp and the ubatch", "Part 1: putting different
    conversations in the same ubatch", describes it as cutting chunks of one
    length per sequence with the sequence ids kept in order.
    Reading of the steps the pages leave open:

    1. scan unused slots in submission order; a slot whose set equals an
       adopted set belongs to it; a set disjoint from every adopted set is
       adopted; a partially overlapping set waits for a later ubatch; stop
       once n_ubatch sets are adopted;
    2. n_seq_tokens = min(fewest unused slots of any adopted set,
       floor(n_ubatch / number of sets));
    3. take that many slots from each set, in submission order;
    4. lay the ubatch out set after set, sets ordered by their smallest id.

    Returns (slot list, n_seq_tokens, n_seqs); an empty list when done.
    """
    adopted = []
    for i, u in enumerate(unused):
        if not u:
            continue
        s = frozenset(seq_sets[i])
        if s in adopted:
            continue
        if any(s & a for a in adopted):
            continue
        adopted.append(s)
        if len(adopted) == n_ubatch:
            break
    if not adopted:
        return [], 0, 0
    members = {a: [i for i, u in enumerate(unused) if u and frozenset(seq_sets[i]) == a]
               for a in adopted}
    n_seq_tokens = min(min(len(v) for v in members.values()), n_ubatch // len(adopted))
    order = sorted(adopted, key=min)
    take = []
    for a in order:
        for i in members[a][:n_seq_tokens]:
            unused[i] = False
            take.append(i)
    return take, n_seq_tokens, len(adopted)


def split_seq(unused: list, seq_sets: list, n_ubatch: int):
    """One split_seq(n_ubatch) step ("Batch、Ubatch 与解码主循环", Part C item 3: every ubatch holds the
    tokens of one sequence set, sequences are never mixed; meant for
    independent decoding).  Reading of what the page leaves open: the set is
    that of the first unused slot in submission order, and the ubatch takes
    the unused slots with exactly that set, in submission order, at most
    n_ubatch of them.  Returns (slot list, n_seq_tokens, n_seqs)."""
    first = next((i for i, u in enumerate(unused) if u), None)
    if first is None:
        return [], 0, 0
    s = frozenset(seq_sets[first])
    take = [i for i, u in enumerate(unused) if u and frozenset(seq_sets[i]) == s][:n_ubatch]
    for i in take:
        unused[i] = False
    return take, len(take), 1


SPLIT_MODES = ("auto", "simple", "equal", "seq")


def split_batch(seq_sets: list, n_ubatch: int, n_stream: int, mode: str = "auto"):
    """The init_batch split loop ("Batch、Ubatch 与解码主循环", Part C, strategy choice): one stream ->
    split_simple, several streams -> split_equal(n_ubatch, true) ("auto");
    a caller may instead name one of the three strategies.  Repeat until a
    split returns no slot.  Returns a list of (slots, n_seq_tokens, n_seqs)
    tuples in ubatch order."""
    if mode not in SPLIT_MODES:
        raise SplitError(f"unknown split mode {mode!r}")
    if mode == "auto":
        mode = "simple" if n_stream == 1 else "equal"
    unused = [True] * len(seq_sets)
    out = []
    while True:
        if mode == "simple":
            take = split_simple(unused, n_ubatch)
            nst, ns = len(take), 1
        elif mode == "equal":
            take, nst, ns = split_equal(unused, seq_sets, n_ubatch)
        else:
            take, nst, ns = split_seq(unused, seq_sets, n_ubatch)
        if not take:
            break
        out.append((take, nst, ns))
    return out


def output_ids(output: list, n_batch: int) -> np.ndarray:
    """Batch row -> output row map, n_batch entries ("llama.cpp and the ubatch", "Where the memory
    actually sits": output_reserve sizes output_ids by n_batch).  Reading:
    flagged slots get their rank among flagged slots in batch order, the rest
    (and the unused tail) get -1."""
    ids = np.full(n_batch, -1, dtype=np.int32)
    r = 0
    for b, o in enumerate(output):
        if o:
            ids[b] = r
            r += 1
    return ids
